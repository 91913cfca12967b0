"""The host planner (csrc/plan.cpp, no HIP calls) under AddressSanitizer and
UndefinedBehaviorSanitizer: a small driver builds 800 random two-stream plans, with and
without workspace caps (some too small, exercising the error paths), and checks that each
is well formed.  Runs on the CPU; skipped where g++ or the sanitizer runtimes are missing."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_planner_is_clean_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "plan_fuzz"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "muon_newton_schulz_momentum_amd", "csrc"),
           os.path.join(ROOT, "tests", "native", "plan_fuzz.cpp"),
           os.path.join(ROOT, "muon_newton_schulz_momentum_amd", "csrc", "plan.cpp"), "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "asan" in build.stderr.lower():
        pytest.skip("sanitizer runtime not available: " + build.stderr[-200:])
    assert build.returncode == 0, build.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "plans ok" in run.stdout
