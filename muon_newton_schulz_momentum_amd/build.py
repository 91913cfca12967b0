"""Build libmuon.so in-tree with hipcc for gfx950.

    python -m muon_newton_schulz_momentum_amd.build [--clean] [-v]

Every HIP translation unit is compiled for gfx950 only, with packed-fp32 instructions
disabled (the hipcc host pass warns that it does not know that feature; harmless).  The
planner (plan.cpp) has no HIP code and is compiled by the same driver as host C++.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmuon.so")

HIP_SOURCES = ["api.hip", "elementwise.hip", "ns_gemm.hip", "ns_small.hip"]
CXX_SOURCES = ["plan.cpp"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmuon)")


def _common_flags():
    return ["-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]


def _compile(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "is not a recognized feature for this target" not in l)
    return r.returncode, " ".join(cmd), msgs


def build(verbose: bool = False, clean: bool = False) -> str:
    """Compile every source and link libmuon.so; returns the library path."""
    hipcc = _hipcc()
    if clean and os.path.isdir(BUILD):
        shutil.rmtree(BUILD)
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append([hipcc, f"--offload-arch={ARCH}", *_common_flags(),
                     "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                     "-c", os.path.join(CSRC, src), "-o", obj])
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append([hipcc, *_common_flags(), "-x", "c++", "-c", os.path.join(CSRC, src), "-o", obj])
    workers = min(len(jobs), int(os.environ.get("MAX_JOBS", "8")) or 1)
    with cf.ThreadPoolExecutor(workers) as ex:
        for rc, cmd, msgs in ex.map(_compile, jobs):
            if verbose or rc:
                print(cmd)
                if msgs:
                    print(msgs)
            if rc:
                raise RuntimeError(f"compile failed: {cmd}")
    tmp = LIB + ".tmp"
    link = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    rc, cmd, msgs = _compile(link)
    if verbose or rc:
        print(cmd)
        if msgs:
            print(msgs)
    if rc:
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--clean", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(verbose=args.verbose, clean=args.clean))


if __name__ == "__main__":
    sys.exit(main())
