"""The side-stream kernels of the two-stream pipeline must fit on a compute unit beside a
Newton–Schulz product workgroup, or they wait for whole product workgroups to retire
instead of running beside them.  Checked at compile time from the compiler's resource
report for gfx950: per SIMD lane 512 registers (VGPRs and AGPRs, allocated in blocks of
8), and 160 KiB of LDS per CU; a product workgroup holds 2 waves per SIMD, a side
workgroup of 256 threads 1.
"""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "muon_newton_schulz_momentum_amd", "csrc")
INCLUDE = os.path.join(HERE, "..", "include")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

REGS_PER_LANE = 512
LDS_PER_CU = 160 * 1024


def _resources(src):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-I", INCLUDE, "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-c", os.path.join(CSRC, src), "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"]
    out = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stderr[-2000:]
    res, name = {}, None
    for line in out.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            res[name] = {}
            continue
        m = re.search(r"remark:\s+(VGPRs|AGPRs|LDS Size \[bytes/block\]|ScratchSize \[bytes/lane\]): (\d+)", line)
        if m and name:
            res[name][m.group(1).split(" ")[0]] = int(m.group(2))
    return res


def _alloc(r):
    return -(-(r["VGPRs"] + r.get("AGPRs", 0)) // 8) * 8


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_side_kernels_fit_beside_a_product_workgroup():
    ew = _resources("elementwise.hip")
    ns = _resources("ns_gemm.hip")
    gemm = [r for k, r in ns.items() if "ns_vs_kernel" in k]
    side = {k: r for k, r in ew.items() if "_side_kernel" in k}
    # 3 modes x (one tile, persistent), plus SYRK and AXPY with the fused normalisation
    assert len(gemm) == 10 and len(side) == 4, (sorted(ns), sorted(ew))
    g_regs = max(_alloc(r) for r in gemm)
    g_lds = max(r["LDS"] for r in gemm)
    for k, r in side.items():
        assert r.get("ScratchSize", 0) == 0, k
        assert 2 * g_regs + _alloc(r) <= REGS_PER_LANE, (k, g_regs, _alloc(r))
        assert g_lds + r["LDS"] <= LDS_PER_CU, (k, g_lds, r["LDS"])
    print(f"product workgroup: {g_regs} registers x 2 waves/SIMD, {g_lds} B LDS; side kernels: "
          + ", ".join(f"{re.sub(r'^_ZN4muon12_GLOBAL__N_1[0-9]+', '', k)[:24]} {_alloc(r)} regs {r['LDS']} B"
                      for k, r in side.items()))
