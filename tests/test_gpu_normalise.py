"""The normalisation X = bf16(X0 / (||X0||_F + eps)) against the float64 oracle, bitwise.

Each matrix is a seeded bf16 Gaussian whose first two entries are raised to the size of
the rest's norm and picked, on the CPU from the oracle, so that the normaliser puts some
of the matrix's values next to a bf16 rounding midpoint: there a product rounded to float32
first and then to bf16 differs from the oracle's one rounding (checked below, so every case
tells the two apart).  One Newton-Schulz iteration with (a, b, c) = (1, 0, 0) returns X
itself (1 X + 0 X is exact), so the output is the normalised matrix.  Every path that
normalises is covered: fused into the first iteration's loads (256-row tiles), the separate
pass, the second stream's pass in the two-stream step, the grouped small-chunk launches and
the fused small-matrix kernel.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from oracle import muon_oracle as orc  # noqa: E402

EPS = 1e-7
SHAPES = [(1100, 1300), (1300, 1100), (512, 4096), (32, 4096), (64, 128), (300, 700), (1, 4096)]


def _float32_product(X0, inv):
    """bf16(f32(X0 * f32(inv))): the normalisation with a float32 product rounded twice."""
    return orc.bf16_round((X0.astype(np.float32) * np.float32(inv)).astype(np.float64))


def _midpoint_matrix(shape, seed, tries=20000):
    """A bf16-valued matrix whose normalisation differs between one and two roundings."""
    rng = np.random.RandomState(seed)
    X0 = orc.bf16_round(rng.standard_normal(shape) * 1e-3)
    X0[0, :2] = 0.0
    rest = np.sum(X0 * X0)
    values = np.unique(np.abs(X0))
    eps = orc.f32(EPS)[()]
    spikes = orc.bf16_round(np.sqrt(rest) * (0.25 + 0.75 * rng.random_sample((tries, 2))))
    for v1, v2 in spikes:
        # screen the distinct magnitudes with the norm summed as rest + spikes
        inv = 1.0 / (np.sqrt(rest + v1 * v1 + v2 * v2) + eps)
        u = np.append(values, [v1, v2])
        if not np.any(orc.bf16_round(u * inv) != _float32_product(u, inv)):
            continue
        X = X0.copy()
        X[0, 0], X[0, 1] = v1, v2
        t = orc.canonical_orientation(*shape)
        Xc = X.T if t else X
        ref = orc.frobenius_normalise(Xc, EPS)
        inv = 1.0 / (np.sqrt(np.sum(Xc * Xc)) + eps)
        n_diff = int(np.sum(ref != _float32_product(Xc, inv)))
        if n_diff:
            return X, ref, n_diff
    raise AssertionError(f"no midpoint case found for {shape}")


@pytest.fixture(scope="module")
def cases():
    return [_midpoint_matrix(s, 900 + s[0] + s[1]) for s in SHAPES]


def _params(cases):
    from muon_newton_schulz_momentum_amd.harness import ParamTensors
    out = []
    for X, _, _ in cases:
        G = torch.from_numpy(X.astype(np.float32)).cuda()
        out.append(ParamTensors(torch.zeros_like(G), torch.zeros_like(G), G))
    return out


@pytest.mark.parametrize("flags,pipeline", [("default", False), ("default", True), ("unfused", False),
                                            ("unfused", True), ("ungrouped", False)])
def test_normalisation_is_the_oracles_one_rounding(cases, flags, pipeline):
    from muon_newton_schulz_momentum_amd import binding as L, harness
    f = {"default": 0, "unfused": L.MUON_PLAN_UNFUSED_NORMALIZE, "ungrouped": L.MUON_PLAN_UNGROUPED}[flags]
    params = _params(cases)
    plan = harness.Plan(params, flags=f | (L.MUON_PLAN_PIPELINE if pipeline else 0))
    assert plan.n_buckets >= 5
    # beta = 0: M takes G, X0 = bf16(G) = the matrix itself
    plan.step_ex(0.0, 0.0, 0.0, coeffs=[(1.0, 0.0, 0.0)], eps=EPS, pipeline=pipeline)
    torch.cuda.synchronize()
    for i, (X, ref, n_diff) in enumerate(cases):
        O = plan.output(i).float().cpu().numpy().astype(np.float64)
        bad = int(np.sum(O != ref))
        assert bad == 0, f"{SHAPES[i]} ({flags}, pipeline {pipeline}): {bad} of {ref.size} normalised values " \
                         f"differ from the oracle ({n_diff} differ between one and two roundings)"
    plan.close()
