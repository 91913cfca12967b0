"""The fused small-matrix kernel (whole Newton–Schulz of a matrix in one workgroup).

* Bitwise equal to the tiled kernels: the same plan built with MUON_PLAN_TILED_SMALL
  takes the tiled path, and W, M and O must agree bit for bit (same K order, same
  epilogue expressions, same normaliser summation).
* Against the float64 oracle: momentum and apply bitwise, O within 1e-2 relative
  Frobenius, for ragged shapes, both orientations, m = 1 and n at the 1024 limit.
* Grouped: several small chunks of different shapes are stepped by one launch of the
  fused kernel next to tiled chunks, with the same results as chunk-by-chunk stepping.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from oracle import muon_oracle as orc  # noqa: E402

A, B, C, K, EPS = 3.4445, -4.7750, 2.0315, 5, 1e-7
BETA, LR, WD = 0.95, 0.02, 0.1
SMALL = [(64, 128), (17, 300), (300, 17), (64, 1024), (1, 64), (5, 1000), (64, 64), (40, 1000)]


def _params(shapes, seed):
    from muon_newton_schulz_momentum_amd.harness import ParamTensors
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    out = []
    for s in shapes:
        W = torch.randn(s, generator=gen, device="cuda") * 0.02
        M = torch.randn(s, generator=gen, device="cuda") * 1e-3
        G = torch.randn(s, generator=gen, device="cuda") * 1e-3
        out.append(ParamTensors(W, M, G))
    return out


def _clone(params):
    from muon_newton_schulz_momentum_amd.harness import ParamTensors
    return [ParamTensors(p.weight.clone(), p.momentum.clone(), p.grad.clone()) for p in params]


def _bits(t):
    return t.detach().contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu()


def test_fused_equals_tiled_bitwise_and_oracle():
    from muon_newton_schulz_momentum_amd import binding as L, harness
    fused_p = _params(SMALL, seed=401)
    tiled_p = _clone(fused_p)
    snap = [(p.weight.cpu().numpy(), p.momentum.cpu().numpy(), p.grad.cpu().numpy()) for p in fused_p]
    fused = harness.Plan(fused_p)
    tiled = harness.Plan(tiled_p, flags=L.MUON_PLAN_TILED_SMALL)
    assert all(fused.chunk_info(c).fused_small for c in range(fused.n_chunks))
    assert not any(tiled.chunk_info(c).fused_small for c in range(tiled.n_chunks))
    fused.step(BETA, LR, WD, A, B, C, K, EPS)
    tiled.step(BETA, LR, WD, A, B, C, K, EPS)
    torch.cuda.synchronize()
    for i, (pf, pt) in enumerate(zip(fused_p, tiled_p)):
        assert torch.equal(_bits(fused.output(i)), _bits(tiled.output(i))), f"O of {SMALL[i]}"
        assert torch.equal(_bits(pf.weight), _bits(pt.weight)), f"W of {SMALL[i]}"
        assert torch.equal(_bits(pf.momentum), _bits(pt.momentum)), f"M of {SMALL[i]}"
    worst = 0.0
    for i, (W0, M0, G0) in enumerate(snap):
        M_ref, X0 = orc.momentum_update(M0, G0, BETA)
        assert np.array_equal(fused_p[i].momentum.cpu().numpy(), M_ref)
        O_ref = orc.newton_schulz(X0, A, B, C, K, EPS, emulate_bf16=True)
        O = fused.output_oriented(i).float().cpu().numpy().astype(np.float64)
        r = np.linalg.norm(O - O_ref) / np.linalg.norm(O_ref)
        worst = max(worst, r)
        assert r <= 1e-2, f"{SMALL[i]}: {r:.3e}"
        assert np.array_equal(fused_p[i].weight.cpu().numpy(), orc.apply_update(W0, O, LR, WD))
    print(f"fused small kernel: worst NS rel err {worst:.2e}")
    fused.close()
    tiled.close()


@pytest.mark.parametrize("steps", [1, 2, 3, 6])
def test_fused_step_counts(steps):
    from muon_newton_schulz_momentum_amd import binding as L, harness
    fused_p = _params([(64, 128), (20, 256)], seed=410 + steps)
    tiled_p = _clone(fused_p)
    fused = harness.Plan(fused_p)
    tiled = harness.Plan(tiled_p, flags=L.MUON_PLAN_TILED_SMALL)
    for pl in (fused, tiled):
        pl.momentum_update(BETA)
        pl.ns_batched(A, B, C, steps, EPS)
    torch.cuda.synchronize()
    for i in range(2):
        assert torch.equal(_bits(fused.output(i)), _bits(tiled.output(i)))
    fused.close()
    tiled.close()


def test_grouped_launch_next_to_tiled_chunks():
    from muon_newton_schulz_momentum_amd import binding as L, harness
    shapes = SMALL + [(256, 384), (384, 256), (130, 200)]
    grouped_p = _params(shapes, seed=420)
    single_p = _clone(grouped_p)
    grouped = harness.Plan(grouped_p)
    single = harness.Plan(single_p)
    n_fused = sum(grouped.chunk_info(c).fused_small for c in range(grouped.n_chunks))
    assert n_fused >= 5 and n_fused < grouped.n_chunks
    grouped.timing_enable(256)
    grouped.step(BETA, LR, WD, A, B, C, K, EPS)           # every chunk: small ones grouped
    for ch in range(single.n_chunks):                      # chunk by chunk
        single.step(BETA, LR, WD, A, B, C, K, EPS, chunk=ch)
    torch.cuda.synchronize()
    ms, launches, work = grouped.timing_read(L.MUON_KERNEL_NS_SMALL)
    assert launches == 1 and work > 0
    grouped.timing_enable(0)
    for i in range(len(shapes)):
        assert torch.equal(_bits(grouped.output(i)), _bits(single.output(i)))
        assert torch.equal(_bits(grouped_p[i].weight), _bits(single_p[i].weight))
    grouped.close()
    single.close()


def test_fused_zero_matrix_and_nan_isolation():
    from muon_newton_schulz_momentum_amd import harness
    ps = _params([(64, 128)] * 3, seed=430)
    for p in ps:
        p.momentum.zero_()
    ps[0].grad.zero_()                  # all-zero momentum: O = 0, W only decays
    ps[1].grad[3, 5] = float("nan")     # NaN stays in its own matrix
    W0 = [p.weight.clone() for p in ps]
    plan = harness.Plan(ps)
    plan.step(BETA, LR, WD, A, B, C, K, EPS)
    torch.cuda.synchronize()
    assert torch.count_nonzero(plan.output(0).float()) == 0
    W_ref = orc.apply_update(W0[0].cpu().numpy(), np.zeros((64, 128)), LR, WD)
    assert np.array_equal(ps[0].weight.cpu().numpy(), W_ref)
    assert torch.isnan(plan.output(1).float()).any()
    assert torch.isfinite(plan.output(2).float()).all()
    assert torch.isfinite(ps[2].weight).all()
    plan.close()
