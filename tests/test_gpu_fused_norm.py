"""The normalisation fused into the first iteration's operand loads (256-row tiles).

A chunk of 256-row output tiles (m >= 1024) run for an odd number of iterations never
writes the normalised X: its first SYRK and GEMM+axpy read X0 and scale each value by the
matrix's normaliser on its way into LDS, with the separate pass's arithmetic.

* Bitwise equal to the separate pass (the same plan built with
  MUON_PLAN_UNFUSED_NORMALIZE): W, M and O for ragged 256-tile shapes in both
  orientations, a shape without padding, a 128-tile bucket next to them, and odd and even
  iteration counts; one matrix per bucket also against the float64 oracle.
* Stale padding: chunks of different shapes sharing one workspace region leave their
  data in each other's padding; the finalize kernel zeroes X0's padding before the fused
  loads read it (the separate pass rewrites it), checked bitwise over two steps.
* NaN recovery: a NaN gradient poisons its matrix's iterates (padding included); once
  the momentum and gradient are finite again, the next step equals the separate pass's.
* X0 bookkeeping: a Newton-Schulz call consumes X0; a second call without a momentum
  update in between is refused, as is one on a chunk whose region another chunk's
  momentum update has since overwritten.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from oracle import muon_oracle as orc  # noqa: E402

A, B, C, K, EPS = 3.4445, -4.7750, 2.0315, 5, 1e-7
BETA, LR, WD = 0.95, 0.02, 0.1
SHAPES = [(1100, 1300), (1300, 1100), (1024, 1536), (1100, 1300), (300, 700)]


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


def _same(pa, pb, plan_a, plan_b, what):
    for i, (a, b) in enumerate(zip(pa, pb)):
        assert torch.equal(_bits(plan_a.output(i)), _bits(plan_b.output(i))), f"{what}: O of {i}"
        assert torch.equal(_bits(a.weight), _bits(b.weight)), f"{what}: W of {i}"
        assert torch.equal(_bits(a.momentum), _bits(b.momentum)), f"{what}: M of {i}"


@pytest.mark.parametrize("steps", [5, 3, 4])
def test_fused_normalisation_bitwise_equal_to_separate_pass(steps):
    from muon_newton_schulz_momentum_amd import binding as L, harness
    fused_p = _params(SHAPES, seed=701 + steps)
    sep_p = _clone(fused_p)
    snap = [(p.weight.cpu().numpy(), p.momentum.cpu().numpy(), p.grad.cpu().numpy()) for p in fused_p]
    fused = harness.Plan(fused_p)
    sep = harness.Plan(sep_p, flags=L.MUON_PLAN_UNFUSED_NORMALIZE)
    fused.step(BETA, LR, WD, A, B, C, steps, EPS)
    sep.step(BETA, LR, WD, A, B, C, steps, EPS)
    torch.cuda.synchronize()
    _same(fused_p, sep_p, fused, sep, f"{steps} iterations")
    for i in (0, 1, 2, 4):
        W0, M0, G0 = snap[i]
        M_ref, X0 = orc.momentum_update(M0, G0, BETA)
        O_ref = orc.newton_schulz(X0, A, B, C, steps, EPS, emulate_bf16=True)
        O = fused.output_oriented(i).float().cpu().numpy().astype(np.float64)
        r = np.linalg.norm(O - O_ref) / np.linalg.norm(O_ref)
        assert r <= 1e-2, f"{SHAPES[i]}, {steps} iterations: {r:.3e}"
        assert np.array_equal(fused_p[i].weight.cpu().numpy(), orc.apply_update(W0, O, LR, WD))
    fused.close()
    sep.close()


def test_fused_normalisation_zeroes_stale_padding():
    """Two buckets share one region under a cap; over two steps each chunk's X0 padding
    holds the other bucket's data before the finalize kernel zeroes it."""
    from muon_newton_schulz_momentum_amd import binding as L, harness
    shapes = [(1100, 1300), (1300, 1100), (1200, 2000), (2000, 1200)]
    fused_p = _params(shapes, seed=720)
    sep_p = _clone(fused_p)
    cap = 40 << 20
    fused = harness.Plan(fused_p, max_workspace_bytes=cap)
    sep = harness.Plan(sep_p, max_workspace_bytes=cap, flags=L.MUON_PLAN_UNFUSED_NORMALIZE)
    assert fused.n_chunks == 2 and fused.chunk_info(0).shared_region
    assert fused.chunk_info(0).region_offset == fused.chunk_info(1).region_offset
    snap = None
    for step in range(2):
        if step == 1:
            snap = [(p.weight.cpu().numpy(), p.momentum.cpu().numpy(), p.grad.cpu().numpy()) for p in fused_p]
        for ch in range(fused.n_chunks):
            fused.step(BETA, LR, WD, A, B, C, K, EPS, chunk=ch)
            sep.step(BETA, LR, WD, A, B, C, K, EPS, chunk=ch)
            torch.cuda.synchronize()
            for i in range(len(shapes)):
                if fused.param_info(i).chunk == ch:
                    assert torch.equal(_bits(fused.output(i)), _bits(sep.output(i))), f"step {step}: O of {i}"
    for a, b in zip(fused_p, sep_p):
        assert torch.equal(_bits(a.weight), _bits(b.weight))
    # the last chunk's outputs are still in the region: one of them against the oracle
    i = max(range(len(shapes)), key=lambda j: fused.param_info(j).chunk)
    W0, M0, G0 = snap[i]
    _, X0 = orc.momentum_update(M0, G0, BETA)
    O_ref = orc.newton_schulz(X0, A, B, C, K, EPS, emulate_bf16=True)
    O = fused.output_oriented(i).float().cpu().numpy().astype(np.float64)
    assert np.linalg.norm(O - O_ref) / np.linalg.norm(O_ref) <= 1e-2
    fused.close()
    sep.close()


def test_fused_normalisation_recovers_after_nan():
    from muon_newton_schulz_momentum_amd import binding as L, harness
    shapes = [(1100, 1300), (1100, 1300)]
    fused_p = _params(shapes, seed=730)
    sep_p = _clone(fused_p)
    good = _clone(fused_p)
    for ps in (fused_p, sep_p):
        ps[0].grad[3, 5] = float("nan")
    fused = harness.Plan(fused_p)
    sep = harness.Plan(sep_p, flags=L.MUON_PLAN_UNFUSED_NORMALIZE)
    fused.step(BETA, LR, WD, A, B, C, K, EPS)
    sep.step(BETA, LR, WD, A, B, C, K, EPS)
    torch.cuda.synchronize()
    assert torch.isnan(fused.output(0).float()).all() and torch.isfinite(fused.output(1).float()).all()
    for ps in (fused_p, sep_p):
        ps[0].momentum.copy_(good[0].momentum)
        ps[0].grad.copy_(good[0].grad)
        ps[0].weight.copy_(good[0].weight)
    fused.step(BETA, LR, WD, A, B, C, K, EPS)
    sep.step(BETA, LR, WD, A, B, C, K, EPS)
    torch.cuda.synchronize()
    assert torch.isfinite(fused.output(0).float()).all()
    _same(fused_p, sep_p, fused, sep, "after NaN")
    fused.close()
    sep.close()


def test_newton_schulz_needs_a_fresh_momentum_cast():
    from muon_newton_schulz_momentum_amd import binding as L, harness
    ps = _params([(1100, 1300), (64, 128)], seed=740)
    pl = harness.Plan(ps)
    st = pl._plan
    # nothing cast yet
    assert L.muon_ns_batched(st, -1, A, B, C, K, EPS, None) == L.MUON_ERR_INVALID_ARG
    assert b"muon_momentum_update" in L.muon_last_error()
    pl.momentum_update(BETA)
    pl.ns_batched(A, B, C, K, EPS)
    torch.cuda.synchronize()
    first = [pl.output(i).clone() for i in range(2)]
    # X0 consumed: a second call is refused (it would start from an overwritten buffer)
    assert L.muon_ns_batched(st, 0, A, B, C, K, EPS, None) == L.MUON_ERR_INVALID_ARG
    # per chunk: a fresh cast of one chunk does not make the other's usable
    pl.momentum_update(0.0, chunk=0)
    assert L.muon_ns_batched(st, 1, A, B, C, K, EPS, None) == L.MUON_ERR_INVALID_ARG
    pl.ns_batched(A, B, C, K, EPS, chunk=0)
    # a whole step makes and consumes its own X0
    pl.step(BETA, LR, WD, A, B, C, K, EPS)
    assert L.muon_ns_batched(st, -1, A, B, C, K, EPS, None) == L.MUON_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert all(torch.isfinite(f.float()).all() for f in first)
    pl.close()
    # chunks sharing a region: a momentum update of one overwrites the other's X0
    shared_p = _params([(1100, 1300), (1200, 2000)], seed=741)
    sh = harness.Plan(shared_p, max_workspace_bytes=24 << 20)
    assert sh.n_chunks == 2 and sh.chunk_info(0).region_offset == sh.chunk_info(1).region_offset
    sh.momentum_update(BETA, chunk=0)
    sh.momentum_update(BETA, chunk=1)
    assert L.muon_ns_batched(sh._plan, 0, A, B, C, K, EPS, None) == L.MUON_ERR_INVALID_ARG
    sh.ns_batched(A, B, C, K, EPS, chunk=1)
    torch.cuda.synchronize()
    sh.close()
