"""The step's variants that the pages leave open (all optional; defaults unchanged):
update-scale rules, per-iteration coefficient schedules, the Nesterov look-ahead, and
device-resident beta/lr/wd read by a captured graph at every replay.  Each is checked
against the float64 oracle: momentum and apply bitwise, O within 1e-2 relative Frobenius.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from oracle import muon_oracle as orc  # noqa: E402

A, B, C, K, EPS = 3.4445, -4.7750, 2.0315, 5, 1e-7
BETA, LR, WD = 0.95, 0.02, 0.1
SCHEDULE = [(4.0848, -6.8946, 2.9270), (3.9505, -6.3029, 2.6377), (3.7418, -5.5913, 2.3037),
            (2.8769, -3.1427, 1.2046), (2.8366, -3.0525, 1.2012)]
SHAPES = [(64, 128), (128, 64), (300, 200), (256, 768), (768, 256)]


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


def _snap(params):
    return [(p.weight.cpu().numpy(), p.momentum.cpu().numpy(), p.grad.cpu().numpy()) for p in params]


def _bits(t):
    return t.detach().contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu()


def _o(plan, i):
    return plan.output_oriented(i).float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("mode,rule", [(1, "aspect"), (2, "rms_match")])
def test_scale_rules(mode, rule):
    from muon_newton_schulz_momentum_amd import harness
    ps = _params(SHAPES, seed=500 + mode)
    snap = _snap(ps)
    plan = harness.Plan(ps, scale_mode=mode)
    plan.step(BETA, LR, WD, A, B, C, K, EPS)
    torch.cuda.synchronize()
    for i, (W0, M0, G0) in enumerate(snap):
        s = orc.update_scale(rule, *W0.shape)
        assert plan.param_info(i).scale == s
        W_ref = orc.apply_update(W0, _o(plan, i), LR, WD, s)
        assert np.array_equal(ps[i].weight.cpu().numpy(), W_ref), (rule, W0.shape)
    plan.close()


def test_coefficient_schedule_against_oracle_and_between_paths():
    from muon_newton_schulz_momentum_amd import binding as L, harness
    ps = _params(SHAPES, seed=510)
    orig = _clone(ps)
    tiled_ps = _clone(ps)
    snap = _snap(ps)
    plan = harness.Plan(ps)
    tiled = harness.Plan(tiled_ps, flags=L.MUON_PLAN_TILED_SMALL)
    for pl in (plan, tiled):
        pl.momentum_update(BETA)
        pl.ns_schedule(SCHEDULE, EPS)
    torch.cuda.synchronize()
    worst = 0.0
    for i, (W0, M0, G0) in enumerate(snap):
        _, X0 = orc.momentum_update(M0, G0, BETA)
        O_ref = orc.newton_schulz_schedule(X0, SCHEDULE, EPS, emulate_bf16=True)
        r = np.linalg.norm(_o(plan, i) - O_ref) / np.linalg.norm(O_ref)
        worst = max(worst, r)
        assert r <= 1e-2, (W0.shape, r)
        assert torch.equal(_bits(plan.output(i)), _bits(tiled.output(i)))
    # a constant schedule is the plain call, bitwise
    p2, p3 = harness.Plan(_clone(orig)), harness.Plan(_clone(orig))
    p2.momentum_update(BETA)
    p2.ns_schedule([(A, B, C)] * K, EPS)
    p3.momentum_update(BETA)
    p3.ns_batched(A, B, C, K, EPS)
    torch.cuda.synchronize()
    for i in range(len(SHAPES)):
        assert torch.equal(_bits(p2.output(i)), _bits(p3.output(i)))
    print(f"schedule: worst NS rel err {worst:.2e}")
    for pl in (plan, tiled, p2, p3):
        pl.close()


def test_long_schedule_takes_the_tiled_kernels_for_small_chunks():
    from muon_newton_schulz_momentum_amd import binding as L, harness
    ps = _params([(64, 128), (32, 256)], seed=520)
    tiled_ps = _clone(ps)
    plan = harness.Plan(ps)
    tiled = harness.Plan(tiled_ps, flags=L.MUON_PLAN_TILED_SMALL)
    assert all(plan.chunk_info(c).fused_small for c in range(plan.n_chunks))
    for pl in (plan, tiled):
        pl.momentum_update(BETA)
        pl.ns_schedule([(A, B, C)] * 40, EPS)     # longer than the fused kernel's table
    torch.cuda.synchronize()
    for i in range(2):
        assert torch.equal(_bits(plan.output(i)), _bits(tiled.output(i)))
        assert torch.isfinite(plan.output(i).float()).all()
    plan.close()
    tiled.close()


def test_nesterov_lookahead():
    from muon_newton_schulz_momentum_amd import harness
    ps = _params(SHAPES, seed=530)
    snap = _snap(ps)
    plan = harness.Plan(ps)
    plan.step_ex(BETA, LR, WD, nesterov=True)
    torch.cuda.synchronize()
    for i, (W0, M0, G0) in enumerate(snap):
        M_ref, X0 = orc.momentum_update(M0, G0, BETA, nesterov=True)
        assert np.array_equal(ps[i].momentum.cpu().numpy(), M_ref)
        O_ref = orc.newton_schulz(X0, A, B, C, K, EPS, emulate_bf16=True)
        O = _o(plan, i)
        assert np.linalg.norm(O - O_ref) / np.linalg.norm(O_ref) <= 1e-2
        assert np.array_equal(ps[i].weight.cpu().numpy(), orc.apply_update(W0, O, LR, WD))
    plan.close()


def test_device_scalars_follow_a_schedule_in_graph_replays():
    from muon_newton_schulz_momentum_amd import harness
    ps = _params(SHAPES, seed=540)
    eager_ps = _clone(ps)
    dev = torch.tensor([BETA, LR, WD], dtype=torch.float32, device="cuda")
    plan = harness.Plan(ps)
    eager = harness.Plan(eager_ps)
    g = plan.capture_ex(0.0, 0.0, 0.0, dev_scalars=dev)    # host values ignored
    lrs = [0.02, 0.015, 0.01, 0.004]
    betas = [0.95, 0.9, 0.95, 0.8]
    for lr_t, beta_t in zip(lrs, betas):
        dev.copy_(torch.tensor([beta_t, lr_t, WD], dtype=torch.float32))   # ordered before the launch
        g.launch()
        eager.step(beta_t, lr_t, WD, A, B, C, K, EPS)
        torch.cuda.synchronize()
        for pe, pg in zip(eager_ps, ps):
            assert torch.equal(_bits(pe.weight), _bits(pg.weight))
            assert torch.equal(_bits(pe.momentum), _bits(pg.momentum))
    g.close()
    plan.close()
    eager.close()
