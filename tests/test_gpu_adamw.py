"""The AdamW companion: the parameters the pages leave to AdamW (norms, scalars,
embeddings) updated by the library, bitwise against the float64 oracle (same operation
order, one rounding each), alone, next to Muon matrices in one call, and in graph replays
that follow the step count through device-resident settings.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from oracle import muon_oracle as orc  # noqa: E402

LR, B1, B2, EPS, WD = 3e-4, 0.9, 0.95, 1e-8, 0.1


def _adam_params(specs, seed):
    """specs: (shape, grad dtype, optimizer) -> ParamTensors with W, M, V, G."""
    from muon_newton_schulz_momentum_amd import binding as L
    from muon_newton_schulz_momentum_amd.harness import ParamTensors
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    out = []
    for shape, gdt, opt in specs:
        W = torch.randn(shape, generator=gen, device="cuda") * 0.02
        M = torch.randn(shape, generator=gen, device="cuda") * 1e-3
        V = torch.rand(shape, generator=gen, device="cuda") * 1e-6
        G = (torch.randn(shape, generator=gen, device="cuda") * 1e-3).to(gdt)
        out.append(ParamTensors(W, M, G, exp_avg_sq=V, optimizer=opt if opt is not None else L.MUON_OPT_DEFAULT))
    return out


def _host(t):
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


def _check(ps, snaps, step):
    for i, (p, (W0, M0, V0, G0)) in enumerate(zip(ps, snaps)):
        w, m, v = orc.adamw_update(W0, M0, V0, G0, lr=LR, beta1=B1, beta2=B2, eps=EPS, wd=WD, step=step)
        assert np.array_equal(_host(p.momentum).reshape(-1).view(np.uint32), m.reshape(-1).view(np.uint32)), f"m of {i}"
        assert np.array_equal(_host(p.exp_avg_sq).reshape(-1).view(np.uint32), v.reshape(-1).view(np.uint32)), f"v of {i}"
        assert np.array_equal(_host(p.weight).reshape(-1).view(np.uint32), w.reshape(-1).view(np.uint32)), f"w of {i}"


def _snap(ps):
    return [(_host(p.weight), _host(p.momentum), _host(p.exp_avg_sq), _host(p.grad)) for p in ps]


def test_adamw_alone_bitwise_over_steps():
    from muon_newton_schulz_momentum_amd import binding as L, harness
    specs = [((4096,), torch.float32, None), ((4099,), torch.float32, None), ((3,), torch.float32, None),
             ((1000, 64), torch.float32, L.MUON_OPT_ADAMW), ((5000,), torch.bfloat16, None),
             ((2, 3, 5), torch.float32, None)]
    ps = _adam_params(specs, seed=600)
    plan = harness.Plan(ps)
    assert plan.n_chunks == 0 and plan.adamw_counts() == (6, 4096 + 4099 + 3 + 64000 + 5000 + 30)
    for t in (1, 2, 3):
        snaps = _snap(ps)
        plan.adamw_step(LR, B1, B2, EPS, WD, t)
        torch.cuda.synchronize()
        _check(ps, snaps, t)
        for p in ps:                       # a new gradient for the next step
            p.grad.copy_(torch.randn(p.grad.shape, device="cuda").to(p.grad.dtype) * 1e-3)
    plan.close()


def test_one_call_updates_muon_and_adamw_parameters():
    from muon_newton_schulz_momentum_amd import binding as L, harness
    from muon_newton_schulz_momentum_amd.harness import ParamTensors
    adam = _adam_params([((2048,), torch.float32, None), ((512, 64), torch.float32, L.MUON_OPT_ADAMW)], seed=610)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(611)
    muon = [ParamTensors(torch.randn(s, generator=gen, device="cuda") * 0.02,
                         torch.randn(s, generator=gen, device="cuda") * 1e-3,
                         torch.randn(s, generator=gen, device="cuda") * 1e-3) for s in ((256, 512), (512, 256))]
    params = muon + adam
    msnap = [(p.weight.cpu().numpy(), p.momentum.cpu().numpy(), p.grad.cpu().numpy()) for p in muon]
    asnap = _snap(adam)
    plan = harness.Plan(params)
    k = plan.adamw_config(LR, B1, B2, EPS, WD, 1)
    plan.timing_enable(64)
    plan.step_ex(0.95, 0.02, 0.1, adamw=k)
    torch.cuda.synchronize()
    _check(adam, asnap, 1)
    for i, (W0, M0, G0) in enumerate(msnap):
        M_ref, X0 = orc.momentum_update(M0, G0, 0.95)
        assert np.array_equal(muon[i].momentum.cpu().numpy(), M_ref)
        O = plan.output_oriented(i).float().cpu().numpy().astype(np.float64)
        O_ref = orc.newton_schulz(X0, 3.4445, -4.775, 2.0315, 5, 1e-7)
        assert np.linalg.norm(O - O_ref) / np.linalg.norm(O_ref) <= 1e-2
        assert np.array_equal(muon[i].weight.cpu().numpy(), orc.apply_update(W0, O, 0.02, 0.1))
    ms, n, work = plan.timing_read(L.MUON_KERNEL_ADAMW)
    assert n == 1 and work == (2048 + 512 * 64) * 28.0
    plan.timing_enable(0)
    plan.close()


def test_graph_follows_adamw_step_through_device_scalars():
    from muon_newton_schulz_momentum_amd import harness
    ps = _adam_params([((4096,), torch.float32, None), ((777,), torch.bfloat16, None)], seed=620)
    eager_ps = [type(p)(p.weight.clone(), p.momentum.clone(), p.grad.clone(), p.exp_avg_sq.clone(), p.optimizer)
                for p in ps]
    plan = harness.Plan(ps)
    eager = harness.Plan(eager_ps)
    dev_muon = torch.tensor([0.95, 0.0, 0.0], device="cuda")
    dev_adam = torch.zeros(4, device="cuda")
    k = plan.adamw_config(0.0, B1, B2, EPS, 0.0, 1, dev_scalars=dev_adam)
    g = plan.capture_ex(0.95, 0.0, 0.0, dev_scalars=dev_muon, adamw=k)
    for t in (1, 2, 3, 4):
        bc1 = np.float32(1.0 - float(np.float32(B1)) ** t)
        bc2 = np.float32(1.0 - float(np.float32(B2)) ** t)
        dev_adam.copy_(torch.tensor([LR, WD, bc1, bc2], dtype=torch.float32))
        g.launch()
        # eager reference with the same float32 bias corrections, through device scalars too
        ke = eager.adamw_config(0.0, B1, B2, EPS, 0.0, 1, dev_scalars=dev_adam)
        eager.adamw_step(0.0, B1, B2, EPS, 0.0, 1, dev_scalars=dev_adam)
        torch.cuda.synchronize()
        for pe, pg in zip(eager_ps, ps):
            assert torch.equal(pe.weight, pg.weight) and torch.equal(pe.exp_avg_sq, pg.exp_avg_sq)
        del ke
    g.close()
    plan.close()
    eager.close()
