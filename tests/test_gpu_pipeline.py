"""The two-stream pipeline (muon_step_config.pipeline): the next chunk's momentum and
normaliser and the previous chunk's apply run on a second stream beside the current
chunk's Newton–Schulz products, in the side-stream kernels.  Its results must be bitwise
those of the one-stream step: momentum, weights and the orthogonalised outputs, eagerly
and in graph replays, with and without a workspace cap (double-buffered regions), for
fp32 and bf16 gradients, transposed and ragged shapes, and the Nesterov and device-scalar
variants.  One chunk of each run is also checked against the float64 oracle.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from oracle import muon_oracle as orc  # noqa: E402

A, B, C, K, EPS = 3.4445, -4.7750, 2.0315, 5, 1e-7
BETA, LR, WD = 0.95, 0.02, 0.1

# Several tiled buckets (both orientations, padded n != cols, cols not a multiple of 4,
# bf16 gradients) and one fused small bucket.
SHAPES = [
    ((300, 520), "f32"), ((520, 300), "f32"), ((300, 520), "f32"),     # one bucket, both orientations
    ((130, 257), "bf16"), ((257, 130), "bf16"),                        # cols % 4 != 0, bf16 G
    ((1024, 768), "f32"), ((768, 1024), "f32"),
    ((96, 1000), "f32"),
    ((64, 200), "f32"), ((200, 64), "f32"),                            # fused small bucket
    ((513, 1030), "f32"),                                              # ragged tail in both
]


def _params(shapes, seed):
    from muon_newton_schulz_momentum_amd.harness import ParamTensors
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    out = []
    for shape, gdt in shapes:
        W = torch.randn(shape, generator=gen, device="cuda") * 0.02
        M = torch.randn(shape, generator=gen, device="cuda") * 1e-3
        G = torch.randn(shape, generator=gen, device="cuda") * 1e-3
        if gdt == "bf16":
            G = G.to(torch.bfloat16)
        out.append(ParamTensors(W, M, G))
    return out


def _clone(params):
    from muon_newton_schulz_momentum_amd.harness import ParamTensors
    return [ParamTensors(p.weight.clone(), p.momentum.clone(), p.grad.clone()) for p in params]


def _bits(t):
    return t.detach().contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu()


def _same(pa, pb, plan_a, plan_b, what):
    for i, (x, y) in enumerate(zip(pa, pb)):
        assert torch.equal(_bits(x.momentum), _bits(y.momentum)), (what, "M", i)
        assert torch.equal(_bits(x.weight), _bits(y.weight)), (what, "W", i)
        assert torch.equal(_bits(plan_a.output(i)), _bits(plan_b.output(i))), (what, "O", i)


def _tiled_chunks(plan):
    return [c for c in range(plan.n_chunks) if not plan.chunk_info(c).fused_small]


def _oracle_anchor(snap, plan, params, index, nesterov=False):
    W0, M0, G0 = snap
    M_ref, X0 = orc.momentum_update(M0, G0, BETA, nesterov=nesterov)
    assert np.array_equal(params[index].momentum.cpu().numpy(), M_ref)
    O = plan.output_oriented(index).float().cpu().numpy().astype(np.float64)
    O_ref = orc.newton_schulz(X0, A, B, C, K, EPS, emulate_bf16=True)
    r = np.linalg.norm(O - O_ref) / np.linalg.norm(O_ref)
    assert r <= 1e-2, r
    assert np.array_equal(params[index].weight.cpu().numpy(), orc.apply_update(W0, O, LR, WD))


def _snap(p):
    return (p.weight.cpu().numpy(), p.momentum.cpu().numpy(), p.grad.float().cpu().numpy())


@pytest.mark.parametrize("nesterov,dev", [(False, False), (True, True)])
def test_pipeline_eager_matches_one_stream(nesterov, dev):
    from muon_newton_schulz_momentum_amd import harness
    ps = _params(SHAPES, seed=700 + int(nesterov))
    ref_ps = _clone(ps)
    anchor = len(SHAPES) - 1
    snap = _snap(ps[anchor])
    plan, ref = harness.Plan(ps), harness.Plan(ref_ps)
    assert len(_tiled_chunks(plan)) >= 4
    kw = dict(nesterov=nesterov)
    if dev:
        kw["dev_scalars"] = torch.tensor([BETA, LR, WD], dtype=torch.float32, device="cuda")
    for step in range(2):
        plan.step_ex(BETA, LR, WD, pipeline=True, **kw)
        ref.step_ex(BETA, LR, WD, pipeline=False, **kw)
        torch.cuda.synchronize()
        _same(ps, ref_ps, plan, ref, f"eager step {step}")
        if step == 0:
            _oracle_anchor(snap, plan, ps, anchor, nesterov=nesterov)
    plan.close()
    ref.close()


def test_pipeline_graph_replays_match_one_stream():
    from muon_newton_schulz_momentum_amd import harness
    ps = _params(SHAPES, seed=710)
    ref_ps = _clone(ps)
    plan, ref = harness.Plan(ps), harness.Plan(ref_ps)
    g = plan.capture_ex(BETA, LR, WD, pipeline=True)
    g_ref = ref.capture_ex(BETA, LR, WD)
    print(f"graph nodes: pipeline {g.nodes}, one stream {g_ref.nodes}")
    assert g.nodes == g_ref.nodes        # the fork and join are edges, not nodes
    for r in range(3):
        g.launch()
        ref.step_ex(BETA, LR, WD)        # eager one-stream steps as the reference
        torch.cuda.synchronize()
        _same(ps, ref_ps, plan, ref, f"replay {r}")
        x = torch.ones(1 << 20, device="cuda").sum()   # unrelated eager work between replays
        assert float(x) == float(1 << 20)
    g.close()
    g_ref.close()
    plan.close()
    ref.close()


def test_pipeline_with_double_buffered_workspace_cap():
    from muon_newton_schulz_momentum_amd import binding as L, harness
    shapes = [((512, 768), "f32")] * 12 + [((768, 512), "bf16")] * 6 + [((64, 96), "f32")] * 3
    ps = _params(shapes, seed=720)
    ref_ps = _clone(ps)
    free = harness.Plan(_clone(ps), bind=False)
    cap = free.workspace_bytes // 3
    free.close()
    plan = harness.Plan(ps, max_workspace_bytes=cap, flags=L.MUON_PLAN_PIPELINE)
    ref = harness.Plan(ref_ps)                  # no cap: its own chunking, same per-matrix math
    assert plan.workspace_bytes <= cap
    tiled = _tiled_chunks(plan)
    assert len(tiled) >= 4
    offs = [plan.chunk_info(c).region_offset for c in tiled]
    assert all(offs[j] != offs[j - 1] for j in range(1, len(offs))) and len(set(offs)) == 2
    # the oracle anchor: a matrix of the last tiled chunk, whose outputs stay in place
    anchor = next(i for i in range(len(shapes)) if plan.param_info(i).chunk == tiled[-1])
    snap = _snap(ps[anchor])
    for step in range(2):
        plan.step_ex(BETA, LR, WD, pipeline=True)
        ref.step_ex(BETA, LR, WD)
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(ps, ref_ps)):
            assert torch.equal(_bits(x.momentum), _bits(y.momentum)), ("M", i)
            assert torch.equal(_bits(x.weight), _bits(y.weight)), ("W", i)
        if step == 0:
            _oracle_anchor(snap, plan, ps, anchor)
    # a single shared region cannot pipeline: the step runs one chunk at a time, same bits
    single_ps = _clone(ref_ps)
    single = harness.Plan(single_ps, max_workspace_bytes=cap)
    single.step_ex(BETA, LR, WD, pipeline=True)
    ref.step_ex(BETA, LR, WD)
    torch.cuda.synchronize()
    for i, (x, y) in enumerate(zip(single_ps, ref_ps)):
        assert torch.equal(_bits(x.weight), _bits(y.weight)), ("W single", i)
    for pl in (plan, ref, single):
        pl.close()


def test_pipeline_with_adamw_params():
    from muon_newton_schulz_momentum_amd import binding as L, harness
    from muon_newton_schulz_momentum_amd.harness import ParamTensors
    ps = _params(SHAPES[:8], seed=730)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(731)

    def adam_param():
        W = torch.randn(4099, generator=gen, device="cuda") * 0.02
        M = torch.zeros(4099, device="cuda")
        G = torch.randn(4099, generator=gen, device="cuda") * 1e-3
        V = torch.zeros(4099, device="cuda")
        return ParamTensors(W, M, G, exp_avg_sq=V, optimizer=L.MUON_OPT_ADAMW)

    ps.append(adam_param())
    ref_ps = _clone(ps[:8]) + [ParamTensors(ps[8].weight.clone(), ps[8].momentum.clone(), ps[8].grad.clone(),
                                            exp_avg_sq=ps[8].exp_avg_sq.clone(), optimizer=L.MUON_OPT_ADAMW)]
    plan, ref = harness.Plan(ps), harness.Plan(ref_ps)
    ad = harness.Plan.adamw_config(1e-3, 0.9, 0.95, 1e-8, 0.1, 1)
    plan.step_ex(BETA, LR, WD, pipeline=True, adamw=ad)
    ref.step_ex(BETA, LR, WD, adamw=ad)
    torch.cuda.synchronize()
    for i, (x, y) in enumerate(zip(ps, ref_ps)):
        assert torch.equal(_bits(x.weight), _bits(y.weight)), ("W", i)
        assert torch.equal(_bits(x.momentum), _bits(y.momentum)), ("M", i)
    assert torch.equal(_bits(ps[8].exp_avg_sq), _bits(ref_ps[8].exp_avg_sq))
    plan.close()
    ref.close()


def test_pipeline_plan_splits_a_large_bucket_and_places_by_window():
    # a large expert-like bucket (split into two chunks by MUON_PLAN_PIPELINE, plus edge
    # chunks) and a one-matrix router chunk, which goes last: its window is far too short
    # to hide the experts' apply, which then runs at full speed on the caller's stream;
    # bits as one stream
    from muon_newton_schulz_momentum_amd import binding as L, harness
    shapes = [((1024, 1536), "f32")] * 420 + [((512, 1536), "f32")]
    ps = _params(shapes, seed=740)
    ref_ps = _clone(ps)
    plan = harness.Plan(ps, flags=L.MUON_PLAN_PIPELINE)
    ref = harness.Plan(ref_ps)
    assert 3 <= plan.n_chunks <= 5 and ref.n_chunks == 2
    assert plan.chunk_info(plan.n_chunks - 1).m == 512
    anchor = 0
    snap = _snap(ps[anchor])
    for step in range(2):
        plan.step_ex(BETA, LR, WD, pipeline=True)
        ref.step_ex(BETA, LR, WD)
        torch.cuda.synchronize()
        _same(ps, ref_ps, plan, ref, f"split step {step}")
        if step == 0:
            _oracle_anchor(snap, plan, ps, anchor)
    g = plan.capture_ex(BETA, LR, WD, pipeline=True)
    g.launch()
    ref.step_ex(BETA, LR, WD)
    torch.cuda.synchronize()
    _same(ps, ref_ps, plan, ref, "split replay")
    g.close()
    plan.close()
    ref.close()


def test_pipeline_argument_checks_and_rebind():
    import ctypes as C
    from muon_newton_schulz_momentum_amd import binding as L, harness
    ps = _params(SHAPES[:8], seed=750)
    ref_ps = _clone(ps)
    plan, ref = harness.Plan(ps), harness.Plan(ref_ps)
    k, keep = harness.Plan.config(BETA, LR, WD)
    k.pipeline = 2
    assert L.muon_step_ex(plan._plan, -1, C.byref(k), None) == L.MUON_ERR_INVALID_ARG
    assert b"pipeline" in L.muon_last_error()
    # binding again (same workspace) keeps the plan's side stream and events usable
    plan.bind()
    plan.step_ex(BETA, LR, WD, pipeline=True)
    ref.step_ex(BETA, LR, WD)
    torch.cuda.synchronize()
    _same(ps, ref_ps, plan, ref, "after rebind")
    del keep
    plan.close()
    ref.close()


def test_random_shape_mixes_two_stream_equal_one_stream():
    # Ten seeded random mixes of shapes (1 to 2300 rows and columns, both orientations, up
    # to four buckets, fp32 or bf16 gradients): the two-stream step, uncapped and under a
    # cap of a third of the one-stream workspace, bitwise equal to the one-stream step; the
    # first and last matrix of each mix against the oracle.
    from muon_newton_schulz_momentum_amd import binding as L, harness
    rng = np.random.default_rng(7)
    dims = [1, 5, 32, 64, 65, 96, 130, 200, 256, 300, 512, 700, 1024, 1100, 1536, 2048, 2300]
    for trial in range(10):
        shapes = []
        for _ in range(int(rng.integers(1, 5))):
            r, c = int(rng.choice(dims)), int(rng.choice(dims))
            shapes += [(r, c)] * int(rng.integers(1, 40 if max(r, c) >= 1024 else 80))
        gdt = "bf16" if rng.random() < 0.3 else "f32"
        base = _params([(s, gdt) for s in shapes], seed=1000 + trial)
        ref_ps = _clone(base)
        ref = harness.Plan(ref_ps)
        ref.step_ex(BETA, LR, WD)
        torch.cuda.synchronize()
        for cap in (0, ref.workspace_bytes // 3):
            ps = _clone(base)
            try:
                plan = harness.Plan(ps, max_workspace_bytes=cap, flags=L.MUON_PLAN_PIPELINE)
            except L.MuonError as e:
                assert cap and e.status == L.MUON_ERR_WORKSPACE_TOO_SMALL, e
                continue
            plan.step_ex(BETA, LR, WD, pipeline=True)
            torch.cuda.synchronize()
            for i, (a, b) in enumerate(zip(ps, ref_ps)):
                assert torch.equal(a.weight, b.weight) and torch.equal(a.momentum, b.momentum), (trial, cap, i)
            plan.close()
        snap = {i: _snap(base[i]) for i in (0, len(shapes) - 1)}
        for i in snap:
            _oracle_anchor(snap[i], ref, ref_ps, i)
        ref.close()
