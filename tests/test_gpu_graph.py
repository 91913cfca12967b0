"""The whole step captured as one HIP graph (muon_graph_capture / muon_graph_launch).

Each replay is checked against the same step run eagerly on an identical copy of the
inputs: W, M and the Newton–Schulz output O must be bitwise equal, replay after replay,
with new gradients written into the captured G buffers before every replay and with
unrelated torch work and host synchronisations between replays.  The first step is also
checked against the float64 oracle, so the graph path is anchored to it and not only to
the eager path.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from oracle import muon_oracle as orc  # noqa: E402

A, B, C, K, EPS = 3.4445, -4.7750, 2.0315, 5, 1e-7
BETA, LR, WD = 0.95, 0.02, 0.1


def _pair(shapes, seed):
    """Two identical parameter sets on the GPU."""
    from muon_newton_schulz_momentum_amd.harness import ParamTensors
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    first, second = [], []
    for s in shapes:
        W = torch.randn(s, generator=gen, device="cuda") * 0.02
        M = torch.randn(s, generator=gen, device="cuda") * 1e-3
        G = torch.randn(s, generator=gen, device="cuda") * 1e-3
        first.append(ParamTensors(W, M, G))
        second.append(ParamTensors(W.clone(), M.clone(), G.clone()))
    return first, second


def _bits(t):
    return t.detach().contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu()


def _other_work():
    """Unrelated eager work on the same stream, then a host synchronisation."""
    x = torch.randn(512, 512, device="cuda")
    y = (x @ x.t()).sum(dim=0)
    torch.cuda.synchronize()
    return float(y[0])


def _replay_against_eager(shapes, seed, replays, max_ws=0):
    from muon_newton_schulz_momentum_amd import harness
    eager_p, graph_p = _pair(shapes, seed)
    snap = [(p.weight.cpu().numpy(), p.momentum.cpu().numpy(), p.grad.cpu().numpy()) for p in eager_p]
    eager = harness.Plan(eager_p, max_workspace_bytes=max_ws)
    plan = harness.Plan(graph_p, max_workspace_bytes=max_ws)
    torch.cuda.synchronize()
    g = plan.capture(BETA, LR, WD, A, B, C, K, EPS)
    infos = [plan.chunk_info(c) for c in range(plan.n_chunks)]
    fused = sum(i.fused_small for i in infos)
    grouped = sum(i.grouped_small for i in infos)
    big = [i for i in infos if not i.fused_small and not i.grouped_small]
    # momentum + apply per chunk; 256-tile chunks: finalize (and normalize unless the first
    # iteration's loads normalise: odd K), 3 per iteration; small tiled chunks: one grouped
    # normalisation and 3 grouped launches per iteration (up to 12 chunks each); fused
    # chunks: one grouped launch (up to 8 chunks) when the chunks have their own regions
    prep = sum(1 if (i.tile == 256 and K % 2 == 1) else 2 for i in big)
    small_launches = fused if infos[0].shared_region else -(-fused // 8)
    group_launches = -(-grouped // 12) * (1 + 3 * K)
    assert g.nodes == 2 * plan.n_chunks + prep + 3 * K * len(big) + small_launches + group_launches
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed + 1)
    for r in range(replays):
        if r > 0:   # a fresh gradient, written in place into the captured G buffers
            for pe, pg in zip(eager_p, graph_p):
                new = torch.randn(pe.grad.shape, generator=gen, device="cuda") * 1e-3
                pe.grad.copy_(new)
                pg.grad.copy_(new)
        eager.step(BETA, LR, WD, A, B, C, K, EPS)
        g.launch()
        torch.cuda.synchronize()
        for i, (pe, pg) in enumerate(zip(eager_p, graph_p)):
            assert torch.equal(_bits(pe.momentum), _bits(pg.momentum)), f"replay {r}: momentum of {i}"
            assert torch.equal(_bits(pe.weight), _bits(pg.weight)), f"replay {r}: weight of {i}"
            if pe.weight.dim() == 2:
                assert torch.equal(_bits(eager.output(i)), _bits(plan.output(i))), f"replay {r}: O of {i}"
        if r == 0:   # anchor the first replay to the oracle
            # a region shared by several chunks holds the last of them's outputs
            last = {}
            for ch in range(plan.n_chunks):
                last[plan.chunk_info(ch).region_offset] = ch
            for i, (W0, M0, G0) in enumerate(snap):
                if W0.ndim != 2:
                    continue
                ch = plan.param_info(i).chunk
                if last[plan.chunk_info(ch).region_offset] != ch:
                    continue
                M_ref, X0 = orc.momentum_update(M0, G0, BETA)
                assert np.array_equal(graph_p[i].momentum.cpu().numpy(), M_ref)
                O_ref = orc.newton_schulz(X0, A, B, C, K, EPS, emulate_bf16=True)
                O = plan.output_oriented(i).float().cpu().numpy().astype(np.float64)
                assert np.linalg.norm(O - O_ref) / np.linalg.norm(O_ref) <= 1e-2
        _other_work()
    g.close()
    eager.close()
    plan.close()


def test_graph_replays_equal_eager_steps():
    _replay_against_eager([(64, 128), (200, 72), (72, 200), (257, 300), (300,), (130, 130), (64, 128)],
                          seed=301, replays=4)


def test_graph_over_chunks_sharing_one_region():
    # a workspace cap that forces several chunks of one bucket into one shared region
    shapes = [(256, 384)] * 6 + [(96, 160)] * 3
    from muon_newton_schulz_momentum_amd import harness
    probe, _ = _pair(shapes, 7)
    full = harness.Plan(probe, bind=False)
    cap = full.workspace_bytes // 3
    full.close()
    capped = harness.Plan(probe, max_workspace_bytes=cap, bind=False)
    assert capped.n_chunks > 2 and any(capped.chunk_info(c).shared_region for c in range(capped.n_chunks))
    capped.close()
    _replay_against_eager(shapes, seed=302, replays=3, max_ws=cap)


def test_graph_on_a_side_stream_orders_with_torch_work():
    """Launch on a non-default torch stream right after torch writes G on that stream."""
    from muon_newton_schulz_momentum_amd import harness
    eager_p, graph_p = _pair([(128, 256), (256, 128)], seed=303)
    eager = harness.Plan(eager_p)
    plan = harness.Plan(graph_p)
    g = plan.capture(BETA, LR, WD, A, B, C, K, EPS)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        for pe, pg in zip(eager_p, graph_p):
            pg.grad.mul_(3.0)    # queued on `side`, must land before the graph reads G
        g.launch(side)
    side.synchronize()
    for pe in eager_p:
        pe.grad.mul_(3.0)
    eager.step(BETA, LR, WD, A, B, C, K, EPS)
    torch.cuda.synchronize()
    for pe, pg in zip(eager_p, graph_p):
        assert torch.equal(_bits(pe.weight), _bits(pg.weight))
        assert torch.equal(_bits(pe.momentum), _bits(pg.momentum))
    g.close()
