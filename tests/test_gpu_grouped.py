"""The grouped launches of the small tiled chunks (routers, gates, narrow KV projections).

Every small tiled chunk of a plan (128- or 64-row tiles: 64 < m < 1024, or m <= 64 with a
padded n above 1024) is normalised by one launch and orthogonalised by one launch per
product and iteration over a single tile queue.

* Bitwise equal to the per-chunk launches (the same plan built with MUON_PLAN_UNGROUPED):
  W, M and O, for 128- and 64-tile buckets in both orientations next to a 256-tile chunk
  and a fused small chunk; one matrix per small bucket also against the float64 oracle.
* Launch count: the MoE slice's four small buckets take 1 + 3k launches in all.
* More chunks than one launch takes (two launches per product).
* In the two-stream step (the group as one unit), under a workspace cap that makes the
  chunks share regions, in graph replays, and stepped chunk by chunk: bitwise the same.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from oracle import muon_oracle as orc  # noqa: E402

A, B, C, K, EPS = 3.4445, -4.7750, 2.0315, 5, 1e-7
BETA, LR, WD = 0.95, 0.02, 0.1
SHAPES = [(512, 4096), (4096, 512), (256, 4096), (32, 4096), (4096, 32), (1, 4096), (300, 700),
          (700, 300), (130, 1100), (1024, 1024), (64, 128)]


def _params(shapes, seed, gdtype=torch.float32):
    from muon_newton_schulz_momentum_amd.harness import ParamTensors
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    out = []
    for s in shapes:
        W = torch.randn(s, generator=gen, device="cuda") * 0.02
        M = torch.randn(s, generator=gen, device="cuda") * 1e-3
        G = (torch.randn(s, generator=gen, device="cuda") * 1e-3).to(gdtype)
        out.append(ParamTensors(W, M, G))
    return out


def _clone(params):
    from muon_newton_schulz_momentum_amd.harness import ParamTensors
    return [ParamTensors(p.weight.clone(), p.momentum.clone(), p.grad.clone()) for p in params]


def _bits(t):
    return t.detach().contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu()


def _same_params(pa, pb, what):
    for i, (a, b) in enumerate(zip(pa, pb)):
        assert torch.equal(_bits(a.weight), _bits(b.weight)), f"{what}: W of {i}"
        assert torch.equal(_bits(a.momentum), _bits(b.momentum)), f"{what}: M of {i}"


def test_grouped_equals_per_chunk_bitwise_and_oracle():
    from muon_newton_schulz_momentum_amd import binding as L, harness
    gp = _params(SHAPES, seed=801)
    up = _clone(gp)
    snap = [(p.weight.cpu().numpy(), p.momentum.cpu().numpy(), p.grad.cpu().numpy()) for p in gp]
    grouped = harness.Plan(gp)
    single = harness.Plan(up, flags=L.MUON_PLAN_UNGROUPED)
    n_grouped = sum(grouped.chunk_info(c).grouped_small for c in range(grouped.n_chunks))
    assert n_grouped == 6 and not any(single.chunk_info(c).grouped_small for c in range(single.n_chunks))
    grouped.step(BETA, LR, WD, A, B, C, K, EPS)
    single.step(BETA, LR, WD, A, B, C, K, EPS)
    torch.cuda.synchronize()
    for i in range(len(SHAPES)):
        assert torch.equal(_bits(grouped.output(i)), _bits(single.output(i))), f"O of {SHAPES[i]}"
    _same_params(gp, up, "grouped vs per chunk")
    seen, worst = set(), 0.0
    for i, (W0, M0, G0) in enumerate(snap):
        key = tuple(sorted(SHAPES[i]))
        if key in seen or not grouped.chunk_info(grouped.param_info(i).chunk).grouped_small:
            continue
        seen.add(key)
        M_ref, X0 = orc.momentum_update(M0, G0, BETA)
        assert np.array_equal(gp[i].momentum.cpu().numpy(), M_ref)
        O_ref = orc.newton_schulz(X0, A, B, C, K, EPS, emulate_bf16=True)
        O = grouped.output_oriented(i).float().cpu().numpy().astype(np.float64)
        r = np.linalg.norm(O - O_ref) / np.linalg.norm(O_ref)
        worst = max(worst, r)
        assert r <= 1e-2, f"{SHAPES[i]}: {r:.3e}"
        assert np.array_equal(gp[i].weight.cpu().numpy(), orc.apply_update(W0, O, LR, WD))
    assert len(seen) == 6
    print(f"grouped small chunks: worst NS rel err {worst:.2e}")
    grouped.close()
    single.close()


def test_grouped_launch_count_of_the_moe_slice_small_buckets():
    from muon_newton_schulz_momentum_amd import binding as L, harness
    shapes = [(512, 4096)] * 4 + [(256, 4096)] * 2 + [(32, 4096)] * 4 + [(1, 4096)] * 4
    pl = harness.Plan(_params(shapes, seed=802, gdtype=torch.bfloat16))
    assert pl.n_chunks == 4
    pl.momentum_update(BETA)
    pl.timing_enable(256)
    pl.ns_batched(A, B, C, K, EPS)
    torch.cuda.synchronize()
    counts = {L.muon_kernel_name(k).decode(): pl.timing_read(k)[1] for k in range(L.MUON_KERNEL_COUNT)}
    launches = sum(counts.values())
    assert counts["ns_grouped"] == 3 * K and counts["prep_grouped"] == 1, counts
    assert launches == 1 + 3 * K, counts
    pl.close()


def test_more_chunks_than_one_grouped_launch_takes():
    from muon_newton_schulz_momentum_amd import binding as L, harness
    shapes = [(64 + 37 * k, 1100 + 13 * k) for k in range(14)] + [(1024, 1536)]
    gp = _params(shapes, seed=803)
    up = _clone(gp)
    grouped = harness.Plan(gp)
    single = harness.Plan(up, flags=L.MUON_PLAN_UNGROUPED)
    assert sum(grouped.chunk_info(c).grouped_small for c in range(grouped.n_chunks)) == 14
    grouped.timing_enable(512)
    grouped.step(BETA, LR, WD, A, B, C, 3, EPS)
    single.step(BETA, LR, WD, A, B, C, 3, EPS)
    torch.cuda.synchronize()
    assert grouped.timing_read(L.MUON_KERNEL_NS_GROUPED)[1] == 2 * 3 * 3
    assert grouped.timing_read(L.MUON_KERNEL_PREP_GROUPED)[1] == 2
    for i in range(len(shapes)):
        assert torch.equal(_bits(grouped.output(i)), _bits(single.output(i))), f"O of {shapes[i]}"
    _same_params(gp, up, "14 grouped chunks")
    grouped.close()
    single.close()


def test_grouped_in_two_stream_step_capped_regions_and_graphs():
    from muon_newton_schulz_momentum_amd import binding as L, harness
    shapes = [(1024, 2048)] * 6 + [(2048, 1024)] * 2 + [(512, 2048)] * 2 + [(32, 2048), (100, 1500), (64, 128)]
    base = _params(shapes, seed=804, gdtype=torch.bfloat16)
    ref_p, pipe_p, cap_p, graph_p, chunk_p = base, _clone(base), _clone(base), _clone(base), _clone(base)
    ref = harness.Plan(ref_p, flags=L.MUON_PLAN_UNGROUPED)
    pipe = harness.Plan(pipe_p, flags=L.MUON_PLAN_PIPELINE)
    need = pipe.workspace_bytes
    capped = harness.Plan(cap_p, flags=L.MUON_PLAN_PIPELINE, max_workspace_bytes=need // 2)
    graphed = harness.Plan(graph_p, flags=L.MUON_PLAN_PIPELINE)
    chunked = harness.Plan(chunk_p, max_workspace_bytes=need // 2)
    assert capped.chunk_info(0).shared_region and chunked.chunk_info(0).shared_region
    for pl in (pipe, capped, graphed, chunked):
        assert sum(pl.chunk_info(c).grouped_small for c in range(pl.n_chunks)) == 3
    g = graphed.capture_ex(BETA, LR, WD, a=A, b=B, c=C, steps=K, eps=EPS, pipeline=True)
    for _ in range(2):
        ref.step(BETA, LR, WD, A, B, C, K, EPS)
        pipe.step_ex(BETA, LR, WD, a=A, b=B, c=C, steps=K, eps=EPS, pipeline=True)
        capped.step_ex(BETA, LR, WD, a=A, b=B, c=C, steps=K, eps=EPS, pipeline=True)
        g.launch()
        for ch in range(chunked.n_chunks):
            chunked.step(BETA, LR, WD, A, B, C, K, EPS, chunk=ch)
        torch.cuda.synchronize()
    for what, ps in (("two streams", pipe_p), ("capped two streams", cap_p), ("graph", graph_p),
                     ("chunk by chunk", chunk_p)):
        _same_params(ref_p, ps, what)
    for i in range(len(shapes)):
        assert torch.equal(_bits(pipe.output(i)), _bits(ref.output(i))), f"O of {shapes[i]}"
    g.close()
    for pl in (ref, pipe, capped, graphed, chunked):
        pl.close()
