"""Parity at the full sizes of the larger workloads, through the C ABI.

Every matrix of the workload is stepped on the GPU, with the one-stream plan and (for the
MoE slice also) in the benchmark's two-stream configuration for that workload; a sample
of matrices is then checked against the float64 oracle:
momentum bitwise, the Newton–Schulz output within 1e-2 relative Frobenius (the whole
five-iteration chain), and the apply bitwise given the GPU's own output.  The sample
covers every bucket, both orientations and the extreme per-expert gradient scales.

One of the 8704 x 8704 matrices is checked against the whole oracle chain (about 2e13
float64 FLOPs, a minute or two on the host).  Both are also checked one iteration at a
time: with beta = 0 the momentum step stages G exactly, and running k = 1..5 iterations
gives every intermediate X_k of the chain; sampled rows of X_k are compared with the
oracle's single iteration applied to the GPU's X_(k-1) (oracle.ns_iteration_rows), at a
tolerance of 2e-3 relative Frobenius per iteration (one iteration's bf16 rounding flips,
without the chaotic growth of the chained bar).
"""
import time

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from oracle import muon_oracle as orc  # noqa: E402

NS_TOL = 1e-2
ITER_TOL = 2e-3
GiB = 1 << 30


def _host(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 \
        else t.detach().cpu().numpy()


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def _need_bytes(w):
    tot = 0
    for p in w.params:
        e = int(np.prod(p.shape))
        tot += e * (8 + (2 if p.grad_dtype == "bf16" else 4))
    return tot


def _setup(key, sample_fn, reserve):
    import gc
    from muon_newton_schulz_momentum_amd import harness, workloads as wl
    w = wl.get(key)
    gc.collect()                      # earlier tests' tensors go back to the device
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    free, total = torch.cuda.mem_get_info()
    need = _need_bytes(w) + reserve
    print(f"[{key}] device memory: {free / 1e9:.1f} GB free of {total / 1e9:.1f} GB; need {need / 1e9:.1f} GB",
          flush=True)
    if need > free:
        pytest.skip(f"{key} needs {need / 1e9:.1f} GB of device memory; {free / 1e9:.1f} GB free")
    print(f"[{key}] generating {len(w.params)} parameters ({_need_bytes(w) / 1e9:.1f} GB)", flush=True)
    params = harness.make_params(w)
    torch.cuda.synchronize()
    sample = sample_fn(w)
    snap = {i: (_host(params[i].weight), _host(params[i].momentum), _host(params[i].grad)) for i in sample}
    return w, params, sample, snap


def _scale_extremes(w):
    """Indices of an expert matrix with the smallest and the largest gradient scale."""
    from muon_newton_schulz_momentum_amd import workloads as wl
    groups = sorted({p.group for p in w.params if p.group >= 0})
    sc = {g: wl.group_scale(w.cid, g) for g in groups}
    lo, hi = min(sc, key=sc.get), max(sc, key=sc.get)
    first = {}
    for i, p in enumerate(w.params):
        first.setdefault(p.group, []).append(i)
    return first[lo][0], first[hi][-1]


def _check(plan, params, snap, w, indices, full_chain=True):
    worst = 0.0
    for i in indices:
        W0, M0, G0 = snap[i]
        M_ref, X0 = orc.momentum_update(M0, G0, w.beta)
        assert np.array_equal(_host(params[i].momentum).view(np.uint32), M_ref.view(np.uint32)), \
            f"momentum of {w.params[i].name}"
        O_gpu = _host(plan.output_oriented(i))
        if full_chain:
            O_ref = orc.newton_schulz(X0, w.a, w.b, w.c, w.steps, w.eps, emulate_bf16=True)
            r = _rel(O_gpu, O_ref)
            worst = max(worst, r)
            print(f"  {w.params[i].name} {w.params[i].shape}: NS rel err {r:.2e}", flush=True)
            assert r <= NS_TOL, f"{w.params[i].name} {w.params[i].shape}: NS relative error {r:.3e}"
        W_ref = orc.apply_update(W0, O_gpu, w.lr, w.wd)
        assert np.array_equal(_host(params[i].weight).view(np.uint32), W_ref.view(np.uint32)), \
            f"apply of {w.params[i].name}"
    return worst


def _iterationwise(plan, params, w, i, rows):
    """Check every iteration of matrix i's chain on sampled rows (beta = 0 staging)."""
    ch = plan.param_info(i).chunk
    G0 = _host(params[i].grad)
    _, X0 = orc.momentum_update(_host(params[i].momentum), G0, 0.0)
    t = orc.canonical_orientation(*X0.shape)
    X = orc.frobenius_normalise(X0.T if t else X0, w.eps)
    prev = X
    for k in range(1, w.steps + 1):
        plan.momentum_update(0.0, chunk=ch)
        plan.ns_batched(w.a, w.b, w.c, k, w.eps, chunk=ch)
        torch.cuda.synchronize()
        Xk = _host(plan.output(i))
        ref = orc.ns_iteration_rows(prev, w.a, w.b, w.c, rows)
        r = _rel(Xk[rows], ref)
        print(f"  {w.params[i].name} iteration {k}: sampled-row rel err {r:.2e}", flush=True)
        assert r <= ITER_TOL, f"{w.params[i].name} iteration {k}: {r:.3e}"
        prev = Xk


@pytest.mark.timeout(900)
def test_moe_bucket_full_size():
    """512 experts x (1024x4096 x2, 4096x1024) + router 512x4096, uncapped workspace."""
    from muon_newton_schulz_momentum_amd import harness

    def pick(w):
        lo, hi = _scale_extremes(w)
        return sorted({0, 1, 2, lo, hi, len(w.params) - 2, len(w.params) - 1})
    w, params, sample, snap = _setup("moe_bucket", pick, reserve=45 * GiB)
    plan = harness.Plan(params)
    assert plan.n_buckets == 2
    plan.step(w.beta, w.lr, w.wd, w.a, w.b, w.c, w.steps, w.eps)
    torch.cuda.synchronize()
    worst = _check(plan, params, snap, w, sample)
    print(f"moe_bucket: {len(sample)} sampled matrices, worst NS rel err {worst:.2e}")
    plan.close()


@pytest.mark.timeout(900)
def test_full_width_share_full_size():
    """4 x 8704^2, shared expert 8704x3072 (x2) + 3072x8704, 21 x 1024x8704, router."""
    from muon_newton_schulz_momentum_amd import harness

    def pick(w):
        names = [p.name for p in w.params]
        return [names.index(n) for n in ("attn.q", "attn.v", "shared.gate", "shared.down", "e0.gate",
                                         "e6.down", "router")]
    w, params, sample, snap = _setup("full_width", pick, reserve=8 * GiB)
    plan = harness.Plan(params)
    assert plan.n_buckets == 4
    plan.step(w.beta, w.lr, w.wd, w.a, w.b, w.c, w.steps, w.eps)
    torch.cuda.synchronize()
    big = [i for i in sample if w.params[i].shape == (8704, 8704)]
    rest = [i for i in sample if i not in big]
    # one 8704^2 matrix against the whole five-iteration oracle chain (about 2e13 float64
    # FLOPs on the host), the other with momentum and apply only
    t0 = time.time()
    print(f"[full_width] whole-chain oracle for {w.params[big[0]].name} (8704 x 8704) ...", flush=True)
    worst_big = _check(plan, params, snap, w, big[:1])
    print(f"[full_width] whole chain done in {time.time() - t0:.0f} s", flush=True)
    _check(plan, params, snap, w, big[1:], full_chain=False)
    worst = max(worst_big, _check(plan, params, snap, w, rest))
    # the 8704^2 chain, iteration by iteration: rows at tile edges, inside, and the last
    rows = [0, 1, 255, 256, 4351, 4352, 6000, 8703]
    for i in big:
        _iterationwise(plan, params, w, i, rows)
    print(f"full_width: worst chained NS rel err {worst:.2e}")
    plan.close()


@pytest.mark.timeout(900)
def test_moe_slice_full_size_graph():
    """6184 matrices in 8 buckets, bf16 gradients, ~261 GB resident; chunked workspace,
    the step captured as one graph and replayed once."""
    from muon_newton_schulz_momentum_amd import harness

    def pick(w):
        names = [p.name for p in w.params]
        lo, hi = _scale_extremes(w)
        want = ["l0.q", "l1.shared.gate", "l0.k", "l3.v", "l2.router", "l3.head_gate", "l0.shared_gate",
                "l0.e0.gate", "l3.e511.down"]
        return sorted({names.index(n) for n in want} | {lo, hi})
    cap = 4 * GiB
    w, params, sample, snap = _setup("moe_slice", pick, reserve=cap + 2 * GiB)
    norms = [i for i, p in enumerate(w.params) if not p.is_matrix]
    norm_before = [params[i].weight.clone() for i in norms]
    plan = harness.Plan(params, max_workspace_bytes=cap)
    assert plan.n_buckets == 8 and plan.n_included == 6184 and plan.n_excluded == len(norms)
    print(f"[moe_slice] {plan.n_chunks} chunks in {plan.workspace_bytes / GiB:.2f} GiB of workspace", flush=True)
    g = plan.capture(w.beta, w.lr, w.wd, w.a, w.b, w.c, w.steps, w.eps)
    g.launch()
    torch.cuda.synchronize()
    g.close()
    for i, before in zip(norms, norm_before):
        assert torch.equal(params[i].weight, before)
    # The graph's momentum and weights of the sampled matrices.  Outputs of chunks that
    # share one workspace region are overwritten by later chunks, so O is recomputed one
    # chunk at a time: the sampled matrices' inputs are restored and the chunk is stepped
    # again eagerly, which must reproduce the graph's weights bitwise (the result of a
    # matrix does not depend on the other matrices of its batch).
    W_graph = {}
    for i in sample:
        W0, M0, G0 = snap[i]
        M_ref, _ = orc.momentum_update(M0, G0, w.beta)
        assert np.array_equal(_host(params[i].momentum).view(np.uint32), M_ref.view(np.uint32))
        W_graph[i] = params[i].weight.clone()
    by_chunk = {}
    for i in sample:
        by_chunk.setdefault(plan.param_info(i).chunk, []).append(i)
    worst = 0.0
    for ch, idx in sorted(by_chunk.items()):
        for i in idx:
            W0, M0, _ = snap[i]
            params[i].weight.copy_(torch.from_numpy(W0))
            params[i].momentum.copy_(torch.from_numpy(M0))
        plan.step(w.beta, w.lr, w.wd, w.a, w.b, w.c, w.steps, w.eps, chunk=ch)
        torch.cuda.synchronize()
        worst = max(worst, _check(plan, params, snap, w, idx))
        for i in idx:
            assert torch.equal(params[i].weight, W_graph[i]), f"graph and eager step differ: {w.params[i].name}"
    print(f"moe_slice: {len(sample)} sampled matrices, worst NS rel err {worst:.2e}")
    plan.close()


@pytest.mark.timeout(900)
def test_moe_slice_full_size_two_stream_graph():
    """The benchmark's configuration of the 261 GB slice: a two-stream plan (edge chunks,
    router and gate buckets last) under an 8 GiB cap, so tiled chunks alternate between
    two workspace regions; the pipelined step captured as one graph and replayed once.
    Sampled matrices are then re-stepped chunk by chunk on one stream, which must give the
    graph's weights bitwise, and checked against the oracle."""
    from muon_newton_schulz_momentum_amd import binding as L, harness

    def pick(w):
        names = [p.name for p in w.params]
        lo, hi = _scale_extremes(w)
        want = ["l0.q", "l2.shared.down", "l1.k", "l3.k", "l3.router", "l1.head_gate", "l2.shared_gate",
                "l0.e0.up", "l3.e511.gate"]
        return sorted({names.index(n) for n in want} | {lo, hi})
    cap = 8 * GiB
    w, params, sample, snap = _setup("moe_slice", pick, reserve=cap + 2 * GiB)
    plan = harness.Plan(params, max_workspace_bytes=cap, flags=L.MUON_PLAN_PIPELINE)
    infos = [plan.chunk_info(c) for c in range(plan.n_chunks)]
    tiled = [c for c, i in enumerate(infos) if not i.fused_small]
    assert all(infos[c].shared_region for c in tiled)
    # the 256-tile chunks alternate between two regions; the small tiled chunks (router,
    # gates, global-layer KV) are grouped, back to back in the region after the last one
    big = [c for c in tiled if not infos[c].grouped_small]
    group = [c for c in tiled if infos[c].grouped_small]
    offs = [infos[c].region_offset for c in big]
    assert len(set(offs)) == 2 and all(offs[j] != offs[j - 1] for j in range(1, len(offs)))
    assert len(group) == 4 and group == tiled[len(big):]
    assert infos[group[0]].region_offset in set(offs) and infos[group[0]].region_offset != offs[-1]
    for a, b in zip(group, group[1:]):
        assert infos[b].region_offset >= infos[a].region_offset + infos[a].region_bytes
    assert [infos[c].tile for c in tiled] == sorted((infos[c].tile for c in tiled), key=lambda t: t != 256)
    print(f"[moe_slice two-stream] {plan.n_chunks} chunks in {plan.workspace_bytes / GiB:.2f} GiB", flush=True)
    g = plan.capture_ex(w.beta, w.lr, w.wd, pipeline=True, a=w.a, b=w.b, c=w.c, steps=w.steps, eps=w.eps)
    g.launch()
    torch.cuda.synchronize()
    g.close()
    W_graph = {}
    for i in sample:
        _, M0, G0 = snap[i]
        M_ref, _ = orc.momentum_update(M0, G0, w.beta)
        assert np.array_equal(_host(params[i].momentum).view(np.uint32), M_ref.view(np.uint32))
        W_graph[i] = params[i].weight.clone()
    by_chunk = {}
    for i in sample:
        by_chunk.setdefault(plan.param_info(i).chunk, []).append(i)
    worst = 0.0
    for ch, idx in sorted(by_chunk.items()):
        for i in idx:
            W0, M0, _ = snap[i]
            params[i].weight.copy_(torch.from_numpy(W0))
            params[i].momentum.copy_(torch.from_numpy(M0))
        plan.step(w.beta, w.lr, w.wd, w.a, w.b, w.c, w.steps, w.eps, chunk=ch)
        torch.cuda.synchronize()
        worst = max(worst, _check(plan, params, snap, w, idx))
        for i in idx:
            assert torch.equal(params[i].weight, W_graph[i]), f"graph and eager step differ: {w.params[i].name}"
    print(f"moe_slice two-stream: {len(sample)} sampled matrices in {len(by_chunk)} chunks, worst NS rel err {worst:.2e}")
    plan.close()


@pytest.mark.timeout(900)
def test_moe_bucket_full_size_two_stream():
    """The MoE bucket in its benchmark configuration: a two-stream plan (experts split into
    chunks with edge chunks, the router last), one pipelined eager step and one graph
    replay from the same state, bitwise equal; sampled matrices from the first, a middle
    and the last expert chunk and the router against the oracle."""
    from muon_newton_schulz_momentum_amd import binding as L, harness

    def pick(w):
        lo, hi = _scale_extremes(w)
        return sorted({0, 1, 2, lo, hi, len(w.params) // 2, len(w.params) - 2, len(w.params) - 1})
    w, params, sample, snap = _setup("moe_bucket", pick, reserve=45 * GiB)
    plan = harness.Plan(params, flags=L.MUON_PLAN_PIPELINE)
    infos = [plan.chunk_info(c) for c in range(plan.n_chunks)]
    assert plan.n_chunks >= 8 and infos[-1].m == 512 and all(i.m == 1024 for i in infos[:-1])
    print(f"[moe_bucket two-stream] {plan.n_chunks} chunks: {[i.count for i in infos]}", flush=True)
    w0 = [p.weight.clone() for p in params]
    m0 = [p.momentum.clone() for p in params]
    kw = dict(a=w.a, b=w.b, c=w.c, steps=w.steps, eps=w.eps)
    plan.step_ex(w.beta, w.lr, w.wd, pipeline=True, **kw)
    torch.cuda.synchronize()
    worst = _check(plan, params, snap, w, sample)
    eager = {i: (params[i].weight.clone(), params[i].momentum.clone()) for i in sample}
    g = plan.capture_ex(w.beta, w.lr, w.wd, pipeline=True, **kw)
    for p, a, b in zip(params, w0, m0):
        p.weight.copy_(a)
        p.momentum.copy_(b)
    del w0, m0
    torch.cuda.synchronize()
    g.launch()
    torch.cuda.synchronize()
    g.close()
    for i in sample:
        assert torch.equal(params[i].weight, eager[i][0]) and torch.equal(params[i].momentum, eager[i][1]), i
    print(f"moe_bucket two-stream: {len(sample)} sampled matrices, worst NS rel err {worst:.2e}")
    plan.close()
