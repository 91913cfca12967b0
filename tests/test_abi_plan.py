"""CPU tests of the C ABI: the library loads, exports what include/muon.h declares, and
the host planner (no device calls) buckets, chunks and validates as documented.

Device pointers here are fake, aligned addresses: the planner only records them.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

from muon_newton_schulz_momentum_amd import binding as L
from muon_newton_schulz_momentum_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon.h")


def test_exports_every_declared_symbol():
    decl = set(re.findall(r"MUON_API[^;(]*?\b(muon_\w+)\s*\(", open(HEADER).read()))
    assert len(decl) >= 15
    lib = C.CDLL(L.LIB_PATH)
    for name in sorted(decl):
        assert hasattr(lib, name), name
    assert decl == set(L.EXPORTED)


class FakeMem:
    """Hands out disjoint, 256-byte aligned fake device addresses."""

    def __init__(self):
        self.next = 1 << 40

    def take(self, nbytes):
        p = self.next
        self.next += (nbytes + 255) // 256 * 256 + 256
        return p


def _descs(shapes, gdtype=L.MUON_DTYPE_F32, mem=None):
    mem = mem or FakeMem()
    arr = (L.muon_param_desc * len(shapes))()
    for i, shp in enumerate(shapes):
        d = arr[i]
        d.ndim = len(shp)
        if len(shp) == 2:
            r, c = shp
            d.rows, d.cols = r, c
            d.grad_dtype = gdtype
            d.weight = mem.take(r * c * 4)
            d.momentum = mem.take(r * c * 4)
            d.grad = mem.take(r * c * (4 if gdtype == L.MUON_DTYPE_F32 else 2))
    return arr


def _plan(arr, n=None, cap=0, scales=None, flags=0):
    opts = L.muon_plan_opts()
    opts.max_workspace_bytes = cap
    opts.flags = flags
    keep = None
    if scales is not None:
        keep = (C.c_float * len(scales))(*scales)
        opts.scale = keep
    p = C.c_void_p()
    st = L.muon_plan_buckets(arr, len(arr) if n is None else n, C.byref(opts), C.byref(p))
    return st, p


def _infos(p):
    nc = C.c_int32()
    L.check(L.muon_plan_counts(p, C.byref(nc), None, None, None), "counts")
    out = []
    for c in range(nc.value):
        info = L.muon_chunk_info()
        L.check(L.muon_plan_info(p, c, C.byref(info)), "info")
        out.append({f: getattr(info, f) for f, _ in L.muon_chunk_info._fields_})
    return out


def _pinfo(p, i):
    info = L.muon_param_info()
    L.check(L.muon_plan_param_info(p, i, C.byref(info)), "param_info")
    return info


@pytest.mark.parametrize("key", ["tiny", "ladder24", "moe_bucket", "full_width", "moe_slice"])
def test_buckets_of_every_workload(key):
    w = wl.get(key)
    shapes = [p.shape for p in w.params]
    gd = L.MUON_DTYPE_BF16 if any(p.grad_dtype == "bf16" for p in w.params) else L.MUON_DTYPE_F32
    arr = _descs(shapes, gd)
    st, p = _plan(arr)
    assert st == L.MUON_OK, L.muon_last_error()
    try:
        nc, nb, ninc, nex = C.c_int32(), C.c_int32(), C.c_int64(), C.c_int64()
        L.muon_plan_counts(p, C.byref(nc), C.byref(nb), C.byref(ninc), C.byref(nex))
        want = {}
        for s in shapes:
            if len(s) == 2:
                k = tuple(sorted(s))
                want[k] = want.get(k, 0) + 1
        assert nb.value == len(want) and nc.value == len(want)   # no cap: one chunk per bucket
        assert ninc.value == sum(want.values())
        assert nex.value == sum(1 for s in shapes if len(s) != 2)
        got = {(i["m"], i["n"]): i["count"] for i in _infos(p)}
        assert got == want
        for i in _infos(p):
            assert i["m_pad"] % i["tile"] == 0 and i["n_pad"] % i["tile"] == 0
            assert i["m_pad"] >= i["m"] and i["n_pad"] >= i["n"] and i["shared_region"] == 0
        # every 2-D parameter sits in exactly one (chunk, slot), transposed iff rows > cols
        seen = set()
        for idx, s in enumerate(shapes):
            pi = _pinfo(p, idx)
            if len(s) != 2:
                assert pi.included == 0
                continue
            assert pi.included == 1 and pi.transposed == int(s[0] > s[1])
            assert (pi.chunk, pi.slot) not in seen
            seen.add((pi.chunk, pi.slot))
            ci = _infos(p)[pi.chunk]
            assert (ci["m"], ci["n"]) == tuple(sorted(s)) and 0 <= pi.slot < ci["count"]
            assert pi.ld == ci["n_pad"] and pi.output_offset % 256 == 0
    finally:
        L.muon_plan_destroy(p)


def test_flops_match_workload_accounting():
    w = wl.get("ladder24")
    arr = _descs([p.shape for p in w.params])
    st, p = _plan(arr)
    assert st == 0
    conv = sum(i["flops_conventional"] for i in _infos(p)) * w.steps
    alg = sum(i["flops_algorithmic"] for i in _infos(p)) * w.steps
    L.muon_plan_destroy(p)
    c2, a2 = w.ns_flops()
    assert abs(conv - c2) / c2 < 1e-12 and abs(alg - a2) / a2 < 1e-12


def test_workspace_size_formula():
    shapes = [(64, 128)] * 3 + [(300, 70)] * 2
    st, p = _plan(_descs(shapes))
    assert st == 0
    nb = C.c_uint64()
    L.muon_plan_workspace_bytes(p, C.byref(nb))
    table = (5 * 64 + 255) // 256 * 256
    total = table
    for i in _infos(p):
        m, n, mp, np_, k = i["m"], i["n"], i["m_pad"], i["n_pad"], i["count"]
        ew = -(-m // 64) * -(-n // 64)
        al = lambda v: (v + 255) // 256 * 256  # noqa: E731
        region = 2 * al(k * mp * np_ * 2) + 2 * al(k * mp * mp * 2) + al(k * ew * 8) + al(k * 8) + 256  # + tile counters
        assert i["region_bytes"] == region and i["region_offset"] == total
        total += region
    assert nb.value == total
    L.muon_plan_destroy(p)


def test_chunking_under_a_cap():
    shapes = [(1024, 4096)] * 40 + [(4096, 1024)] * 20 + [(512, 4096)]
    st, p = _plan(_descs(shapes))
    full = C.c_uint64()
    L.muon_plan_workspace_bytes(p, C.byref(full))
    L.muon_plan_destroy(p)
    cap = full.value // 5
    st, p = _plan(_descs(shapes), cap=cap)
    assert st == 0, L.muon_last_error()
    nb = C.c_uint64()
    L.muon_plan_workspace_bytes(p, C.byref(nb))
    assert nb.value <= cap
    infos = _infos(p)
    assert len(infos) > 2 and all(i["shared_region"] == 1 for i in infos)
    big = [i for i in infos if i["m"] == 1024]
    assert sum(i["count"] for i in big) == 60
    assert max(i["count"] for i in big) - min(i["count"] for i in big) <= 1
    slots = {(_pinfo(p, k).chunk, _pinfo(p, k).slot) for k in range(len(shapes))}
    assert len(slots) == len(shapes)
    # chunk = -1 is refused for shared regions (checked before any device call)
    assert L.muon_momentum_update(p, -1, 0.9, None) == L.MUON_ERR_NOT_BOUND  # not bound yet
    L.muon_plan_destroy(p)
    # a cap below one matrix fails cleanly
    st, p = _plan(_descs(shapes), cap=1 << 20)
    assert st == L.MUON_ERR_WORKSPACE_TOO_SMALL and not p.value


def test_validation_errors():
    mem = FakeMem()
    arr = _descs([(8, 8)], mem=mem)
    arr[0].rows = 0
    assert _plan(arr)[0] == L.MUON_ERR_SHAPE
    arr = _descs([(8, 8)], mem=mem)
    arr[0].weight = arr[0].weight + 4
    assert _plan(arr)[0] == L.MUON_ERR_ALIGNMENT
    arr = _descs([(8, 8)], mem=mem)
    arr[0].momentum = arr[0].weight
    assert _plan(arr)[0] == L.MUON_ERR_INVALID_ARG
    arr = _descs([(8, 8), (8, 8)], mem=mem)
    arr[1].weight = arr[0].momentum + 64        # overlaps parameter 0's momentum
    assert _plan(arr)[0] == L.MUON_ERR_INVALID_ARG
    arr = _descs([(8, 8), (8, 8)], mem=mem)
    arr[1].grad = arr[0].grad                   # shared read-only gradients are allowed
    assert _plan(arr)[0] == L.MUON_OK
    arr = _descs([(8, 8)], mem=mem)
    arr[0].grad_dtype = 7
    assert _plan(arr)[0] == L.MUON_ERR_INVALID_ARG
    arr = _descs([(8, 8)], mem=mem)
    arr[0].grad = None
    assert _plan(arr)[0] == L.MUON_ERR_INVALID_ARG
    p = C.c_void_p()
    assert L.muon_plan_buckets(None, 3, None, C.byref(p)) == L.MUON_ERR_INVALID_ARG
    assert L.muon_plan_buckets(None, 0, None, None) == L.MUON_ERR_INVALID_ARG
    assert b"out" in L.muon_last_error()
    arr = _descs([(8, 8)], mem=mem)
    assert _plan(arr, scales=[float("nan")])[0] == L.MUON_ERR_INVALID_ARG
    # a non-2-D parameter is excluded, not an error, and its pointers are not looked at
    arr = _descs([(8,), (8, 8)], mem=mem)
    st, p = _plan(arr)
    assert st == 0
    L.muon_plan_destroy(p)


def test_empty_plan():
    st, p = _plan((L.muon_param_desc * 1)(), n=0)
    assert st == 0
    nb = C.c_uint64()
    L.muon_plan_workspace_bytes(p, C.byref(nb))
    assert nb.value > 0
    assert _infos(p) == []
    L.muon_plan_destroy(p)


def test_plan_is_deterministic_and_validates():
    shapes = [(64, 128), (128, 64), (7, 300), (300, 7), (5,), (2048, 2048)]
    mem = FakeMem()
    arr = _descs(shapes, mem=mem)
    st1, p1 = _plan(arr)
    st2, p2 = _plan(arr)
    assert st1 == st2 == 0
    assert _infos(p1) == _infos(p2)
    for i in range(len(shapes)):
        a, b = _pinfo(p1, i), _pinfo(p2, i)
        assert bytes(a) == bytes(b)
    assert L.muon_plan_validate(p1, arr, len(shapes)) == L.MUON_OK
    arr[2].cols = 301
    assert L.muon_plan_validate(p1, arr, len(shapes)) == L.MUON_ERR_STALE_PLAN
    assert L.muon_plan_validate(p1, arr, 3) == L.MUON_ERR_STALE_PLAN
    L.muon_plan_destroy(p1)
    L.muon_plan_destroy(p2)


def test_step_calls_refused_before_bind_and_bind_checks():
    st, p = _plan(_descs([(64, 128)]))
    assert st == 0
    assert L.muon_momentum_update(p, 0, 0.95, None) == L.MUON_ERR_NOT_BOUND
    assert L.muon_ns_batched(p, 0, 3.4445, -4.775, 2.0315, 5, 1e-7, None) == L.MUON_ERR_NOT_BOUND
    assert L.muon_apply(p, 0, 0.02, 0.1, None) == L.MUON_ERR_NOT_BOUND
    assert L.muon_step(p, -1, 0.95, 3.4, -4.7, 2.0, 5, 1e-7, 0.02, 0.1, None) == L.MUON_ERR_NOT_BOUND
    g = C.c_void_p(1)
    assert L.muon_graph_capture(p, 0.95, 3.4, -4.7, 2.0, 5, 1e-7, 0.02, 0.1, C.byref(g)) == L.MUON_ERR_NOT_BOUND
    assert not g.value    # *out is cleared on every error
    assert L.muon_graph_capture(p, 0.95, 3.4, -4.7, 2.0, 5, 1e-7, 0.02, 0.1, None) == L.MUON_ERR_INVALID_ARG
    assert L.muon_graph_capture(None, 0.95, 3.4, -4.7, 2.0, 5, 1e-7, 0.02, 0.1, C.byref(g)) \
        == L.MUON_ERR_INVALID_ARG
    assert L.muon_graph_launch(None, None) == L.MUON_ERR_INVALID_ARG
    L.muon_graph_destroy(None)
    assert L.muon_plan_bind(p, None, 1 << 30, None) == L.MUON_ERR_INVALID_ARG
    assert L.muon_plan_bind(p, 1 << 40 | 16, 1 << 30, None) == L.MUON_ERR_ALIGNMENT
    assert L.muon_plan_bind(p, 1 << 40, 16, None) == L.MUON_ERR_WORKSPACE_TOO_SMALL
    assert L.muon_plan_info(p, 5, C.byref(L.muon_chunk_info())) == L.MUON_ERR_INVALID_ARG
    assert L.muon_plan_param_info(p, -1, C.byref(L.muon_param_info())) == L.MUON_ERR_INVALID_ARG
    assert L.muon_kernel_name(L.MUON_KERNEL_GEMM_AXPY) == b"gemm_axpy"
    assert L.muon_status_string(L.MUON_ERR_STALE_PLAN) == b"stale plan"
    L.muon_plan_destroy(p)
    L.muon_plan_destroy(None)


def test_fused_small_path_is_chosen_by_shape_and_flag():
    # canonical m <= 64 (padded to one 64-row tile) and padded n <= 1024 take the fused
    # whole-iteration kernel; everything else the tiled kernels
    shapes = [(64, 128), (300, 17), (32, 1000), (64, 1088), (65, 128), (1, 4096), (1, 64)]
    want = {(64, 128): 1, (17, 300): 1, (32, 1000): 1, (64, 1088): 0, (65, 128): 0, (1, 4096): 0, (1, 64): 1}
    for flags, expect in ((0, want), (L.MUON_PLAN_TILED_SMALL, {k: 0 for k in want})):
        st, p = _plan(_descs(shapes), flags=flags)
        assert st == 0
        got = {(i["m"], i["n"]): i["fused_small"] for i in _infos(p)}
        assert got == expect
        L.muon_plan_destroy(p)
    assert L.muon_kernel_name(L.MUON_KERNEL_NS_SMALL) == b"ns_small"


def test_scale_modes_set_each_parameters_update_scale():
    from oracle import muon_oracle as orc
    shapes = [(4096, 1024), (1024, 4096), (2048, 2048), (5632, 2048), (300,)]
    for mode, rule in ((L.MUON_SCALE_NONE, "none"), (L.MUON_SCALE_ASPECT, "aspect"),
                       (L.MUON_SCALE_RMS_MATCH, "rms_match")):
        opts = L.muon_plan_opts()
        opts.scale_mode = mode
        p = C.c_void_p()
        assert L.muon_plan_buckets(_descs(shapes), len(shapes), C.byref(opts), C.byref(p)) == 0
        for i, shp in enumerate(shapes):
            info = L.muon_param_info()
            L.check(L.muon_plan_param_info(p, i, C.byref(info)), "param_info")
            if len(shp) == 2:
                assert info.scale == orc.update_scale(rule, *shp), (rule, shp)
        L.muon_plan_destroy(p)
    # an explicit scale array wins over the rule; an unknown rule is refused
    opts = L.muon_plan_opts()
    opts.scale_mode = L.MUON_SCALE_ASPECT
    keep = (C.c_float * 1)(0.5)
    opts.scale = keep
    p = C.c_void_p()
    assert L.muon_plan_buckets(_descs([(4096, 1024)]), 1, C.byref(opts), C.byref(p)) == 0
    info = L.muon_param_info()
    L.check(L.muon_plan_param_info(p, 0, C.byref(info)), "param_info")
    assert info.scale == 0.5
    L.muon_plan_destroy(p)
    opts = L.muon_plan_opts()
    opts.scale_mode = 7
    assert L.muon_plan_buckets(_descs([(64, 64)]), 1, C.byref(opts), C.byref(p)) == L.MUON_ERR_INVALID_ARG


def test_adamw_parameters_are_planned_by_role():
    mem = FakeMem()
    shapes = [(64, 128), (4096,), (32000, 64), (300,)]
    arr = (L.muon_param_desc * 4)()
    for i, shp in enumerate(shapes):
        d = arr[i]
        d.ndim = len(shp)
        numel = int(np.prod(shp))
        d.rows, d.cols = (shp if len(shp) == 2 else (numel, 1))
        d.grad_dtype = L.MUON_DTYPE_F32
        d.weight, d.momentum, d.grad = mem.take(numel * 4), mem.take(numel * 4), mem.take(numel * 4)
    arr[1].exp_avg_sq = mem.take(4096 * 4)                   # 1-D with a second moment: AdamW
    arr[2].exp_avg_sq = mem.take(32000 * 64 * 4)
    arr[2].optimizer = L.MUON_OPT_ADAMW                      # a 2-D embedding: AdamW
    # arr[3]: 1-D without a second moment: excluded
    st, p = _plan(arr)
    assert st == 0
    n_chunks, _, n_inc, n_exc = C.c_int32(), None, C.c_int64(), C.c_int64()
    L.check(L.muon_plan_counts(p, C.byref(n_chunks), None, C.byref(n_inc), C.byref(n_exc)), "counts")
    assert (n_chunks.value, n_inc.value, n_exc.value) == (1, 1, 1)
    na, ne = C.c_int64(), C.c_int64()
    L.check(L.muon_plan_adamw_counts(p, C.byref(na), C.byref(ne)), "adamw counts")
    assert (na.value, ne.value) == (2, 4096 + 32000 * 64)
    roles = []
    for i in range(4):
        info = L.muon_param_info()
        L.check(L.muon_plan_param_info(p, i, C.byref(info)), "param_info")
        roles.append(info.included)
    assert roles == [1, 2, 2, 0]
    assert L.muon_plan_validate(p, arr, 4) == 0
    arr[1].exp_avg_sq = mem.take(4096 * 4)
    assert L.muon_plan_validate(p, arr, 4) == L.MUON_ERR_STALE_PLAN
    L.muon_plan_destroy(p)
    # a second moment overlapping a weight is refused; so is an unknown optimizer
    arr[1].exp_avg_sq = arr[0].weight
    assert _plan(arr)[0] == L.MUON_ERR_INVALID_ARG
    arr[1].exp_avg_sq = mem.take(4096 * 4)
    arr[3].optimizer = 9
    assert _plan(arr)[0] == L.MUON_ERR_INVALID_ARG
    # AdamW refuses an unbound plan and bad settings before touching the device
    arr[3].optimizer = 0
    st, p = _plan(arr)
    k = L.muon_adamw_config()
    k.lr, k.beta1, k.beta2, k.eps, k.wd, k.step = 1e-3, 0.9, 0.95, 1e-8, 0.1, 1
    assert L.muon_adamw_step(p, C.byref(k), None) == L.MUON_ERR_NOT_BOUND
    L.muon_plan_destroy(p)


def _unsplit_edges(sizes, want):
    """The balanced split of `want` chunks that `sizes` came from (merging a head chunk
    into the next one and a tail chunk into the one before), or None."""
    for head in (0, 1):
        for tail in (0, 1):
            v = list(sizes)
            if head and len(v) > 1:
                v = [v[0] + v[1]] + v[2:]
            elif head:
                continue
            if tail and len(v) > 1:
                v = v[:-2] + [v[-2] + v[-1]]
            elif tail:
                continue
            if len(v) == want and max(v) - min(v) <= 1:
                return v
    return None


def test_pipeline_plans_split_large_buckets():
    # up to 8 chunks per bucket, each with at least 2048 SYRK workgroups (upper-triangle
    # tiles of 256 x 256: 10 for m = 1024, 36 for m = 2048, 595 for m = 8704), then at most
    # one edge chunk split off each end of the 256-tile buckets' run
    cases = [((1024, 4096), 1536, 7), ((2048, 2048), 96, 1), ((2048, 2048), 200, 3), ((8704, 8704), 4, 1),
             ((2048, 2048), 5000, 8), ((64, 512), 3000, 1)]
    for shape, count, want in cases:
        for flags in (0, L.MUON_PLAN_PIPELINE):
            st, p = _plan(_descs([shape] * count), flags=flags)
            assert st == 0, L.muon_last_error()
            infos = _infos(p)
            sizes = [i["count"] for i in infos]
            assert sum(sizes) == count
            if flags == 0:
                assert sizes == [count]
            else:
                assert _unsplit_edges(sizes, want) is not None, (shape, count, sizes)
                if min(shape) < 1024:
                    assert len(sizes) == want      # no edge chunks outside the 256-tile buckets
            assert all(i["shared_region"] == 0 for i in infos)
            L.muon_plan_destroy(p)


def test_pipeline_edge_chunks_of_the_layer_ladder():
    # 96 x (2048, 2048) and 72 x (2048, 5632): a smaller chunk off the front of the first
    # bucket and off the back of the last, sized so that no product launch gains a partial
    # wave of tiles on the 256 compute units; without the flag, one chunk per bucket
    w = wl.get("ladder24")
    shapes = [p.shape for p in w.params]
    st, p = _plan(_descs(shapes))
    assert [(i["m"], i["n"], i["count"]) for i in _infos(p)] == [(2048, 2048, 96), (2048, 5632, 72)]
    L.muon_plan_destroy(p)
    st, p = _plan(_descs(shapes), flags=L.MUON_PLAN_PIPELINE)
    infos = _infos(p)
    L.muon_plan_destroy(p)
    assert len(infos) == 4
    a, b, c, d = (i["count"] for i in infos)
    assert [(i["m"], i["n"]) for i in infos] == [(2048, 2048)] * 2 + [(2048, 5632)] * 2
    assert a + b == 96 and c + d == 72 and a < b and d < c
    waves = lambda x: -(-x // 256)
    for (n, total, parts) in ((2048, 96, (a, b)), (5632, 72, (c, d))):
        tri, full = 8 * 9 // 2, 8 * (n // 256)
        for per in (tri, full):
            assert sum(waves(per * k) for k in parts) == waves(per * total)


def test_pipeline_plans_put_smaller_tiles_last():
    # the 512-row router bucket (128 tiles) after the 256-tile expert chunks
    shapes = [(512, 4096)] + [(1024, 4096)] * 300
    st, p = _plan(_descs(shapes), flags=L.MUON_PLAN_PIPELINE)
    infos = _infos(p)
    L.muon_plan_destroy(p)
    assert infos[-1]["m"] == 512 and all(i["m"] == 1024 for i in infos[:-1])
    st, p = _plan(_descs(shapes))
    assert [i["m"] for i in _infos(p)] == [512, 1024]
    L.muon_plan_destroy(p)


def test_double_buffered_regions_under_a_cap():
    # tiled chunks alternate between two regions, each within half the remaining cap; the
    # fused small chunks stay in the first; without a binding cap (and buckets too small to
    # split) the flag adds at most the edge chunks, each in a region of its own
    shapes = [(1024, 4096)] * 40 + [(4096, 1024)] * 20 + [(64, 512)] * 5
    st, p = _plan(_descs(shapes))
    full = C.c_uint64()
    L.muon_plan_workspace_bytes(p, C.byref(full))
    plain = _infos(p)
    L.muon_plan_destroy(p)
    st, p = _plan(_descs(shapes), flags=L.MUON_PLAN_PIPELINE)
    piped = _infos(p)
    assert st == 0 and len(plain) <= len(piped) <= len(plain) + 2
    for key in ("m", "n"):
        assert sorted(set(i[key] for i in piped)) == sorted(set(i[key] for i in plain))
    assert sum(i["count"] for i in piped) == sum(i["count"] for i in plain)
    assert all(i["shared_region"] == 0 for i in piped)
    ends = sorted((i["region_offset"], i["region_offset"] + i["region_bytes"]) for i in piped)
    assert all(ends[j][1] <= ends[j + 1][0] for j in range(len(ends) - 1))
    L.muon_plan_destroy(p)
    cap = full.value // 5
    st, p = _plan(_descs(shapes), cap=cap, flags=L.MUON_PLAN_PIPELINE)
    assert st == 0, L.muon_last_error()
    nb = C.c_uint64()
    L.muon_plan_workspace_bytes(p, C.byref(nb))
    assert nb.value <= cap
    infos = _infos(p)
    tiled = [i for i in infos if not i["fused_small"]]
    offs = [i["region_offset"] for i in tiled]
    assert len(set(offs)) == 2 and all(offs[j] != offs[j - 1] for j in range(1, len(offs)))
    lo, hi = sorted(set(offs))
    assert all(i["region_offset"] == lo for i in infos if i["fused_small"])
    # regions never overlap and end within the workspace
    for i in infos:
        end = i["region_offset"] + i["region_bytes"]
        assert end <= nb.value
        if i["region_offset"] == lo:
            assert end <= hi
    # about half the matrices per chunk of the single-region plan under the same cap
    st1, p1 = _plan(_descs(shapes), cap=cap)
    single = max(i["count"] for i in _infos(p1) if i["m"] == 1024)
    double = max(i["count"] for i in tiled if i["m"] == 1024)
    assert double <= (single + 1) // 2 + 1
    L.muon_plan_destroy(p1)
    L.muon_plan_destroy(p)
    # too small for two matrices of the largest bucket
    st, p = _plan(_descs([(4096, 4096)] * 2), cap=3 * 4096 * 4096 * 2 * 2,
                  flags=L.MUON_PLAN_PIPELINE)
    assert st == L.MUON_ERR_WORKSPACE_TOO_SMALL and b"double buffering" in L.muon_last_error()


def test_unknown_plan_flags_are_refused():
    st, p = _plan(_descs([(128, 256)]), flags=1 << 7)
    assert st == L.MUON_ERR_INVALID_ARG and not p.value
    assert b"flag" in L.muon_last_error()


def test_pipeline_plans_of_random_bucket_mixes_are_well_formed():
    # Many seeded shape mixes, with and without a workspace cap: every matrix lands in
    # exactly one chunk, no chunk is empty, chunks of one bucket are contiguous and
    # together hold the bucket, the 256-tile buckets come before the others, tiled chunks
    # under a cap alternate between two regions, and the workspace stays within the cap.
    rng = np.random.default_rng(20261202)
    dims = [64, 96, 200, 512, 1024, 1100, 2048, 3000, 4096]
    for trial in range(40):
        nb = int(rng.integers(1, 5))
        shapes = []
        for _ in range(nb):
            r, c = (int(x) for x in rng.choice(dims, 2))
            shapes += [(r, c)] * int(rng.integers(1, 120))
        rng.shuffle(shapes)
        st, p = _plan(_descs(shapes), flags=L.MUON_PLAN_PIPELINE)
        assert st == 0, (trial, L.muon_last_error())
        full = C.c_uint64()
        L.muon_plan_workspace_bytes(p, C.byref(full))
        L.muon_plan_destroy(p)
        for cap in (0, full.value // 3):
            st, p = _plan(_descs(shapes), cap=cap, flags=L.MUON_PLAN_PIPELINE)
            if st == L.MUON_ERR_WORKSPACE_TOO_SMALL:
                continue
            assert st == 0, (trial, cap, L.muon_last_error())
            infos = _infos(p)
            assert all(i["count"] >= 1 for i in infos)
            assert sum(i["count"] for i in infos) == len(shapes)
            seen, order = set(), []
            for i in infos:
                if not order or order[-1] != i["bucket"]:
                    assert i["bucket"] not in seen, "chunks of one bucket are contiguous"
                    order.append(i["bucket"])
                    seen.add(i["bucket"])
            want = {}
            for r, c in shapes:
                key = (min(r, c), max(r, c))
                want[key] = want.get(key, 0) + 1
            got = {}
            for i in infos:
                got[(i["m"], i["n"])] = got.get((i["m"], i["n"]), 0) + i["count"]
            assert got == want
            tiles = [i["tile"] for i in infos if not i["fused_small"]]
            assert tiles == sorted(tiles, key=lambda t: t != 256), "256-tile buckets first"
            for k in range(len(shapes)):
                pi = _pinfo(p, k)
                assert pi.included == 1 and 0 <= pi.slot < infos[pi.chunk]["count"]
            nbytes = C.c_uint64()
            L.muon_plan_workspace_bytes(p, C.byref(nbytes))
            if cap:
                assert nbytes.value <= cap
                tiled = [i for i in infos if not i["fused_small"]]
                if tiled and tiled[0]["shared_region"]:
                    offs = [i["region_offset"] for i in tiled]
                    assert all(offs[j] != offs[j - 1] for j in range(1, len(offs)))
            for i in infos:
                assert i["region_offset"] + i["region_bytes"] <= nbytes.value
            L.muon_plan_destroy(p)


def test_grouped_small_chunks_layout():
    """Small tiled chunks (128/64-row tiles, not fused) are marked for the grouped launches;
    under a cap they sit back to back in one region (the two-stream plan: the region after
    the last 256-tile chunk's), and when they do not fit in one region each runs alone."""
    shapes = [(1024, 2048)] * 8 + [(512, 4096)] * 2 + [(256, 4096), (32, 4096), (4096, 1), (64, 128), (300, 700)]
    st, p = _plan(_descs(shapes))
    assert st == 0
    infos = _infos(p)
    grouped = {(i["m"], i["n"]) for i in infos if i["grouped_small"]}
    assert grouped == {(512, 4096), (256, 4096), (32, 4096), (1, 4096), (300, 700)}
    assert all(not i["grouped_small"] for i in infos if i["tile"] == 256 or i["fused_small"])
    L.muon_plan_destroy(p)
    st, p = _plan(_descs(shapes), flags=L.MUON_PLAN_UNGROUPED)
    assert st == 0 and not any(i["grouped_small"] for i in _infos(p))
    full = C.c_uint64()
    L.muon_plan_workspace_bytes(p, C.byref(full))
    L.muon_plan_destroy(p)
    for flags in (0, L.MUON_PLAN_PIPELINE):
        cap = full.value // 2
        st, p = _plan(_descs(shapes), cap=cap, flags=flags)
        assert st == 0, L.muon_last_error()
        nb = C.c_uint64()
        L.muon_plan_workspace_bytes(p, C.byref(nb))
        infos = _infos(p)
        group = [i for i in infos if i["grouped_small"]]
        assert len(group) == 5 and all(i["shared_region"] for i in infos)
        for a, b in zip(group, group[1:]):
            assert b["region_offset"] == a["region_offset"] + a["region_bytes"]
        g_lo, g_hi = group[0]["region_offset"], group[-1]["region_offset"] + group[-1]["region_bytes"]
        assert g_hi <= nb.value
        big = [i for i in infos if i["tile"] == 256]
        starts = sorted({i["region_offset"] for i in big})
        assert g_lo in starts
        if flags:
            assert g_lo != big[-1]["region_offset"]      # the group follows the last big chunk
        L.muon_plan_destroy(p)
    # a group too large for one region under the cap: every small chunk on its own
    many = [(1024, 1024)] * 2 + [(512, 4096)] * 40 + [(256, 4096)] * 2
    st, p = _plan(_descs(many), flags=L.MUON_PLAN_UNGROUPED)
    L.muon_plan_workspace_bytes(p, C.byref(full))
    L.muon_plan_destroy(p)
    st, p = _plan(_descs(many), cap=full.value // 3)
    assert st == 0, L.muon_last_error()
    assert not any(i["grouped_small"] for i in _infos(p))
    L.muon_plan_destroy(p)
