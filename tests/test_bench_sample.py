"""The benchmark's CPU-oracle sample (host logic, no GPU).

For the MoE workloads the giant expert bucket gets 16 matrices including its first, its
last and the experts with the smallest and the largest gradient scale; every other bucket
that the oracle can run within the budget gets all of its matrices up to 16; buckets whose
single matrix exceeds the budget are left out; the estimated oracle time of the sample stays
within the budget.
"""
import bench
from muon_newton_schulz_momentum_amd import workloads as wl


def _check(key):
    w = wl.get(key)
    pick, buckets = bench.oracle_sample(w)

    def cost(k):
        m, n = k
        return w.steps * (4.0 * m * m * n + 2.0 * m ** 3) / bench.ORACLE_RATE

    total = sum(cost(k) * len(v) for k, v in pick.items())
    assert total <= bench.ORACLE_BUDGET_S * 1.5, total
    for k, idx in buckets.items():
        if cost(k) > bench.ORACLE_BUDGET_S:
            assert k not in pick, k
            continue
        sel = pick[k]
        assert set(sel) <= set(idx) and len(sel) == len(set(sel))
        assert idx[0] in sel
        if len(idx) > bench.ORACLE_MAX_PER_BUCKET:
            assert idx[-1] in sel
            grouped = [i for i in idx if w.params[i].group >= 0]
            if w.scale_groups and grouped:
                sc = {i: wl.group_scale(w.cid, w.params[i].group) for i in grouped}
                assert min(grouped, key=lambda i: sc[i]) in sel
                assert max(grouped, key=lambda i: sc[i]) in sel
    return w, pick, buckets


def test_moe_slice_sample():
    w, pick, buckets = _check("moe_slice")
    giant = max(buckets, key=lambda k: len(buckets[k]))
    assert giant == (1024, 4096) and len(pick[giant]) == bench.ORACLE_MAX_PER_BUCKET
    small = [k for k in buckets if len(buckets[k]) <= bench.ORACLE_MAX_PER_BUCKET and k[0] <= 512]
    assert small and all(len(pick[k]) == len(buckets[k]) for k in small)


def test_moe_bucket_and_full_width_samples():
    _, pick, buckets = _check("moe_bucket")
    assert len(pick[(1024, 4096)]) == bench.ORACLE_MAX_PER_BUCKET and len(pick[(512, 4096)]) == 1
    _, pick, buckets = _check("full_width")
    assert (8704, 8704) not in pick
