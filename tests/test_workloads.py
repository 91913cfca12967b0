"""Workload helpers pinned to constants the pages print (tests/golden/pages_constants.txt)."""
import math
import os

import numpy as np
import pytest

from muon_newton_schulz_momentum_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_constants.txt")


def _golden():
    out = {}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = (t.strip() for t in line.split("="))
            out[k] = float(v)
    return out


def test_ladder_rule_reproduces_printed_architecture():
    g = _golden()
    L = int(g["layers"])
    assert wl.ladder_hidden(L) == int(g["d_model"])
    assert wl.ladder_query_heads(L) == int(g["query_heads"])
    assert wl.ladder_hidden(24) == 2048


@pytest.mark.parametrize("steps", [1e4, 1e5, 3e5])
@pytest.mark.parametrize("base", [math.e, 10.0])
def test_lr_wd_laws_match_printed_constants(steps, base):
    g = _golden()
    tpp = g["train_tokens"] / g["active_params"]
    lr, wd = wl.lr_wd_from_laws(steps, tpp, base=base)
    assert abs(lr * wd * steps - g["lrwd_numerator"]) < 1e-9
    lg = lambda v: math.log(v, base)  # noqa: E731
    want = g["loglr_intercept"] + g["loglr_tpp_coef"] * lg(tpp) + g["loglr_steps_coef"] * lg(steps)
    assert abs(lg(lr) - want) < 1e-12


def test_lr_wd_natural_log_reading_at_1e5_steps():
    lr, wd = wl.lr_wd_from_laws(1e5, 625.0)
    assert abs(lr - 9.30e-4) < 1e-6 and abs(wd - 0.1832) < 1e-3
    assert wl.get("moe_slice").lr == lr


def test_workload_shapes_and_buckets():
    def buckets(w):
        out = {}
        for p in w.params:
            if p.is_matrix:
                k = tuple(sorted(p.shape))
                out[k] = out.get(k, 0) + 1
        return out
    assert buckets(wl.get("tiny")) == {(64, 128): 8}
    assert buckets(wl.get("ladder24")) == {(2048, 2048): 96, (2048, 5632): 72}
    assert buckets(wl.get("moe_bucket")) == {(1024, 4096): 1536, (512, 4096): 1}
    assert buckets(wl.get("full_width")) == {(8704, 8704): 4, (3072, 8704): 3,
                                             (1024, 8704): 21, (512, 8704): 1}
    b5 = buckets(wl.get("moe_slice"))
    assert b5 == {(4096, 4096): 8, (3072, 4096): 12, (2048, 4096): 6, (1024, 4096): 6144,
                  (512, 4096): 4, (256, 4096): 2, (32, 4096): 4, (1, 4096): 4}
    assert sum(b5.values()) == 6184
    assert sum(1 for p in wl.get("moe_slice").params if not p.is_matrix) == 8


def test_generator_is_seeded_and_per_matrix():
    import torch
    w = wl.get("tiny")
    a = wl.generate(w, 3)
    b = wl.generate(w, 3)
    c = wl.generate(w, 4)
    for r in "WMG":
        assert torch.equal(a[r], b[r])
        assert a[r].dtype == torch.float32 and tuple(a[r].shape) == (64, 128)
        assert not torch.equal(a[r], c[r])
    assert abs(float(a["W"].std()) - 0.02) < 0.002
    assert len({wl.seed_of(1, i, r) for i in range(50) for r in range(3)}) == 150


def test_expert_scales_log_uniform_and_shared():
    w = wl.get("moe_bucket")
    s = np.array([wl.group_scale(w.cid, e) for e in range(512)])
    assert s.min() >= 0.1 and s.max() <= 10.0
    assert abs(np.log(s).mean()) < 0.3
    g0 = wl.generate(w, 0, roles=("G",))["G"]
    assert abs(float(g0.std()) / 1e-3 - s[0]) / s[0] < 0.05


def test_conventional_and_algorithmic_flops():
    conv, alg = wl.get("ladder24").ns_flops()
    assert abs(conv - 6.494e13) / 6.494e13 < 1e-3
    assert abs(alg - 4.511e13) / 4.511e13 < 1e-3
