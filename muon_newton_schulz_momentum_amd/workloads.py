"""Synthetic workloads and their seeded input generators.

This module holds shapes, hyper-parameters and seeded random draws only — none of the
Muon step's arithmetic.  Both the HIP path (through the harness) and the CPU oracle take
their inputs from here; nothing else is shared between them.

Every parameter i of workload c draws its weight, initial momentum and gradient from a
torch generator of its own, seeded from (SEED, c, i, role), so any single matrix can be
drawn again on its own.  Per-expert gradient scales come from numpy's
Generator(PCG64([SEED, c, expert, 3])).

Shapes follow the pages' architecture where they give it:
  * ladder rule: hidden = (256/3)*L and query heads = L rounded to the nearest multiple
    of 16 ("Frontier Pre-training at Microsoft AI", method details section 1);
  * 102 layers, d_model 8704, 512 experts, 1 shared + top-7 routed, 96 query heads with
    16 KV heads on local and 2 on global attention layers (same page, setup section 2);
  * Muon covers the 2-D non-embedding matrices only; 1-D parameters go elsewhere (same
    page, setup section 4).
The routed-expert inner dimension 1024 and the d=4096 slice are synthetic stand-ins for
the private MAI-Base-2 training run; no dataset or trained weight is involved.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

SEED = 20261202
ROLE_W, ROLE_M, ROLE_G, ROLE_SCALE = 0, 1, 2, 3

# The quintic coefficients and step count most commonly used with Muon; the pages give
# none, so they are call parameters with these defaults.
NS_A, NS_B, NS_C = 3.4445, -4.7750, 2.0315
NS_STEPS = 5
NS_EPS = 1e-7


def ladder_hidden(layers: int) -> int:
    """Hidden size of a ladder rung: (256/3) * L (notes page, method section 1)."""
    return int(round(256 * layers / 3))


def ladder_query_heads(layers: int) -> int:
    """Query heads of a ladder rung: L rounded to the nearest multiple of 16.

    A tie (L an odd multiple of 8) has no stated rule; it rounds up here.
    """
    return int(16 * math.floor(layers / 16 + 0.5))


def lr_wd_from_laws(steps: float, tpp: float, base: float = math.e) -> Tuple[float, float]:
    """Learning rate and weight decay from the pages' fitted laws.

    LR* x WD* = 17.04 / steps and log LR* = -1.51 + 0.175 log TPP - 0.573 log steps
    (recipe page, section "Small Models Must Also Undergo the 'Repeated Learning' of
    Large Models"; the same laws on its Japanese translation).  The log base is not
    stated; the natural log is the default reading, base=10 the alternative.
    """
    lg = lambda v: math.log(v) / math.log(base)  # noqa: E731
    lr = base ** (-1.51 + 0.175 * lg(tpp) - 0.573 * lg(steps))
    wd = (17.04 / steps) / lr
    return lr, wd


@dataclass(frozen=True)
class ParamSpec:
    name: str
    shape: Tuple[int, ...]
    w_std: float
    g_std: float
    m_std: float
    grad_dtype: str = "f32"          # "f32" or "bf16"
    group: int = -1                  # expert id whose scale multiplies the gradient

    @property
    def is_matrix(self) -> bool:
        return len(self.shape) == 2


@dataclass
class Workload:
    key: str
    cid: int
    description: str
    params: List[ParamSpec]
    beta: float = 0.95
    lr: float = 0.02
    wd: float = 0.1
    a: float = NS_A
    b: float = NS_B
    c: float = NS_C
    steps: int = NS_STEPS
    eps: float = NS_EPS
    scale_groups: bool = False
    notes: dict = field(default_factory=dict)

    @property
    def matrices(self) -> List[int]:
        return [i for i, p in enumerate(self.params) if p.is_matrix]

    def elements(self) -> int:
        return sum(int(np.prod(p.shape)) for p in self.params)

    def ns_flops(self) -> Tuple[float, float]:
        """(conventional, algorithmic) NS FLOPs of one step over every 2-D parameter.

        Per iteration on canonical (m, n): conventional 4 m^2 n + 2 m^3 (X X^T, A A and
        B X as plain GEMMs); algorithmic m(m+1)n + m^2(m+1) + 2 m^2 n (the two symmetric
        products computed on one triangle).
        """
        conv = alg = 0.0
        for p in self.params:
            if not p.is_matrix:
                continue
            m, n = sorted(p.shape)
            conv += 4.0 * m * m * n + 2.0 * m ** 3
            alg += m * (m + 1.0) * n + m * m * (m + 1.0) + 2.0 * m * m * n
        return conv * self.steps, alg * self.steps


def _tiny() -> Workload:
    ps = [ParamSpec(f"w{i}", (64, 128), 0.02, 0.02, 0.02) for i in range(8)]
    return Workload("tiny", 1, "8 fp32 matrices 64x128, W/M/G ~ N(0, 0.02)", ps)


def _ladder24() -> Workload:
    L = 24
    d = ladder_hidden(L)           # 2048
    ffn = 5632
    ps = []
    for layer in range(L):
        for nm in ("q", "k", "v", "o"):
            ps.append(ParamSpec(f"l{layer}.{nm}", (d, d), 0.02, 1e-3, 1e-3))
        ps.append(ParamSpec(f"l{layer}.gate", (ffn, d), 0.02, 1e-3, 1e-3))
        ps.append(ParamSpec(f"l{layer}.up", (ffn, d), 0.02, 1e-3, 1e-3))
        ps.append(ParamSpec(f"l{layer}.down", (d, ffn), 0.02, 1e-3, 1e-3))
    return Workload("ladder24", 2, "ladder rung L=24 (d=2048): 24 x (4 x 2048^2, "
                    "2 x 5632x2048, 2048x5632) = 168 matrices", ps)


def _moe_bucket() -> Workload:
    ps = []
    for e in range(512):
        ps.append(ParamSpec(f"e{e}.gate", (1024, 4096), 0.02, 1e-3, 1e-3, group=e))
        ps.append(ParamSpec(f"e{e}.up", (1024, 4096), 0.02, 1e-3, 1e-3, group=e))
        ps.append(ParamSpec(f"e{e}.down", (4096, 1024), 0.02, 1e-3, 1e-3, group=e))
    ps.append(ParamSpec("router", (512, 4096), 0.02, 1e-3, 1e-3))
    return Workload("moe_bucket", 3, "512 experts x (1024x4096 x2, 4096x1024) + router "
                    "512x4096; per-expert grad scale log-uniform [0.1, 10]", ps,
                    scale_groups=True)


def _full_width() -> Workload:
    L = 102
    d = ladder_hidden(L)           # 8704
    ps = [ParamSpec(f"attn.{nm}", (d, d), 0.02, 1e-3, 1e-3) for nm in ("q", "k", "v", "o")]
    ps.append(ParamSpec("shared.gate", (d, 3072), 0.02, 1e-3, 1e-3))
    ps.append(ParamSpec("shared.up", (d, 3072), 0.02, 1e-3, 1e-3))
    ps.append(ParamSpec("shared.down", (3072, d), 0.02, 1e-3, 1e-3))
    for e in range(7):
        for nm in ("gate", "up", "down"):
            ps.append(ParamSpec(f"e{e}.{nm}", (1024, d), 0.02, 1e-3, 1e-3))
    ps.append(ParamSpec("router", (512, d), 0.02, 1e-3, 1e-3))
    return Workload("full_width", 4, "ladder rule at L=102 (d=8704): 4 x 8704^2, shared "
                    "expert 2 x 8704x3072 + 3072x8704, 21 x 1024x8704, router 512x8704", ps)


def _moe_slice() -> Workload:
    d, head = 4096, 128
    ps = []
    e_id = 0
    for layer in range(4):
        glob = layer == 3
        kv = 2 if glob else 16
        ps.append(ParamSpec(f"l{layer}.q", (d, d), 0.02, 1e-3, 1e-3, "bf16"))
        ps.append(ParamSpec(f"l{layer}.k", (kv * head, d), 0.02, 1e-3, 1e-3, "bf16"))
        ps.append(ParamSpec(f"l{layer}.v", (kv * head, d), 0.02, 1e-3, 1e-3, "bf16"))
        ps.append(ParamSpec(f"l{layer}.o", (d, d), 0.02, 1e-3, 1e-3, "bf16"))
        ps.append(ParamSpec(f"l{layer}.head_gate", (32, d), 0.02, 1e-3, 1e-3, "bf16"))
        ps.append(ParamSpec(f"l{layer}.shared.gate", (3072, d), 0.02, 1e-3, 1e-3, "bf16"))
        ps.append(ParamSpec(f"l{layer}.shared.up", (3072, d), 0.02, 1e-3, 1e-3, "bf16"))
        ps.append(ParamSpec(f"l{layer}.shared.down", (d, 3072), 0.02, 1e-3, 1e-3, "bf16"))
        ps.append(ParamSpec(f"l{layer}.shared_gate", (1, d), 0.02, 1e-3, 1e-3, "bf16"))
        ps.append(ParamSpec(f"l{layer}.router", (512, d), 0.02, 1e-3, 1e-3, "bf16"))
        ps.append(ParamSpec(f"l{layer}.norm1", (d,), 0.02, 1e-3, 1e-3, "bf16"))
        ps.append(ParamSpec(f"l{layer}.norm2", (d,), 0.02, 1e-3, 1e-3, "bf16"))
        for e in range(512):
            for nm, shp in (("gate", (1024, d)), ("up", (1024, d)), ("down", (d, 1024))):
                ps.append(ParamSpec(f"l{layer}.e{e}.{nm}", shp, 0.02, 1e-3, 1e-3, "bf16",
                                    group=e_id))
            e_id += 1
    lr, wd = lr_wd_from_laws(1e5, 50e12 / 80e9)
    return Workload("moe_slice", 5, "4-layer MoE slice, d=4096, 32 heads, 512 experts "
                    "(inner 1024), bf16 grads; 6184 matrices in 8 buckets + 8 norm vectors",
                    ps, lr=lr, wd=wd, scale_groups=True,
                    notes={"lr_wd": "laws at steps=1e5, TPP=625, natural log"})


_BUILDERS = {"tiny": _tiny, "ladder24": _ladder24, "moe_bucket": _moe_bucket,
             "full_width": _full_width, "moe_slice": _moe_slice}
WORKLOADS = tuple(_BUILDERS)


def get(key: str) -> Workload:
    if key not in _BUILDERS:
        raise KeyError(f"unknown workload {key!r}; known: {', '.join(WORKLOADS)}")
    return _BUILDERS[key]()


def _rng(cid: int, index: int, role: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([SEED, cid, index, role]))


def seed_of(cid: int, index: int, role: int) -> int:
    """64-bit seed of one (workload, parameter, role) draw."""
    h = hashlib.blake2b(f"{SEED}:{cid}:{index}:{role}".encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def group_scale(cid: int, group: int) -> float:
    """Per-expert gradient scale, log-uniform in [0.1, 10] (mimics skewed token load)."""
    u = _rng(cid, group, ROLE_SCALE).uniform(math.log(0.1), math.log(10.0))
    return float(math.exp(u))


def generate(w: Workload, index: int, roles=("W", "M", "G"), device="cpu") -> dict:
    """Seeded float32 torch tensors for parameter `index` of workload `w` on `device`.

    Each role is N(0, std) from torch's generator on that device, seeded with
    seed_of(cid, index, role) (on a GPU that is torch's counter-based Philox generator).
    The draw depends on the device type, so parity tests draw on the GPU and hand the
    oracle host copies taken before any library call.  Expert gradients are multiplied by
    their expert's scale.  G is float32 here; a bf16-gradient parameter is rounded to
    bf16 (nearest even) by the caller that builds its tensor.
    """
    import torch

    p = w.params[index]
    dev = torch.device(device)
    out = {}
    for role, code, std in (("W", ROLE_W, p.w_std), ("M", ROLE_M, p.m_std), ("G", ROLE_G, p.g_std)):
        if role not in roles:
            continue
        g = torch.Generator(device=dev)
        g.manual_seed(seed_of(w.cid, index, code))
        t = torch.randn(p.shape, generator=g, device=dev, dtype=torch.float32)
        scale = std
        if role == "G" and w.scale_groups and p.group >= 0:
            scale = std * group_scale(w.cid, p.group)
        out[role] = t.mul_(float(np.float32(scale)))
    return out
