"""The symmetric intermediates of one Newton-Schulz iteration, read back from the workspace.

SYRK computes the upper-triangle tiles of A = X X^T and stores each also as its mirror;
the poly computes the upper-triangle tiles of B = bA + cA^2 the same way, and on a
diagonal tile only the blocks on or above the diagonal, the ones below being stored as
transposes read from the waves that computed them.  After one iteration (beta = 0, so X0 is
the gradient's bf16 value) A and B must be exactly symmetric, and close to float64 products
of the GPU's own inputs: X from the oracle's normalisation (bitwise the GPU's), B from the
GPU's A.  Shapes cover persistent launches (at least 512 tiles) and one-tile-per-workgroup
launches of the 256-row tiles, with and without padding.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from oracle import muon_oracle as orc  # noqa: E402

A_, B_, C_, EPS = 3.4445, -4.7750, 2.0315, 1e-7
ALIGN = 256


def _align(v):
    return (v + ALIGN - 1) // ALIGN * ALIGN


def _params(shape, count, seed):
    from muon_newton_schulz_momentum_amd.harness import ParamTensors
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    out = []
    for _ in range(count):
        G = torch.randn(shape, generator=gen, device="cuda") * 1e-3
        out.append(ParamTensors(torch.zeros_like(G), torch.zeros_like(G), G))
    return out


def _buffers(plan, chunk):
    """A and B of every matrix of a chunk (count x m_pad x m_pad bf16), from the region
    layout: X ping-pong (XP, XQ), then A, then B, each 256-byte aligned."""
    ci = plan.chunk_info(chunk)
    xb = ci.count * ci.m_pad * ci.n_pad * 2
    ab = ci.count * ci.m_pad * ci.m_pad * 2
    off_a = _align(_align(ci.region_offset + xb) + xb)
    off_b = _align(off_a + ab)
    ws = plan.workspace

    def view(off):
        start = plan._ws_off + off
        return ws[start:start + ab].view(torch.bfloat16).view(ci.count, ci.m_pad, ci.m_pad)
    return view(off_a), view(off_b), ci


@pytest.mark.parametrize("shape,count", [((1024, 4096), 64), ((1100, 1300), 2), ((4096, 2048), 2),
                                         ((2048, 5632), 16)])
def test_symmetric_intermediates(shape, count):
    from muon_newton_schulz_momentum_amd import harness
    params = _params(shape, count, seed=900 + shape[0] // 7 + count)
    plan = harness.Plan(params)
    assert plan.n_chunks == 1
    plan.momentum_update(0.0)
    plan.ns_batched(A_, B_, C_, 1, EPS)
    torch.cuda.synchronize()
    A, B, ci = _buffers(plan, 0)
    assert ci.tile == 256
    m = ci.m
    tiles = (ci.m_pad // 256) * (ci.m_pad // 256 + 1) // 2 * ci.count
    print(f"{shape} x {count}: {tiles} upper-triangle tiles per launch")
    for name, T in (("A", A), ("B", B)):
        t = T[:, :m, :m].contiguous().view(torch.int16)
        bad = (t != t.transpose(1, 2)).sum().item()
        assert bad == 0, f"{name} of {shape}: {bad} elements differ from their mirror"
    for k in sorted({0, count // 2, count - 1}):
        X0 = params[k].grad.cpu().numpy().astype(np.float64)
        X0 = orc.bf16_round(X0)
        t = orc.canonical_orientation(*X0.shape)
        X = orc.frobenius_normalise(X0.T if t else X0, EPS)
        Ag = A[k, :m, :m].float().cpu().numpy().astype(np.float64)
        Bg = B[k, :m, :m].float().cpu().numpy().astype(np.float64)
        A_ref = X @ X.T
        B_ref = B_ * Ag + C_ * (Ag @ Ag)
        ea = np.linalg.norm(Ag - A_ref) / np.linalg.norm(A_ref)
        eb = np.linalg.norm(Bg - B_ref) / np.linalg.norm(B_ref)
        print(f"  matrix {k}: A rel err {ea:.2e}, B rel err {eb:.2e}")
        # one bf16 rounding of each result (2^-9 relative) on top of float32 accumulation
        assert ea <= 4e-3 and eb <= 4e-3, (k, ea, eb)
    plan.close()
