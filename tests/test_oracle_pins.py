"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test ties one oracle function to mathematics, to a library routine, to brute force
on tiny inputs, or to values the pages print (tests/golden/), so that a plausible
mistake (a dropped term, a wrong sign, a transposed operand, a rounding at the wrong
place) fails at least one of them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import muon_oracle as orc

A, B, C = 3.4445, -4.7750, 2.0315
K = 5
EPS = 1e-7


# ----------------------------------------------------------------------------------------
# bf16 rounding
# ----------------------------------------------------------------------------------------

def _all_finite_bf16():
    """Every finite bf16 value (as float64), sorted, with its 16-bit pattern."""
    pats = np.arange(1 << 16, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        vals = (pats << 16).view(np.float32).astype(np.float64)
    keep = np.isfinite(vals)
    pats, vals = pats[keep], vals[keep]
    # one zero is enough; -0 and +0 compare equal
    order = np.argsort(vals, kind="stable")
    vals, pats = vals[order], pats[order]
    uniq = np.concatenate([[True], vals[1:] != vals[:-1]])
    return vals[uniq], pats[uniq]


_BF_VALS, _BF_PATS = _all_finite_bf16()
_BF_MAX = _BF_VALS[-1]


def _nearest_bf16_bruteforce(x: float) -> float:
    """Nearest bf16 by search over the table of all bf16 values; ties to even pattern."""
    if x == 0.0:
        return x
    if abs(x) > _BF_MAX:
        # halfway between the largest finite value and 2^128 (the next step) rounds away
        step = 2.0 ** 120
        return np.copysign(np.inf, x) if abs(x) >= _BF_MAX + step / 2 else np.copysign(_BF_MAX, x)
    i = int(np.searchsorted(_BF_VALS, x))
    lo, hi = _BF_VALS[i - 1], _BF_VALS[i]
    if hi == x:
        return hi
    dlo, dhi = Fraction(x) - Fraction(lo), Fraction(hi) - Fraction(x)
    if dlo < dhi:
        return lo
    if dhi < dlo:
        return hi
    return lo if (_BF_PATS[i - 1] & 1) == 0 else hi


def test_bf16_round_matches_bruteforce_nearest():
    rng = np.random.default_rng(1)
    xs = list(rng.standard_normal(3000) * np.exp(rng.uniform(-30, 30, 3000)))
    # exact midpoints between neighbouring bf16 values (ties) and their neighbours
    idx = rng.integers(1, len(_BF_VALS) - 1, 2000)
    mids = (_BF_VALS[idx] + _BF_VALS[idx + 1]) / 2.0
    xs += list(mids) + list(np.nextafter(mids, np.inf)) + list(np.nextafter(mids, -np.inf))
    # gradual-underflow range and the overflow threshold
    xs += list(rng.uniform(-2.0 ** -126, 2.0 ** -126, 500))
    xs += [2.0 ** -133, 2.0 ** -134, 1.5 * 2.0 ** -134, 3 * 2.0 ** -135, -2.0 ** -135]
    xs += [float(_BF_MAX), float(_BF_MAX) + 2.0 ** 119, np.nextafter(float(_BF_MAX) + 2.0 ** 119, 0)]
    xs = np.array(xs, dtype=np.float64)
    got = orc.bf16_round(xs)
    want = np.array([_nearest_bf16_bruteforce(float(v)) for v in xs])
    np.testing.assert_array_equal(got, want)


def test_bf16_round_matches_torch_cast_on_fp32_patterns():
    # Every high half-word (sign, exponent, top mantissa bits) with the low half-words
    # that decide rounding: exact, just under/at/over the tie, and a random spread.
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x3FFF, 0x7FFF, 0x8000, 0x8001, 0xC000, 0xFFFF]
                    + list(np.random.default_rng(2).integers(0, 1 << 16, 8)), dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).reshape(-1)
    f = bits.view(np.float32)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).to(torch.float32).numpy()
    with np.errstate(invalid="ignore"):
        got = orc.bf16_round(f.astype(np.float64)).astype(np.float32)
    nan_w, nan_g = np.isnan(want), np.isnan(got)
    np.testing.assert_array_equal(nan_w, nan_g)
    np.testing.assert_array_equal(got[~nan_g].view(np.uint32), want[~nan_w].view(np.uint32))


def test_f32_matches_fraction_rounding():
    rng = np.random.default_rng(3)
    xs = rng.standard_normal(200) * np.exp(rng.uniform(-20, 20, 200))
    got = orc.f32(xs)
    for v, g in zip(xs, got):
        # float32 neighbours bracket v; the closer one (ties: even mantissa) must be chosen
        lo = np.float32(v)
        cands = [np.nextafter(lo, np.float32(-np.inf)), lo, np.nextafter(lo, np.float32(np.inf))]
        best = min(cands, key=lambda c: (abs(Fraction(float(c)) - Fraction(float(v))),
                                          int(np.array(c).view(np.uint32)) & 1))
        assert float(best) == g


# ----------------------------------------------------------------------------------------
# momentum update
# ----------------------------------------------------------------------------------------

def test_momentum_one_step_exact_rational():
    rng = np.random.default_rng(4)
    M = (rng.standard_normal(64) * 0.02).astype(np.float32)
    G = (rng.standard_normal(64) * 1e-3).astype(np.float32)
    beta = 0.95
    Mn, X0 = orc.momentum_update(M, G, beta)
    b = Fraction(float(np.float32(beta)))
    omb = Fraction(float(np.float32(1.0) - np.float32(beta)))
    assert omb == 1 - b  # Sterbenz: exact in float32 for beta in [0.5, 1]
    for i in range(64):
        exact = b * Fraction(float(M[i])) + omb * Fraction(float(G[i]))
        want = np.float32(float(exact))  # float(Fraction) rounds to nearest float64
        assert Mn[i] == want
        assert X0[i] == _nearest_bf16_bruteforce(float(Mn[i]))
    assert Mn.dtype == np.float32


def test_momentum_closed_form_constant_gradient():
    # M_0 = 0 and a constant G give M_t = (1 - beta^t) G.
    rng = np.random.default_rng(5)
    G = (rng.standard_normal((16, 24)) * 1e-3).astype(np.float32)
    beta = 0.9
    M = np.zeros_like(G)
    for t in range(1, 41):
        M, _ = orc.momentum_update(M, G, beta)
        want = (1 - np.float64(np.float32(beta)) ** t) * G.astype(np.float64)
        err = np.abs(M - want) / np.abs(want)
        assert err.max() <= t * 2.0 ** -24


def test_momentum_beta_zero_stages_gradient():
    rng = np.random.default_rng(6)
    M = rng.standard_normal((5, 7)).astype(np.float32)
    G = rng.standard_normal((5, 7)).astype(np.float32)
    Mn, _ = orc.momentum_update(M, G, 0.0)
    np.testing.assert_array_equal(Mn, G)


def test_momentum_bf16_gradient_widens_exactly():
    G32 = np.random.default_rng(7).standard_normal(100).astype(np.float32)
    Gb = torch.from_numpy(G32).to(torch.bfloat16).to(torch.float32).numpy()
    Mn, _ = orc.momentum_update(np.zeros(100, np.float32), Gb, 0.0)
    np.testing.assert_array_equal(Mn, Gb)


# ----------------------------------------------------------------------------------------
# Newton–Schulz: exact mode against the SVD closed form
# ----------------------------------------------------------------------------------------

def _p(s, a=A, b=B, c=C):
    a, b, c = (float(np.float32(v)) for v in (a, b, c))
    return a * s + b * s ** 3 + c * s ** 5


def _pk(s, k=K):
    for _ in range(k):
        s = _p(s)
    return s


def _svd_closed_form(X0, k=K, eps=EPS):
    U, S, Vt = np.linalg.svd(X0, full_matrices=False)
    nu = np.linalg.norm(X0)
    eps64 = float(np.float32(eps))
    return (U * _pk(S / (nu + eps64), k)) @ Vt


@pytest.mark.parametrize("shape", [(5, 9), (16, 16), (9, 4), (1, 12), (12, 1), (32, 48), (40, 17)])
@pytest.mark.parametrize("k", [1, 2, 5])
def test_ns_exact_mode_equals_svd_closed_form(shape, k):
    X0 = np.random.default_rng(hash(shape) % 1000 + k).standard_normal(shape)
    O = orc.newton_schulz(X0, A, B, C, k, EPS, emulate_bf16=False)
    ref = _svd_closed_form(X0, k)
    assert O.shape == X0.shape
    assert np.linalg.norm(O - ref) <= 1e-10 * max(np.linalg.norm(ref), 1e-300)


def test_ns_exact_mode_rank_deficient():
    rng = np.random.default_rng(8)
    X0 = rng.standard_normal((12, 3)) @ rng.standard_normal((3, 20))
    O = orc.newton_schulz(X0, A, B, C, K, EPS, emulate_bf16=False)
    assert np.linalg.norm(O - _svd_closed_form(X0)) <= 1e-10 * np.linalg.norm(O)


def test_ns_each_coefficient_matters():
    # Changing any one coefficient changes the result as the closed form predicts.
    X0 = np.random.default_rng(9).standard_normal((6, 10))
    for a, b, c in [(A, 0.0, 0.0), (0.0, B, 0.0), (0.0, 0.0, C), (1.0, -1.0, 0.5)]:
        O = orc.newton_schulz(X0, a, b, c, 2, EPS, emulate_bf16=False)
        U, S, Vt = np.linalg.svd(X0, full_matrices=False)
        s = S / (np.linalg.norm(X0) + float(np.float32(EPS)))
        for _ in range(2):
            s = _p(s, a, b, c)
        ref = (U * s) @ Vt
        assert np.linalg.norm(O - ref) <= 1e-10 * max(np.linalg.norm(ref), 1e-30)


# ----------------------------------------------------------------------------------------
# Newton–Schulz: special cases
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("emulate", [True, False])
def test_ns_zero_matrix_is_zero(emulate):
    O = orc.newton_schulz(np.zeros((7, 11)), A, B, C, K, EPS, emulate_bf16=emulate)
    assert np.all(O == 0.0)


def test_ns_rank_one_scalar_map():
    # A rank-1 X0 = nu u v^T has the single singular value nu; after normalising it is
    # nu/(nu+eps) and the output is p^k(that) * X0 / nu.
    rng = np.random.default_rng(10)
    for shape in [(1, 64), (64, 1), (8, 8), (3, 50)]:
        u = rng.standard_normal((shape[0], 1))
        v = rng.standard_normal((1, shape[1]))
        X0 = u @ v
        nu = np.linalg.norm(X0)
        O = orc.newton_schulz(X0, A, B, C, K, EPS, emulate_bf16=False)
        s = _pk(nu / (nu + float(np.float32(EPS))))
        np.testing.assert_allclose(O, s * X0 / nu, rtol=1e-12, atol=1e-15)
    # the scalar itself at s0 = 1: 0.6964364095 with the decimal coefficients, and a
    # few 1e-8 lower once they are rounded to float32 as the library receives them
    s = 1.0
    for _ in range(K):
        s = A * s + B * s ** 3 + C * s ** 5
    assert abs(s - 0.6964364095) < 1e-9
    assert abs(_pk(1.0) - 0.6964364095) < 1e-7


def test_ns_diagonal_and_orthogonal():
    d = np.array([3.0, -1.0, 0.5, 2.0, 0.25])
    X0 = np.diag(d)
    O = orc.newton_schulz(X0, A, B, C, K, EPS, emulate_bf16=False)
    nu = np.linalg.norm(d) + float(np.float32(EPS))
    # p is odd, so signs carry through
    np.testing.assert_allclose(O, np.diag(np.sign(d) * _pk(np.abs(d) / nu)), rtol=1e-12, atol=1e-15)
    Q, _ = np.linalg.qr(np.random.default_rng(11).standard_normal((24, 24)))
    O = orc.newton_schulz(Q, A, B, C, K, EPS, emulate_bf16=False)
    s = _pk(1.0 / (np.sqrt(24) + float(np.float32(EPS))))
    np.testing.assert_allclose(O, s * Q, rtol=1e-11, atol=1e-13)


# ----------------------------------------------------------------------------------------
# Newton–Schulz: invariances
# ----------------------------------------------------------------------------------------

def test_ns_transpose_equivariance_bitwise_for_rectangular():
    X0 = orc.bf16_round(np.random.default_rng(12).standard_normal((9, 20)))
    O1 = orc.newton_schulz(X0, A, B, C, K, EPS, emulate_bf16=True)
    O2 = orc.newton_schulz(X0.T.copy(), A, B, C, K, EPS, emulate_bf16=True)
    np.testing.assert_array_equal(O1, O2.T)


def test_ns_orthogonal_equivariance_exact_mode():
    rng = np.random.default_rng(13)
    X0 = rng.standard_normal((10, 16))
    Q, _ = np.linalg.qr(rng.standard_normal((10, 10)))
    R, _ = np.linalg.qr(rng.standard_normal((16, 16)))
    O = orc.newton_schulz(X0, A, B, C, K, EPS, emulate_bf16=False)
    O2 = orc.newton_schulz(Q @ X0 @ R, A, B, C, K, EPS, emulate_bf16=False)
    assert np.linalg.norm(O2 - Q @ O @ R) <= 1e-10 * np.linalg.norm(O)


def test_ns_orthogonal_equivariance_bf16_mode():
    rng = np.random.default_rng(14)
    X0 = rng.standard_normal((32, 64))
    Q, _ = np.linalg.qr(rng.standard_normal((32, 32)))
    R, _ = np.linalg.qr(rng.standard_normal((64, 64)))
    O = orc.newton_schulz(orc.bf16_round(X0), A, B, C, K, EPS)
    O2 = orc.newton_schulz(orc.bf16_round(Q @ X0 @ R), A, B, C, K, EPS)
    ref = Q @ O @ R
    assert np.linalg.norm(O2 - ref) <= 5e-2 * np.linalg.norm(ref)


def test_ns_scale_invariance():
    X0 = np.random.default_rng(15).standard_normal((12, 30))
    O = orc.newton_schulz(X0, A, B, C, K, 0.0, emulate_bf16=False)
    O2 = orc.newton_schulz(X0 * 1e-3, A, B, C, K, 0.0, emulate_bf16=False)
    np.testing.assert_allclose(O, O2, rtol=1e-10, atol=1e-13)


# ----------------------------------------------------------------------------------------
# Newton–Schulz: singular-value band and the bf16/exact gap
# ----------------------------------------------------------------------------------------

def _band(lo):
    s = np.linspace(lo, 1.0, 200001)
    v = _pk(s)
    return v.min(), v.max()


def test_quintic_band_values():
    lo5, hi5 = _band(5e-3)
    lo1, hi1 = _band(1e-2)
    assert abs(_p(1.0) - 0.701) < 1e-3
    s = np.linspace(0, 1, 1000001)
    assert abs(_p(s).max() - 1.2024) < 1e-3
    assert 0.68 <= lo1 and hi1 <= 1.14


@pytest.mark.parametrize("shape", [(32, 64), (64, 128), (48, 48)])
def test_ns_output_singular_values_in_band(shape):
    rng = np.random.default_rng(shape[0] * 1000 + shape[1])
    X0 = orc.bf16_round(rng.standard_normal(shape))
    S0 = np.linalg.svd(X0, compute_uv=False) / (np.linalg.norm(X0) + float(np.float32(EPS)))
    for emulate, slack in [(False, 1e-9), (True, 2e-2)]:
        O = orc.newton_schulz(X0, A, B, C, K, EPS, emulate_bf16=emulate)
        S = np.linalg.svd(O, compute_uv=False)
        # singular values are sorted descending in both; the scalar map is monotone on the
        # part of [0, 1] the normalised values occupy only piecewise, so compare the set of
        # outputs coming from inputs above the threshold with the band over that range
        thr = 1e-2
        keep = S0 >= thr
        lo, hi = _band(max(S0[keep].min(), thr))
        exact_out = np.sort(_pk(S0[keep]))
        assert exact_out.min() >= lo - 1e-12 and exact_out.max() <= hi + 1e-12
        big = np.sort(S)[::-1][: keep.sum()]
        assert big.max() <= hi + slack
        assert big.min() >= lo - slack


@pytest.mark.parametrize("shape", [(64, 128), (128, 128)])
def test_ns_bf16_vs_exact_gap_is_small(shape):
    X0 = orc.bf16_round(np.random.default_rng(16).standard_normal(shape))
    Ob = orc.newton_schulz(X0, A, B, C, K, EPS, emulate_bf16=True)
    Oe = orc.newton_schulz(X0, A, B, C, K, EPS, emulate_bf16=False)
    gap = np.linalg.norm(Ob - Oe) / np.linalg.norm(Oe)
    assert 1e-4 < gap < 5e-2, gap   # rounding is really applied, and stays moderate


# ----------------------------------------------------------------------------------------
# Newton–Schulz: bf16 mode by brute force with exact rationals on a tiny input
# ----------------------------------------------------------------------------------------

def _frac_mat(X):
    return [[Fraction(float(v)) for v in row] for row in X]


def _mm(P, Q):
    return [[sum(P[i][k] * Q[k][j] for k in range(len(Q))) for j in range(len(Q[0]))]
            for i in range(len(P))]


def _rb(P):
    return [[Fraction(_nearest_bf16_bruteforce(float(v))) for v in row] for row in P]


def test_ns_iterate_bf16_bruteforce_rational():
    # Small integers times powers of two keep every float64 intermediate of the oracle
    # exact, so its one rounding per stored matrix must equal exact-rational rounding.
    rng = np.random.default_rng(17)
    X = rng.integers(-40, 41, (3, 4)).astype(np.float64) / 64.0
    X = orc.bf16_round(X)
    a, b, c = (Fraction(float(np.float32(v))) for v in (A, B, C))
    Xr = _frac_mat(X)
    for _ in range(2):
        Ar = _rb(_mm(Xr, [list(r) for r in zip(*Xr)]))
        AA = _mm(Ar, Ar)
        Br = _rb([[b * Ar[i][j] + c * AA[i][j] for j in range(3)] for i in range(3)])
        BX = _mm(Br, Xr)
        Xr = _rb([[a * Xr[i][j] + BX[i][j] for j in range(4)] for i in range(3)])
    got = orc.ns_iterate(X, A, B, C, 2, emulate_bf16=True)
    want = np.array([[float(v) for v in row] for row in Xr])
    np.testing.assert_array_equal(got, want)


def test_ns_iteration_rows_bf16_bruteforce_rational():
    # one step on a tiny exact input, rows picked out of order and repeated
    rng = np.random.default_rng(23)
    X = orc.bf16_round(rng.integers(-40, 41, (4, 6)).astype(np.float64) / 64.0)
    a, b, c = (Fraction(float(np.float32(v))) for v in (A, B, C))
    Xr = _frac_mat(X)
    Ar = _rb(_mm(Xr, [list(r) for r in zip(*Xr)]))
    AA = _mm(Ar, Ar)
    Br = _rb([[b * Ar[i][j] + c * AA[i][j] for j in range(4)] for i in range(4)])
    BX = _mm(Br, Xr)
    X1 = _rb([[a * Xr[i][j] + BX[i][j] for j in range(6)] for i in range(4)])
    rows = [3, 0, 3]
    got = orc.ns_iteration_rows(X, A, B, C, rows, emulate_bf16=True)
    want = np.array([[float(v) for v in X1[r]] for r in rows])
    np.testing.assert_array_equal(got, want)


def test_ns_iteration_rows_exact_mode_is_svd_polynomial():
    # exact mode: one step maps X = U S V^T to U p(S) V^T, p(s) = a s + b s^3 + c s^5
    rng = np.random.default_rng(24)
    X = rng.standard_normal((20, 33))
    X /= np.linalg.norm(X)
    U, S, Vt = np.linalg.svd(X, full_matrices=False)
    a, b, c = (float(np.float32(v)) for v in (A, B, C))
    P = (U * (a * S + b * S ** 3 + c * S ** 5)) @ Vt
    rows = [0, 7, 19, 4]
    got = orc.ns_iteration_rows(X, A, B, C, rows, emulate_bf16=False)
    np.testing.assert_allclose(got, P[rows], rtol=0, atol=1e-12)


def test_normalise_rounds_scaled_values_once():
    X0 = orc.bf16_round(np.random.default_rng(18).standard_normal((4, 6)))
    X = orc.frobenius_normalise(X0, EPS)
    nu = np.sqrt(np.sum(X0 ** 2))
    inv = 1.0 / (nu + float(np.float32(EPS)))
    for v, g in zip(X0.ravel(), X.ravel()):
        assert g == _nearest_bf16_bruteforce(float(v * inv))
    assert abs(np.linalg.norm(X) - 1.0) < 1e-2


# ----------------------------------------------------------------------------------------
# apply
# ----------------------------------------------------------------------------------------

def test_apply_one_step_exact_rational():
    rng = np.random.default_rng(19)
    W = (rng.standard_normal(50) * 0.02).astype(np.float32)
    O = orc.bf16_round(rng.standard_normal(50))
    lr, wd, s = 0.02, 0.1, 1.5
    got = orc.apply_update(W, O, lr, wd, s)
    lr_, wd_, s_ = (Fraction(float(np.float32(v))) for v in (lr, wd, s))
    d = Fraction(float(1 - lr_ * wd_))          # one float64 rounding of 1 - lr*wd
    u = lr_ * s_                                 # exact in float64
    assert Fraction(float(u)) == u
    for i in range(50):
        t1 = Fraction(float(d * Fraction(float(W[i]))))
        t2 = Fraction(float(u * Fraction(float(O[i]))))
        want = np.float32(float(t1 - t2))
        assert got[i] == want


def test_apply_closed_form_over_steps():
    # Fixed O over t steps: W_t = d^t W_0 - u O (1 - d^t) / (1 - d).
    rng = np.random.default_rng(20)
    W0 = (rng.standard_normal((8, 8)) * 0.02).astype(np.float32)
    O = orc.bf16_round(rng.standard_normal((8, 8)) * 0.1)
    lr, wd = 0.02, 0.1
    W = W0
    d = 1 - float(np.float32(lr)) * float(np.float32(wd))
    u = float(np.float32(lr))
    for t in range(1, 31):
        W = orc.apply_update(W, O, lr, wd)
        want = d ** t * W0.astype(np.float64) - u * O * (1 - d ** t) / (1 - d)
        scale = np.abs(W0).max() + u * np.abs(O).max() * t
        assert np.abs(W - want).max() <= 2 * t * 2.0 ** -24 * scale


def test_apply_zero_update_is_pure_decay():
    W = np.random.default_rng(21).standard_normal(20).astype(np.float32)
    got = orc.apply_update(W, np.zeros(20), 0.5, 0.0)
    np.testing.assert_array_equal(got, W)


# ----------------------------------------------------------------------------------------
# whole step
# ----------------------------------------------------------------------------------------

def test_step_cast_points_and_order():
    rng = np.random.default_rng(22)
    W = (rng.standard_normal((6, 10)) * 0.02).astype(np.float32)
    M = (rng.standard_normal((6, 10)) * 0.02).astype(np.float32)
    G = (rng.standard_normal((6, 10)) * 0.02).astype(np.float32)
    kw = dict(beta=0.95, a=A, b=B, c=C, steps=K, eps=EPS, lr=0.02, wd=0.1)
    out = orc.muon_step_ref(W, M, G, **kw)
    Mn, X0 = orc.momentum_update(M, G, 0.95)
    np.testing.assert_array_equal(out["M"], Mn)
    # the NS input is the bf16 cast of the float32 momentum, not of the float64 sum
    np.testing.assert_array_equal(out["X0"], orc.bf16_round(Mn.astype(np.float64)))
    np.testing.assert_array_equal(out["O"], orc.bf16_round(out["O"]))
    np.testing.assert_array_equal(out["W"], orc.apply_update(W, out["O"], 0.02, 0.1))
    assert out["W"].dtype == np.float32 and out["M"].dtype == np.float32


# ----------------------------------------------------------------------------------------
# update-scale rules
# ----------------------------------------------------------------------------------------

def test_update_scale_rules_exact_values():
    # values the formulas fix exactly (perfect squares, and 1 for wide matrices)
    assert orc.update_scale("none", 4096, 1024) == 1.0
    assert orc.update_scale("aspect", 4096, 1024) == 2.0          # sqrt(4)
    assert orc.update_scale("aspect", 9 * 64, 64) == 3.0          # sqrt(9)
    assert orc.update_scale("aspect", 1024, 4096) == 1.0          # wide: max(1, 1/4)
    assert orc.update_scale("aspect", 2048, 2048) == 1.0
    assert orc.update_scale("rms_match", 1024, 4096) == float(np.float32(0.2 * 64.0))
    assert orc.update_scale("rms_match", 4096, 1024) == float(np.float32(0.2 * 64.0))   # symmetric
    assert orc.update_scale("rms_match", 100, 2500) == float(np.float32(0.2 * 50.0))
    # aspect never shrinks an update; rms_match grows as the square root of the long side
    for r, c in ((5632, 2048), (32, 4096), (8704, 3072)):
        assert orc.update_scale("aspect", r, c) >= 1.0
        assert abs(orc.update_scale("rms_match", r, c) / orc.update_scale("rms_match", 4 * r, 4 * c) - 0.5) < 1e-7
    with pytest.raises(ValueError):
        orc.update_scale("bogus", 2, 2)


# ----------------------------------------------------------------------------------------
# coefficient schedules and the Nesterov look-ahead
# ----------------------------------------------------------------------------------------

SCHEDULE = [(4.0848, -6.8946, 2.9270), (3.9505, -6.3029, 2.6377), (3.7418, -5.5913, 2.3037),
            (2.8769, -3.1427, 1.2046), (2.8366, -3.0525, 1.2012)]


def test_schedule_exact_mode_is_composed_svd_polynomial():
    rng = np.random.default_rng(31)
    X0 = rng.standard_normal((24, 40))
    U, S, Vt = np.linalg.svd(X0, full_matrices=False)
    s = S / (np.linalg.norm(X0) + float(np.float32(EPS)))
    for a, b, c in SCHEDULE:
        a, b, c = (float(np.float32(v)) for v in (a, b, c))
        s = a * s + b * s ** 3 + c * s ** 5
    want = (U * s) @ Vt
    got = orc.newton_schulz_schedule(X0, SCHEDULE, EPS, emulate_bf16=False)
    assert np.linalg.norm(got - want) / np.linalg.norm(want) < 1e-10
    # the transpose goes through the canonical orientation
    got_t = orc.newton_schulz_schedule(X0.T, SCHEDULE, EPS, emulate_bf16=False)
    assert np.linalg.norm(got_t - want.T) / np.linalg.norm(want) < 1e-10


def test_schedule_bf16_bruteforce_rational():
    rng = np.random.default_rng(32)
    X = orc.bf16_round(rng.integers(-40, 41, (3, 5)).astype(np.float64) / 64.0)
    sched = SCHEDULE[:2]
    Xr = _frac_mat(X)
    for a, b, c in sched:
        a, b, c = (Fraction(float(np.float32(v))) for v in (a, b, c))
        Ar = _rb(_mm(Xr, [list(r) for r in zip(*Xr)]))
        AA = _mm(Ar, Ar)
        Br = _rb([[b * Ar[i][j] + c * AA[i][j] for j in range(3)] for i in range(3)])
        BX = _mm(Br, Xr)
        Xr = _rb([[a * Xr[i][j] + BX[i][j] for j in range(5)] for i in range(3)])
    got = orc.ns_iterate_schedule(X, sched, emulate_bf16=True)
    np.testing.assert_array_equal(got, np.array([[float(v) for v in row] for row in Xr]))


def test_nesterov_lookahead_closed_form_and_rational():
    # constant G from M0 = 0: M_t = (1 - beta^t) G, look-ahead N_t = (1 - beta^(t+1)) G
    beta = 0.9
    G = np.random.default_rng(33).standard_normal(64).astype(np.float32)
    M = np.zeros_like(G)
    b = float(np.float32(beta))
    for t in range(1, 8):
        M, X0 = orc.momentum_update(M, G, beta, nesterov=True)
        want = (1.0 - b ** (t + 1)) * G.astype(np.float64)
        np.testing.assert_allclose(X0, want, rtol=2 ** -8 + t * 2 ** -23, atol=0)
    # one step by exact rationals: N = RN32(RN64(b*M_new + (1-b)*G)), X0 = RNE_bf16(N)
    rng = np.random.default_rng(34)
    M0 = rng.standard_normal(40).astype(np.float32)
    G0 = rng.standard_normal(40).astype(np.float32)
    M1, X1 = orc.momentum_update(M0, G0, 0.95, nesterov=True)
    b = Fraction(float(np.float32(0.95)))
    omb = Fraction(float(np.float32(1.0) - np.float32(0.95)))
    for m0, g0, m1, x1 in zip(M0, G0, M1, X1):
        m_new = Fraction(float(np.float32(float(b * Fraction(float(m0)) + omb * Fraction(float(g0))))))
        assert float(m_new) == float(m1)
        n64 = float(b * m_new + omb * Fraction(float(g0)))          # one float64 rounding
        assert x1 == _nearest_bf16_bruteforce(float(np.float32(n64)))
    # beta = 0: the look-ahead is G itself (rounded to bf16)
    _, X = orc.momentum_update(M0, G0, 0.0, nesterov=True)
    np.testing.assert_array_equal(X, orc.bf16_round(G0.astype(np.float64)))


# ----------------------------------------------------------------------------------------
# AdamW companion
# ----------------------------------------------------------------------------------------

def _r64(x):
    return Fraction(float(x))          # one float64 rounding of an exact rational


def test_adamw_one_step_exact_rational():
    rng = np.random.default_rng(41)
    W = (rng.standard_normal(30) * 0.02).astype(np.float32)
    M = (rng.standard_normal(30) * 1e-3).astype(np.float32)
    V = np.abs(rng.standard_normal(30) * 1e-6).astype(np.float32)
    G = (rng.standard_normal(30) * 1e-3).astype(np.float32)
    lr, b1, b2, eps, wd, t = 1e-3, 0.9, 0.95, 1e-8, 0.1, 7
    w1, m1, v1 = orc.adamw_update(W, M, V, G, lr=lr, beta1=b1, beta2=b2, eps=eps, wd=wd, step=t)
    F = lambda v: Fraction(float(np.float32(v)))       # noqa: E731  float32 input, exact
    lr_, wd_, eps_ = F(lr), F(wd), F(eps)
    b1_, b2_ = F(b1), F(b2)
    omb1 = Fraction(float(np.float32(1.0) - np.float32(b1)))
    omb2 = Fraction(float(np.float32(1.0) - np.float32(b2)))
    bc1 = _r64(1 - _r64(float(b1_) ** t))
    bc2 = _r64(1 - _r64(float(b2_) ** t))
    for w0, m0, v0, g0, wg, mg, vg in zip(W, M, V, G, w1, m1, v1):
        g = Fraction(float(g0))
        m = Fraction(float(np.float32(float(_r64(b1_ * Fraction(float(m0)) + omb1 * g)))))
        sq = _r64(omb2 * (g * g))                       # g*g exact, then one rounding
        v = Fraction(float(np.float32(float(_r64(b2_ * Fraction(float(v0)) + sq)))))
        mhat = _r64(m / bc1)
        vhat = _r64(v / bc2)
        den = _r64(Fraction(math.sqrt(float(vhat))) + eps_)   # sqrt correctly rounded
        upd = _r64(_r64(lr_ * mhat) / den)
        d = _r64(1 - lr_ * wd_)
        w = float(np.float32(float(_r64(_r64(d * Fraction(float(w0))) - upd))))
        assert (float(m), float(v), w) == (float(mg), float(vg), float(wg))


def test_adamw_first_step_closed_form():
    # t = 1 from zero moments: m/bc1 = g and v/bc2 = g^2 up to roundings, so the update is
    # lr * g / (|g| + eps): a sign step of size lr for |g| >> eps
    rng = np.random.default_rng(42)
    G = (rng.standard_normal(200) * 1e-2).astype(np.float32)
    W = (rng.standard_normal(200) * 0.02).astype(np.float32)
    Z = np.zeros_like(G)
    lr, wd = 1e-3, 0.0
    w1, m1, v1 = orc.adamw_update(W, Z, Z, G, lr=lr, beta1=0.9, beta2=0.999, eps=1e-12, wd=wd, step=1)
    lr32 = float(np.float32(lr))
    np.testing.assert_allclose(w1.astype(np.float64), W.astype(np.float64) - lr32 * np.sign(G),
                               rtol=0, atol=4e-9)
    np.testing.assert_allclose(m1, (1 - np.float32(0.9)) * G, rtol=1e-6)
    np.testing.assert_allclose(v1, (1 - np.float32(0.999)) * G.astype(np.float64) ** 2, rtol=1e-6)
    # lr = 0 and wd = 0 leave W untouched whatever the moments
    w0, _, _ = orc.adamw_update(W, m1, v1, G, lr=0.0, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.0, step=3)
    np.testing.assert_array_equal(w0, W)
