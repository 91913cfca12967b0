"""Plain, slow CPU oracle for one Muon optimizer step (float64 between bf16 cast points).

TEST INFRASTRUCTURE ONLY.  This module is the checker, not the product: only the
tests, the package's smoke check and the benchmark's CPU-baseline leg may import it.
It imports nothing from the HIP path and shares no code with it.

What it computes follows the pages' description of the Muon step
("Frontier Pre-training at Microsoft AI", method details section 5, "Scaling Muon to
16K GPUs", resharding steps 1, 3 and 5; the same step in "Microsoft Reveals MAI-Base-2
Training Recipe ...", section "How to Make Parameter Updates Faster and More Stable?",
and in "MAI-Base-2 в 4–12 раз экономнее DeepSeek на предобучении", section
"Muon обошёл AdamW, но потребовал пересобирать матрицы между GPU"):

  1. update the FP32 momentum of each matrix and cast it to BF16;
  3. orthogonalise each whole momentum matrix with a Newton–Schulz iteration;
  5. cast the update back to FP32 and apply it to the weights.

The pages leave the momentum form, the iteration's coefficients and step count, the
normaliser, the orientation and the weight-decay form open; each reading taken here is
marked READING below and listed with its reason in the design notes.

Two modes for the orthogonalisation:
  emulate_bf16=True   parity mode: X, A = X X^T and B = bA + cA^2 are rounded to bf16
                      (round to nearest, ties to even) at the same points as the GPU
                      stores them; every product and sum in between is float64.
  emulate_bf16=False  exact mode: no rounding beyond float64; checked against the SVD
                      closed form U p^k(S/nu) V^T.

Scalars that cross the C ABI as float32 (beta, a, b, c, eps, lr, wd, s) are rounded to
float32 first and then widened, exactly as the library receives them.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "f32",
    "bf16_round",
    "momentum_update",
    "canonical_orientation",
    "ns_iteration_rows",
    "frobenius_normalise",
    "ns_iterate",
    "ns_iterate_schedule",
    "newton_schulz_schedule",
    "newton_schulz",
    "apply_update",
    "update_scale",
    "adamw_update",
    "muon_step_ref",
]

_TWO_128 = 2.0 ** 128


def f32(x) -> np.ndarray:
    """Round to float32 (to nearest, ties to even) and widen back to float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even; result in float64.

    bfloat16 keeps float32's 8-bit exponent and 8 significant bits.  A finite value with
    binary exponent e (|x| in [2^(e-1), 2^e)) is therefore a multiple of 2^(e-8); below
    the smallest normal 2^-126 the step stays at 2^-133 (gradual underflow).  The value
    is scaled by that power of two (exact), rounded to an integer half-to-even, and
    scaled back (exact).  Results of magnitude 2^128 or more overflow to infinity.
    NaN and infinities pass through.

    READING: one rounding, directly from float64.  (The notes page, section 5 step 1,
    names the momentum's BF16 conversion with a term whose literal sense is truncation;
    the other three pages speak of a plain cast.  Round-to-nearest-even is taken for
    every cast.)
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    finite = np.isfinite(x)
    xf = x[finite]
    _, e = np.frexp(xf)
    q = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(xf, -q)), q)
    big = np.abs(r) >= _TWO_128
    r[big] = np.copysign(np.inf, r[big])
    out[finite] = r
    return out


def momentum_update(M, G, beta, nesterov=False):
    """Momentum EMA in float64 with one float32 store; returns (M_new as float32, X0 bf16-valued).

    READING (the pages only say the FP32 momentum shard is updated locally and then cast
    to BF16 — notes page section 5 step 1; recipe page, "How to Make Parameter Updates
    Faster and More Stable?"): M <- beta*M + (1-beta)*G, and by default no Nesterov term.

    (1-beta) is formed in float32 as the library forms it.  Both products are exact in
    float64 (24-bit by 24-bit significands); the sum is rounded once to float64 and then
    once to float32.  G may hold float32 or bfloat16 values; both widen exactly.

    With nesterov=True the matrix handed on is the look-ahead N = beta*M_new + (1-beta)*G,
    formed the same way (float64 products and sum, one float32 rounding) and then cast;
    the returned momentum is M_new either way.  READING: the pages orthogonalise the
    momentum itself; the look-ahead is the common Muon variant, offered as an option.
    """
    b32 = np.float32(beta)
    omb32 = np.float32(1.0) - b32
    M64 = np.asarray(M, dtype=np.float32).astype(np.float64)
    G64 = np.asarray(G, dtype=np.float64)
    acc = np.float64(b32) * M64 + np.float64(omb32) * G64
    M_new = acc.astype(np.float32)
    if nesterov:
        N = (np.float64(b32) * M_new.astype(np.float64) + np.float64(omb32) * G64).astype(np.float32)
        return M_new, bf16_round(N.astype(np.float64))
    X0 = bf16_round(M_new.astype(np.float64))
    return M_new, X0


def canonical_orientation(rows: int, cols: int) -> bool:
    """True when the matrix is orthogonalised as its transpose.

    READING: the Gram matrix is formed on the short side, so a matrix with more rows than
    columns is transposed first (m = min(rows, cols), n = max(rows, cols)).
    """
    return rows > cols


def frobenius_normalise(X0, eps, emulate_bf16=True):
    """X = X0 / (||X0||_F + eps), rounded to bf16 in parity mode.

    READING: the pages give no normaliser; the Frobenius norm with eps added to the norm
    bounds every singular value of X by 1, where the quintic below is designed to act.
    The norm is summed in float64 over the bf16 values of X0.
    """
    X0 = np.asarray(X0, dtype=np.float64)
    nu = np.sqrt(np.sum(X0 * X0))
    inv = 1.0 / (nu + f32(eps)[()])
    X = X0 * inv
    return bf16_round(X) if emulate_bf16 else X


def ns_iterate(X, a, b, c, steps, emulate_bf16=True):
    """k quintic Newton–Schulz steps on an m x n matrix X (m <= n expected).

    Each step (notes page section 5 step 3: an NS operator built for the symmetric
    intermediates; Russian page: several matrix products in a row):
        A = X X^T            symmetric m x m
        B = b A + c A A      symmetric, since A is
        X = a X + B X
    so every singular value s of X maps to a s + b s^3 + c s^5.
    READING: the coefficients (a, b, c) and the step count are the caller's (the pages
    give none); the same (a, b, c) is used at every step.
    In parity mode A, B and the new X are each rounded once to bf16 from float64.
    """
    R = bf16_round if emulate_bf16 else (lambda v: v)
    a = f32(a)[()]
    b = f32(b)[()]
    c = f32(c)[()]
    X = np.asarray(X, dtype=np.float64)
    for _ in range(int(steps)):
        A = R(X @ X.T)
        B = R(b * A + c * (A @ A))
        X = R(a * X + B @ X)
    return X


def ns_iterate_schedule(X, coeffs, emulate_bf16=True):
    """Newton–Schulz steps with their own coefficients: coeffs = [(a_1, b_1, c_1), ...].

    Step t is the step of ns_iterate with (a_t, b_t, c_t), so every singular value s maps
    through p_t(s) = a_t s + b_t s^3 + c_t s^5 in turn.  READING: the pages fix no
    coefficients; a per-step schedule is offered next to the constant one.
    """
    R = bf16_round if emulate_bf16 else (lambda v: v)
    X = np.asarray(X, dtype=np.float64)
    for a, b, c in coeffs:
        a = f32(a)[()]
        b = f32(b)[()]
        c = f32(c)[()]
        A = R(X @ X.T)
        B = R(b * A + c * (A @ A))
        X = R(a * X + B @ X)
    return X


def newton_schulz_schedule(X0, coeffs, eps, emulate_bf16=True):
    """newton_schulz with a per-step coefficient schedule (orientation, normalisation, steps)."""
    X0 = np.asarray(X0, dtype=np.float64)
    if X0.ndim != 2:
        raise ValueError("Newton–Schulz takes 2-D matrices only")
    t = canonical_orientation(*X0.shape)
    Xc = X0.T if t else X0
    X = frobenius_normalise(Xc, eps, emulate_bf16)
    O = ns_iterate_schedule(X, coeffs, emulate_bf16)
    return O.T if t else O


def ns_iteration_rows(X, a, b, c, rows, emulate_bf16=True):
    """Selected rows of ONE Newton–Schulz step applied to X (m x n, m <= n expected).

    The same step as ns_iterate (A = X X^T, B = b A + c A A, X' = a X + B X, with the
    same cast points), evaluated only where it is needed for the requested rows of X':
    A in full (B's rows need all of A), then B's rows as b A[r] + c A[r] A, then
    X'[r] = a X[r] + B[r] X.  Row r of each product is the matching row of the full
    product, so the result equals ns_iterate(X, ..., steps=1)[rows].  Used to check an
    iteration of a matrix too large for the whole oracle chain, one iteration at a time.
    """
    R = bf16_round if emulate_bf16 else (lambda v: v)
    a = f32(a)[()]
    b = f32(b)[()]
    c = f32(c)[()]
    X = np.asarray(X, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    A = R(X @ X.T)
    Br = R(b * A[rows] + c * (A[rows] @ A))
    return R(a * X[rows] + Br @ X)


def newton_schulz(X0, a, b, c, steps, eps, emulate_bf16=True):
    """Orthogonalise one momentum matrix X0 (rows x cols, bf16 values in parity mode).

    Orientation, normalisation, then the iteration; the result is returned in the
    original rows x cols layout.
    """
    X0 = np.asarray(X0, dtype=np.float64)
    if X0.ndim != 2:
        raise ValueError("Newton–Schulz takes 2-D matrices only")
    t = canonical_orientation(*X0.shape)
    Xc = X0.T if t else X0
    X = frobenius_normalise(Xc, eps, emulate_bf16)
    O = ns_iterate(X, a, b, c, steps, emulate_bf16)
    return O.T if t else O


def apply_update(W, O, lr, wd, scale=1.0):
    """Decoupled weight decay and the scaled update, float64 math, one float32 store.

    READING (the pages fix the decay's time scale as 1/(LR*WD), a fixed fraction of
    training — notes page method section 3; recipe page "Small Models Must Also Undergo
    the 'Repeated Learning' of Large Models"): W <- (1 - lr*wd) W - lr*s*O, both terms
    from the old W.  Each operation below is a separate float64 rounding, in this order,
    with no fused multiply-add: d = 1 - lr*wd; u = lr*s; W = f32(d*W - u*O).
    lr*wd and lr*s are exact in float64 (products of two float32 values).
    """
    lr64 = f32(lr)[()]
    wd64 = f32(wd)[()]
    s64 = f32(scale)[()]
    d = 1.0 - lr64 * wd64
    u = lr64 * s64
    W64 = np.asarray(W, dtype=np.float32).astype(np.float64)
    O64 = np.asarray(O, dtype=np.float64)
    t1 = d * W64
    t2 = u * O64
    return (t1 - t2).astype(np.float32)


def update_scale(rule, rows, cols):
    """The update scale s_i of a shape rule, as the float32 value the library uses.

    READING (the pages give no rule; one notes that careful per-parameter update scaling
    mattered in the prior work it names, Russian page, section on Muon versus AdamW):
      "none"       s = 1
      "aspect"     s = sqrt(max(1, rows / cols))   (rows = outputs of the stored matrix)
      "rms_match"  s = 0.2 * sqrt(max(rows, cols)) (an update RMS near AdamW's)
    Each is evaluated in float64 and rounded once to float32.
    """
    r, c = float(rows), float(cols)
    if rule == "none":
        v = 1.0
    elif rule == "aspect":
        v = np.sqrt(max(1.0, r / c))
    elif rule == "rms_match":
        v = 0.2 * np.sqrt(max(r, c))
    else:
        raise ValueError(f"unknown update-scale rule {rule!r}")
    return float(np.float32(v))


def adamw_update(W, M, V, G, *, lr, beta1, beta2, eps, wd, step):
    """AdamW for the parameters the pages leave to it (embeddings, norms, scalars).

    The pages name AdamW as Muon's companion for the parameters that are not 2-D
    non-embedding matrices (notes page setup section 4; recipe page "How to Make Parameter
    Updates Faster and More Stable?") and give none of its settings.  READING: the usual
    AdamW with bias correction and decoupled decay, per element in float64 with each
    operation rounded once, in this order:
        m = f32(beta1*m + (1-beta1)*g)          (1-beta1) formed in float32
        v = f32(beta2*v + (1-beta2)*(g*g))
        bc1 = 1 - beta1^t,  bc2 = 1 - beta2^t   (float64, of the float32 betas)
        w = f32((1 - lr*wd)*w - (lr*(m/bc1)) / (sqrt(v/bc2) + eps))
    Returns (W, M, V) as float32.
    """
    lr64 = f32(lr)[()]
    wd64 = f32(wd)[()]
    b1 = np.float32(beta1)
    b2 = np.float32(beta2)
    omb1 = np.float64(np.float32(1.0) - b1)
    omb2 = np.float64(np.float32(1.0) - b2)
    b1 = np.float64(b1)
    b2 = np.float64(b2)
    eps64 = f32(eps)[()]
    bc1 = 1.0 - float(b1) ** int(step)
    bc2 = 1.0 - float(b2) ** int(step)
    g = np.asarray(G, dtype=np.float64)
    m = (b1 * np.asarray(M, dtype=np.float32).astype(np.float64) + omb1 * g).astype(np.float32)
    v = (b2 * np.asarray(V, dtype=np.float32).astype(np.float64) + omb2 * (g * g)).astype(np.float32)
    mhat = m.astype(np.float64) / bc1
    vhat = v.astype(np.float64) / bc2
    den = np.sqrt(vhat) + eps64
    upd = (lr64 * mhat) / den
    d = 1.0 - lr64 * wd64
    w = (d * np.asarray(W, dtype=np.float32).astype(np.float64) - upd).astype(np.float32)
    return w, m, v


def muon_step_ref(W, M, G, *, beta, a, b, c, steps, eps, lr, wd, scale=1.0,
                  emulate_bf16=True):
    """One whole Muon step for one 2-D parameter, in the pages' order.

    Returns a dict with the new weight W (float32), the new momentum M (float32), the
    bf16 momentum X0 (float64 holding bf16 values, rows x cols) and the update O
    (rows x cols; bf16 values in parity mode).
    """
    M_new, X0 = momentum_update(M, G, beta)
    O = newton_schulz(X0, a, b, c, steps, eps, emulate_bf16)
    W_new = apply_update(W, O, lr, wd, scale)
    return {"W": W_new, "M": M_new, "X0": X0, "O": O}
