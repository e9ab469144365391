"""CPU oracle for the Muon optimizer's hot path: Nesterov momentum, then quintic
Newton-Schulz orthogonalisation (NS5) run in bfloat16.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The GPU
library shares no code with it and never calls it.

Source: Synced (机器之心) report on Modded-NanoGPT, section "Muon optimizer":
  * the printed function ``zeroth_power_via_newtonschulz5(G, steps=5, eps=1e-7)``
    fixes the coefficients (a, b, c) = (3.4445, -4.7750, 2.0315), the
    normalisation by the Frobenius norm plus eps, the bf16 cast, the rule that
    a matrix with more rows than columns is iterated as its transpose, the
    three products per step, and the output dtype (the input's);
  * the summary paragraph that follows says momentum is Nesterov's and that
    orthogonalisation comes after it, and that the iteration runs in bfloat16.

Arithmetic contract (where the section is silent, the plainest reading the
rest of it supports):
  * every sum and product is carried in float64 (exact for the bf16 x bf16
    products, ~1e-16 relative for the sums);
  * a value is rounded straight from float64 to bfloat16 (round to nearest,
    ties to even; no detour through float32) at exactly the points where the
    GPU stores bf16: the scaled input X0, and A, B and X of every step;
  * momentum rounds each of its two results once to float32.

The one deliberate library primitive is ``numpy.matmul`` in float64, used as
the plain definition of a matrix product (sum over the shared index).
"""

import numpy as np

#: Coefficients of the quintic p(x) = a*x + b*x**3 + c*x**5, as printed in the
#: Muon section's listing.  The GPU uses their float32 values; so does the
#: oracle (promoted exactly to float64).
NS5_COEFFS = (3.4445, -4.7750, 2.0315)
NS5_STEPS = 5
NS5_EPS = 1e-7

_BF16_MAX = float.fromhex("0x1.fep127")   # largest finite bfloat16, (2 - 2**-7) * 2**127
_BF16_MIN_QUANTUM_EXP = -133                 # spacing of bf16 subnormals is 2**-133


def f32(x):
    """The float32 value of ``x``, as a Python float (exact float64)."""
    return float(np.float32(x))


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 has float32's exponent range and an 8-bit significand (7 stored
    bits plus the implicit one), so a finite value x = m * 2**e with
    0.5 <= |m| < 1 is rounded to a multiple of 2**(e - 8), or of 2**-133 in the
    subnormal range.  Scaling by a power of two is exact, so ``rint`` (which
    rounds half to even) performs the single rounding.  Values whose rounded
    magnitude exceeds the largest finite bf16 become +-inf.  The result is
    returned as float64 holding bf16-representable values.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e - 8, _BF16_MIN_QUANTUM_EXP)
    with np.errstate(invalid="ignore", over="ignore"):
        r = np.ldexp(np.rint(np.ldexp(x, -q)), q)
        r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, x), r)
        r = np.where(np.isfinite(x), r, x)
    return r


def round_f32(x):
    """Round float64 values to the nearest float32 value, ties to even (the
    IEEE conversion), returned as float64 holding float32-representable
    values."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def momentum_nesterov(g, buf, mu=0.95):
    """One Nesterov-momentum step on a gradient.  The Muon section's summary
    paragraph names Nesterov momentum as part of the update and places the
    orthogonalisation after it; the update formula itself did not survive in
    the page, so the reading used is plain SGD-Nesterov without dampening:

        buf <- mu * buf + g
        u   <- g + mu * buf          (with the new buf)

    Each result is formed in float64 from float32 operands and rounded once to
    float32.  Returns ``(buf_new, u)`` as float32 arrays; inputs are untouched.
    """
    mu64 = f32(mu)
    g64 = np.asarray(g, dtype=np.float32).astype(np.float64)
    b64 = np.asarray(buf, dtype=np.float32).astype(np.float64)
    buf_new = (mu64 * b64 + g64).astype(np.float32)
    u = (g64 + mu64 * buf_new.astype(np.float64)).astype(np.float32)
    return buf_new, u


def _quintic_step(X, coeffs, rnd):
    """One step of the iteration on a short-side-first X (m <= n rows):

        X  <-  p(X X^T) X  with  p(S) = a I + b S + c S^2,

    which maps every singular value s of X to a s + b s^3 + c s^5 and keeps
    the singular vectors.  Three matrices are stored, each rounded once by
    ``rnd``: the Gram matrix S = X X^T, the polynomial part b S + c S S, and
    the new iterate a X + (b S + c S S) X.  Sums are carried in float64."""
    a, b, c = coeffs
    gram = rnd(X @ X.T)
    poly = rnd(b * gram + c * (gram @ gram))
    return rnd(a * X + poly @ X)


def ns5(G, steps=NS5_STEPS, eps=NS5_EPS, coeffs=NS5_COEFFS, precision="bf16"):
    """Quintic Newton-Schulz orthogonalisation of one 2-D matrix (Muon
    section, the printed zeroth_power_via_newtonschulz5):

      * scale: X = G / (||G||_F + eps), the norm of the float32 input taken in
        float64 and never rounded to bf16; in bf16 the input is cast before
        the division and the quotient rounded again (two roundings);
      * orientation: a matrix with more rows than columns is iterated as its
        transpose, so the Gram matrix is the smaller one, and transposed back
        at the end;
      * ``steps`` applications of ``_quintic_step``, whose stored matrices
        are rounded once each to bf16;
      * the result in float32 (G's dtype).

    Returns a float32 array of G's shape.

    ``precision="f32"``: the same iteration carried in float32 instead of
    bfloat16, the precision the summary paragraph contrasts with bf16 (it
    notes the iteration stays stable in bf16, unlike methods that need
    float32): there is no bf16 cast, X = G / (||G||_F + eps) is rounded once
    to float32, and every stored matrix of every step is rounded once to
    float32.
    """
    if precision not in ("bf16", "f32"):
        raise ValueError("precision is 'bf16' or 'f32'")
    G = np.asarray(G)
    if G.ndim != 2:
        raise ValueError("ns5 expects a 2-D matrix")
    k = tuple(f32(v) for v in coeffs)
    eps = f32(eps)
    u = G.astype(np.float32).astype(np.float64)
    denom = np.sqrt(np.sum(u * u)) + eps
    rnd = round_bf16 if precision == "bf16" else round_f32
    X = rnd(rnd(u) / denom) if precision == "bf16" else rnd(u / denom)
    tall = G.shape[0] > G.shape[1]
    W = X.T if tall else X
    for _ in range(steps):
        W = _quintic_step(W, k, rnd)
    out = W.T if tall else W
    return np.ascontiguousarray(out).astype(np.float32)


def ns5_grouped(Gs, steps=NS5_STEPS, eps=NS5_EPS, coeffs=NS5_COEFFS):
    """NS5 of each matrix in a list; the matrices are independent."""
    return [ns5(G, steps=steps, eps=eps, coeffs=coeffs) for G in Gs]


def muon_step(gs, bufs, mu=0.95, steps=NS5_STEPS, eps=NS5_EPS):
    """Momentum then NS5 for a list of gradient matrices (the order the Muon
    section's summary paragraph prescribes).  Returns ``(new_bufs, updates)``."""
    new_bufs, outs = [], []
    for g, buf in zip(gs, bufs):
        b, u = momentum_nesterov(g, buf, mu)
        new_bufs.append(b)
        outs.append(ns5(u, steps=steps, eps=eps))
    return new_bufs, outs


def apply_update(p, O, lr):
    """The parameter update that follows the orthogonalisation.  The Muon
    section's summary paragraph orders the step as momentum, then
    orthogonalisation, and the update uses the result; its formula did not
    survive in the page, so the reading is the plain one with a learning
    rate and no other scaling:

        p <- p - lr * O

    formed in float64 from float32 operands (lr * O is exact there for a
    bf16-valued O) and rounded once to float32, like the momentum.  Returns
    the new parameters as float32; inputs are untouched.
    """
    p64 = np.asarray(p, dtype=np.float32).astype(np.float64)
    O64 = np.asarray(O, dtype=np.float32).astype(np.float64)
    return (p64 - f32(lr) * O64).astype(np.float32)


def muon_step_apply(gs, bufs, ps, mu=0.95, lr=0.02, steps=NS5_STEPS, eps=NS5_EPS):
    """The whole Muon step with its update: momentum, NS5 of u, then
    ``p - lr * NS5(u)``.  Returns ``(new_bufs, new_params)``."""
    new_bufs, outs = muon_step(gs, bufs, mu=mu, steps=steps, eps=eps)
    return new_bufs, [apply_update(p, O, lr) for p, O in zip(ps, outs)]


def polar_factor(G, rank_tol=1e-6):
    """U V^T of G = U S V^T: the orthogonalisation the Muon section says NS5
    approximates (and calls too slow to compute through an SVD).  Written as
    its definition: the thin SVD of G in float64 (LAPACK through numpy, the
    library primitive here), keeping the singular values above ``rank_tol``
    times the largest; for a rank-deficient G the factor on the null space is
    not unique, and U_r V_r^T over the kept ones is the unique part.  G = 0
    gives 0.  Returns float32 of G's shape."""
    A = np.asarray(G, dtype=np.float32).astype(np.float64)
    if A.ndim != 2:
        raise ValueError("polar_factor expects a 2-D matrix")
    U, s, Vt = np.linalg.svd(A, full_matrices=False)
    if s.size == 0 or s[0] == 0.0:
        return np.zeros(A.shape, dtype=np.float32)
    keep = s > rank_tol * s[0]
    return (U[:, keep] @ Vt[keep]).astype(np.float32)


def ns5_nominal_flops(rows, cols, steps=NS5_STEPS):
    """Nominal NS5 flop count, 2 flops per multiply-add: per step the products
    X X^T (2 m^2 n), A A (2 m^3) and B X (2 m^2 n), with m <= n."""
    m, n = min(rows, cols), max(rows, cols)
    return steps * (4 * m * m * n + 2 * m ** 3)
