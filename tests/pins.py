"""Checks that pin an NS5 implementation to facts fixed by the Muon section of
the Synced report on Modded-NanoGPT and by mathematics, independent of any
implementation.  Each check takes an ``ns5(G, steps=5, eps=1e-7)`` callable
and returns ``(ok, detail)``; the oracle must pass all of them and every
planted mistake must fail at least one.
"""

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "muon_section.txt")


def page_facts():
    vals = {}
    with open(GOLDEN, encoding="utf-8") as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split()
                vals[k] = float(v)
    return vals


def _f32(x):
    return float(np.float32(x))


def bf16_nearest_scalar(x):
    """Nearest bfloat16 to a Python float/Fraction x, ties to even, computed
    exactly: enumerate the two neighbours from the float32 bit pattern."""
    fx = Fraction(x)
    if fx == 0:
        return 0.0
    # bracket x between consecutive bf16 values using float64 arithmetic on
    # an exact truncation of x, then decide exactly with Fractions
    xf = float(fx)
    bits = int(np.array([xf], dtype=np.float32).view(np.uint32)[0]) & 0xFFFF0000
    cands = []
    for d in (-2, -1, 0, 1, 2):
        hb = ((bits >> 16) + d) & 0xFFFF
        v = np.array([hb << 16], dtype=np.uint32).view(np.float32)[0]
        if np.isfinite(v):
            cands.append((hb, float(v)))
    best = None
    for hb, v in cands:
        err = abs(Fraction(v) - fx)
        key = (err, hb & 1)          # smaller error, then even significand
        if best is None or key < best[0]:
            best = (key, v)
    return best[1]


def p_scalar(x, coeffs):
    a, b, c = coeffs
    return a * x + b * x ** 3 + c * x ** 5


def check_diagonal(ns5, shape=(6, 9), diag=(1.0, 0.5, 0.1, 0.01, 1e-3, 0.0)):
    """A diagonal G stays diagonal; each diagonal entry follows the scalar
    quintic with bf16 rounding at the stored values (A, B and X of every step),
    and lies within bf16 error of p applied 5 times to s_i / ||G||_F."""
    facts = page_facts()
    a, b, c = (_f32(facts[k]) for k in ("a", "b", "c"))
    eps = _f32(facts["eps"])
    k = min(shape)
    G = np.zeros(shape, dtype=np.float32)
    d = np.array(diag[:k], dtype=np.float32)
    G[np.arange(k), np.arange(k)] = d
    out = ns5(G, steps=5, eps=1e-7)
    off = out.copy()
    off[np.arange(k), np.arange(k)] = 0.0
    if np.any(off != 0):
        return False, "off-diagonal entries are not exactly zero"
    norm = float(np.sqrt(sum(float(v) ** 2 for v in d)))
    expect_round, expect_exact = [], []
    for si in d:
        x = bf16_nearest_scalar(Fraction(bf16_nearest_scalar(float(si))) / (Fraction(norm) + Fraction(eps)))
        xe = float(si) / (norm + 1e-7)
        for _ in range(5):
            A = bf16_nearest_scalar(Fraction(x) * Fraction(x))
            B = bf16_nearest_scalar(Fraction(b) * Fraction(A) + Fraction(c) * Fraction(A) * Fraction(A))
            x = bf16_nearest_scalar(Fraction(a) * Fraction(x) + Fraction(B) * Fraction(x))
            xe = p_scalar(xe, (a, b, c))
        expect_round.append(x)
        expect_exact.append(xe)
    got = out[np.arange(k), np.arange(k)].astype(np.float64)
    if not np.array_equal(got, np.array(expect_round)):
        return False, f"diagonal {got} != scalar bf16 recursion {expect_round}"
    if np.max(np.abs(got - np.array(expect_exact))) > 0.03:
        return False, f"diagonal {got} far from exact p^5 {expect_exact}"
    return True, ""


def check_transpose(ns5, seed=11, shape=(24, 40)):
    """NS5(G^T) == NS5(G)^T bitwise for a non-square G (the tall rule)."""
    rng = np.random.default_rng(seed)
    G = rng.standard_normal(shape).astype(np.float32)
    o1 = ns5(G)
    o2 = ns5(np.ascontiguousarray(G.T))
    if o1.shape != shape or o2.shape != shape[::-1]:
        return False, "output shape differs from input shape"
    if not np.array_equal(o2, o1.T):
        return False, "NS5(G^T) != NS5(G)^T"
    return True, ""


def check_sign_and_zero(ns5, seed=12, shape=(16, 24)):
    """p is odd and round-to-nearest-even is symmetric: NS5(-G) = -NS5(G)
    bitwise; G = 0 gives exactly 0 (eps keeps the division finite)."""
    rng = np.random.default_rng(seed)
    G = rng.standard_normal(shape).astype(np.float32)
    if not np.array_equal(ns5(-G), -ns5(G)):
        return False, "NS5(-G) != -NS5(G)"
    z = ns5(np.zeros(shape, dtype=np.float32))
    if not (np.all(z == 0) and np.all(np.isfinite(z))):
        return False, "NS5(0) != 0"
    return True, ""


def orthogonal_pair(rng, rows, cols):
    k = min(rows, cols)
    U, _ = np.linalg.qr(rng.standard_normal((rows, k)))
    V, _ = np.linalg.qr(rng.standard_normal((cols, k)))
    return U, V


def check_closed_form(ns5, seed=13, shape=(32, 48), lo=0.02, hi=1.0, tol_diag=0.03, tol_off=0.06):
    """For G = U diag(s) V^T, exact arithmetic gives
    NS5(G) = U diag(p^5(s / (||s||_2 + eps))) V^T, so U^T NS5(G) V must be
    nearly diagonal with that diagonal (bf16 noise aside)."""
    facts = page_facts()
    coeffs = tuple(_f32(facts[k]) for k in ("a", "b", "c"))
    rng = np.random.default_rng(seed)
    U, V = orthogonal_pair(rng, *shape)
    k = min(shape)
    s = np.exp(rng.uniform(np.log(lo), np.log(hi), k))
    G = ((U * s) @ V.T).astype(np.float32)
    out = ns5(G).astype(np.float64)
    if out.shape != shape:
        return False, "shape"
    s_hat = s / (np.linalg.norm(G.astype(np.float64)) + 1e-7)
    pred = s_hat.copy()
    for _ in range(5):
        pred = p_scalar(pred, coeffs)
    M = U.T @ out @ V
    dg = np.diag(M)
    offd = M - np.diag(dg)
    if np.max(np.abs(dg - pred)) > tol_diag:
        return False, f"diag of U^T O V off by {np.max(np.abs(dg - pred)):.3g}"
    rel_off = np.linalg.norm(offd) / np.linalg.norm(pred)
    if rel_off > tol_off:
        return False, f"off-diagonal mass {rel_off:.3g}"
    return True, ""


def check_square_closed_form(ns5, seed=14):
    """The closed form on a square input (no transpose rule involved)."""
    return check_closed_form(ns5, seed=seed, shape=(40, 40))


def check_tall_closed_form(ns5, seed=15):
    """The closed form on a tall input (iterated as its transpose)."""
    return check_closed_form(ns5, seed=seed, shape=(56, 24))


ALL_NS5_CHECKS = [check_diagonal, check_transpose, check_sign_and_zero, check_closed_form,
                  check_square_closed_form, check_tall_closed_form]
