"""Pins of the oracle's float32 iteration (``ns5(..., precision="f32")``): the
same steps as the printed zeroth_power_via_newtonschulz5 of the Muon section
(Synced report on Modded-NanoGPT) carried in float32 instead of bfloat16, the
contrast its summary paragraph draws.  Pinned against exact rational
arithmetic, the scalar recursion on diagonal inputs, the closed form
U p^5(S / (||G|| + eps)) V^T, the transpose and sign invariants, and planted
mistakes."""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from newton_schulz_09_amd import workloads

from . import pins


def f32_nearest_scalar(x):
    """Nearest float32 to a Python float/Fraction x, ties to even, decided
    exactly: the candidates are float32 neighbours of a float64 approximation."""
    fx = Fraction(x)
    if fx == 0:
        return 0.0
    v = np.float32(float(fx))
    cands = {float(v), float(np.nextafter(v, np.float32(np.inf))), float(np.nextafter(v, np.float32(-np.inf)))}
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        bits = int(np.array([c], dtype=np.float32).view(np.uint32)[0])
        key = (abs(Fraction(c) - fx), bits & 1)   # nearer, then even significand
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def ns5_f32(G, **kw):
    return oracle.ns5(G, precision="f32", **kw)


def _coeffs():
    facts = pins.page_facts()
    return tuple(Fraction(float(np.float32(facts[k]))) for k in ("a", "b", "c")), \
        Fraction(float(np.float32(facts["eps"])))


def _mat(M):
    return [[f32_nearest_scalar(v) for v in row] for row in M]


def _mm(P, Q):
    return [[sum(Fraction(P[i][k]) * Fraction(Q[k][j]) for k in range(len(Q))) for j in range(len(Q[0]))]
            for i in range(len(P))]


def _t(P):
    return [list(r) for r in zip(*P)]


def test_f32_rounding_helper():
    assert f32_nearest_scalar(Fraction(1, 3)) == float(np.float32(1 / 3))
    # a tie between 1 and 1 + 2^-23 goes to the even significand (1)
    assert f32_nearest_scalar(Fraction(1) + Fraction(1, 2 ** 24)) == 1.0
    assert f32_nearest_scalar(Fraction(1) + Fraction(3, 2 ** 24)) == 1.0 + 2.0 ** -22


def test_tiny_bitwise_against_exact_rationals():
    """Every product and sum exact (fractions), one rounding to float32 at each
    stored matrix: X0, and A, B and X of every step."""
    (a, b, c), eps = _coeffs()
    for shape, seed in (((3, 5), 21), ((5, 3), 22), ((4, 4), 23)):
        G = workloads.gaussian(shape, seed=seed)
        norm = Fraction(float(np.sqrt(sum(float(v) ** 2 for v in G.ravel().astype(np.float64)))))
        X = _mat([[Fraction(float(v)) / (norm + eps) for v in row] for row in G])
        tall = shape[0] > shape[1]
        if tall:
            X = _t(X)
        for _ in range(5):
            A = _mat(_mm(X, _t(X)))
            AA = _mm(A, A)
            B = _mat([[b * Fraction(A[i][j]) + c * AA[i][j] for j in range(len(A))] for i in range(len(A))])
            BX = _mm(B, X)
            X = _mat([[a * Fraction(X[i][j]) + BX[i][j] for j in range(len(X[0]))] for i in range(len(X))])
        if tall:
            X = _t(X)
        want = np.array(X, dtype=np.float32)
        assert np.array_equal(ns5_f32(G), want), shape


def test_diagonal_follows_the_scalar_recursion():
    (a, b, c), eps = _coeffs()
    d = np.array([1.0, 0.5, 0.1, 0.01, 1e-3, 0.0], dtype=np.float32)
    G = np.zeros((6, 9), dtype=np.float32)
    G[np.arange(6), np.arange(6)] = d
    out = ns5_f32(G)
    off = out.copy()
    off[np.arange(6), np.arange(6)] = 0
    assert not np.any(off)
    norm = Fraction(float(np.sqrt(sum(float(v) ** 2 for v in d))))
    want = []
    for s in d:
        x = f32_nearest_scalar(Fraction(float(s)) / (norm + eps))
        for _ in range(5):
            A = f32_nearest_scalar(Fraction(x) * Fraction(x))
            B = f32_nearest_scalar(b * Fraction(A) + c * Fraction(A) * Fraction(A))
            x = f32_nearest_scalar(a * Fraction(x) + Fraction(B) * Fraction(x))
        want.append(x)
    assert np.array_equal(out[np.arange(6), np.arange(6)].astype(np.float64), np.array(want))


def _p5(x):
    a, b, c = (float(np.float32(v)) for v in oracle.NS5_COEFFS)
    for _ in range(5):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


@pytest.mark.parametrize("shape", [(32, 48), (40, 40), (48, 32)])
def test_closed_form(shape):
    """For G = U diag(s) V^T the exact iteration gives U diag(p^5(s / (||s|| +
    eps))) V^T.  Carried in float32 the result stays within float32 rounding
    of it (measured 1.1e-6), far inside the bf16 iteration's distance
    (6e-2 .. 9e-2 on the same inputs)."""
    rng = np.random.default_rng(3)
    m, n = shape
    k = min(m, n)
    U, V = pins.orthogonal_pair(rng, m, n) if m <= n else pins.orthogonal_pair(rng, n, m)[::-1]
    s = np.exp(rng.uniform(np.log(1e-3), 0, k))
    G = ((U[:, :k] * s) @ V[:, :k].T).astype(np.float32)
    Uu, ss, Vt = np.linalg.svd(G.astype(np.float64), full_matrices=False)
    sh = ss / (np.linalg.norm(G.astype(np.float64)) + float(np.float32(1e-7)))
    want = (Uu * _p5(sh)) @ Vt
    got = ns5_f32(G).astype(np.float64)
    assert np.linalg.norm(got - want) / np.linalg.norm(want) < 1e-5
    assert np.max(np.abs(np.linalg.svd(got, compute_uv=False) - np.sort(_p5(sh))[::-1])) < 1e-5


@pytest.mark.parametrize("check", [pins.check_transpose, pins.check_sign_and_zero])
def test_invariants(check):
    ok, detail = check(ns5_f32)
    assert ok, detail


def test_differs_from_the_bf16_iteration_by_bf16_error():
    G, _ = workloads.single_64x128()
    r = np.linalg.norm(ns5_f32(G).astype(np.float64) - oracle.ns5(G).astype(np.float64)) / \
        np.linalg.norm(ns5_f32(G).astype(np.float64))
    assert 1e-3 < r < 5e-2


def test_steps_zero_is_the_normalised_input():
    G = workloads.gaussian((7, 5), seed=8)
    u = G.astype(np.float64)
    want = (u / (np.sqrt(np.sum(u * u)) + float(np.float32(1e-7)))).astype(np.float32)
    assert np.array_equal(ns5_f32(G, steps=0), want)


def _mutant(kind):
    """Copies of the float32 iteration with one planted mistake each."""
    a, b, c = (float(np.float32(v)) for v in oracle.NS5_COEFFS)

    def f(G, steps=5, eps=1e-7):
        u = G.astype(np.float64)
        X = u / (np.sqrt(np.sum(u * u)) + float(np.float32(eps)))
        if kind == "bf16_input":
            X = oracle.round_bf16(oracle.round_bf16(u) / (np.sqrt(np.sum(u * u)) + float(np.float32(eps))))
        X = oracle.round_f32(X)
        tall = G.shape[0] > G.shape[1]
        if tall:
            X = X.T
        for _ in range(steps):
            A = oracle.round_f32(X @ X.T)
            B = oracle.round_f32(b * A + c * (A @ A))
            if kind == "no_b":
                X = oracle.round_f32(a * X + oracle.round_f32(c * (A @ A)) @ X)
            else:
                X = oracle.round_f32(a * X + B @ X)
        if tall:
            X = X.T
        return np.ascontiguousarray(X).astype(np.float32)
    return f


@pytest.mark.parametrize("kind", ["bf16_input", "no_b"])
def test_pins_catch_planted_mistakes(kind):
    f = _mutant(kind)
    rng = np.random.default_rng(3)
    U, V = pins.orthogonal_pair(rng, 32, 48)
    s = np.exp(rng.uniform(np.log(1e-3), 0, 32))
    G = ((U * s) @ V.T).astype(np.float32)
    Uu, ss, Vt = np.linalg.svd(G.astype(np.float64), full_matrices=False)
    sh = ss / (np.linalg.norm(G.astype(np.float64)) + float(np.float32(1e-7)))
    want = (Uu * _p5(sh)) @ Vt
    with np.errstate(all="ignore"):   # a mutant may diverge to inf / nan
        got = f(G).astype(np.float64)
        r = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert not r < 1e-5


def test_unmutated_copy_agrees():
    G = workloads.gaussian((24, 40), seed=4)
    assert np.array_equal(_mutant("none")(G), ns5_f32(G))
