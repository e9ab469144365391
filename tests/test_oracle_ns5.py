"""Pins for the oracle's NS5 (Muon section of the Synced report on
Modded-NanoGPT: the printed ``zeroth_power_via_newtonschulz5`` and the summary
paragraph after it).  The oracle must pass every check in ``pins``; planted
mistakes (in copies of the oracle, on the CPU) must each fail one."""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import jacobi_svd, ns5, round_bf16
from newton_schulz_09_amd import workloads

from . import pins


def test_constants_are_the_pages():
    facts = pins.page_facts()
    assert oracle.NS5_COEFFS == (facts["a"], facts["b"], facts["c"])
    assert oracle.NS5_STEPS == int(facts["steps"])
    assert oracle.NS5_EPS == facts["eps"]


def test_quintic_settles_in_the_pages_band():
    # Summary paragraph: repeated application lands in 0.68 .. 1.13, not at 1.
    facts = pins.page_facts()
    coeffs = tuple(float(np.float32(facts[k])) for k in ("a", "b", "c"))
    x = np.linspace(0.01, 1.0, 2000)
    for _ in range(60):
        x = pins.p_scalar(x, coeffs)
    lo, hi = facts["band_lo"], facts["band_hi"]
    # the page prints the band rounded to two decimals
    assert x.min() >= lo - 0.005 and x.max() <= hi + 0.005
    assert x.min() < lo + 0.01 and x.max() > hi - 0.01
    # p'(0) = a is the largest slope at zero among the listed coefficients
    assert abs(pins.p_scalar(1e-6, coeffs) / 1e-6 - coeffs[0]) < 1e-6


@pytest.mark.parametrize("check", pins.ALL_NS5_CHECKS, ids=lambda f: f.__name__)
def test_oracle_passes_pin(check):
    ok, detail = check(ns5)
    assert ok, detail


def test_output_is_bf16_valued_and_shaped():
    G = workloads.gaussian((20, 36), seed=5)
    out = ns5(G)
    assert out.dtype == np.float32 and out.shape == G.shape
    assert np.array_equal(round_bf16(out.astype(np.float64)), out.astype(np.float64))


def test_zero_steps_is_the_normalised_input():
    G = workloads.gaussian((20, 36), seed=6)
    out = ns5(G, steps=0).astype(np.float64)
    ref = G.astype(np.float64) / np.linalg.norm(G.astype(np.float64))
    assert np.max(np.abs(out - ref)) <= 2.0 ** -8 * np.max(np.abs(ref)) * 1.01
    assert abs(np.linalg.norm(out) - 1.0) < 1e-2


# ---------------------------------------------------------------------------
# Exact brute force on a tiny input: same rounding points, exact rationals.


def _bf16_mat(M):
    return [[Fraction(pins.bf16_nearest_scalar(v)) for v in row] for row in M]


_MACS = [0]   # multiply-adds performed by _matmul, for the flop-count pin


def _matmul(P, Q):
    _MACS[0] += len(P) * len(Q[0]) * len(Q)
    return [[sum(P[i][k] * Q[k][j] for k in range(len(Q))) for j in range(len(Q[0]))]
            for i in range(len(P))]


def _transpose(P):
    return [list(r) for r in zip(*P)]


def test_tiny_ns5_bitwise_against_exact_rationals():
    facts = pins.page_facts()
    a, b, c = (Fraction(float(np.float32(facts[k]))) for k in ("a", "b", "c"))
    eps = Fraction(float(np.float32(facts["eps"])))
    for shape, seed in (((3, 5), 21), ((5, 3), 22), ((4, 4), 23)):
        G = workloads.gaussian(shape, seed=seed)
        norm = Fraction(float(np.sqrt(sum(float(v) ** 2 for v in G.ravel().astype(np.float64)))))
        X = _bf16_mat([[pins.bf16_nearest_scalar(float(v)) for v in row] for row in G])
        X = _bf16_mat([[v / (norm + eps) for v in row] for row in X])
        tall = shape[0] > shape[1]
        if tall:
            X = _transpose(X)
        for _ in range(5):
            A = _bf16_mat(_matmul(X, _transpose(X)))
            AA = _matmul(A, A)
            B = _bf16_mat([[b * A[i][j] + c * AA[i][j] for j in range(len(A))] for i in range(len(A))])
            BX = _matmul(B, X)
            X = _bf16_mat([[a * X[i][j] + BX[i][j] for j in range(len(X[0]))] for i in range(len(X))])
        if tall:
            X = _transpose(X)
        want = np.array([[float(v) for v in row] for row in X], dtype=np.float32)
        assert np.array_equal(ns5(G), want), shape


def test_nominal_flops_count_the_brute_forces_multiply_adds():
    """oracle.ns5_nominal_flops is 2 flops per multiply-add of the plain
    products the iteration performs (X X^T, A A and B X in full, no symmetry
    used): counted here while the exact-rational brute force runs them, for
    wide, tall and square shapes and several step counts."""
    for shape, steps in (((3, 5), 5), ((5, 3), 5), ((4, 4), 2), ((2, 7), 3), ((7, 2), 1)):
        G = workloads.gaussian(shape, seed=1).astype(np.float64)
        X = [[Fraction(float(v)) for v in row] for row in (G if shape[0] <= shape[1] else G.T)]
        _MACS[0] = 0
        for _ in range(steps):
            A = _matmul(X, _transpose(X))
            B = _matmul(A, A)
            X = _matmul(B, X)
        assert 2 * _MACS[0] == oracle.ns5_nominal_flops(*shape, steps=steps), shape
    assert oracle.ns5_nominal_flops(768, 2304) == 5 * (4 * 768 ** 2 * 2304 + 2 * 768 ** 3)


# ---------------------------------------------------------------------------
# The SVD characterisation: NS5 approximately replaces G = U S V^T by U V^T.


def test_jacobi_svd_is_an_svd():
    rng = np.random.default_rng(7)
    for shape in ((6, 9), (9, 6), (7, 7)):
        M = rng.standard_normal(shape)
        U, s, Vt = jacobi_svd(M)
        np.testing.assert_allclose(U @ np.diag(s) @ Vt, M, atol=1e-12)
        np.testing.assert_allclose(U.T @ U, np.eye(len(s)), atol=1e-12)
        np.testing.assert_allclose(Vt @ Vt.T, np.eye(len(s)), atol=1e-12)
        assert np.all(np.diff(s) <= 0)
        # the singular values of a matrix are its Gram matrix's eigenvalues' roots
        ev = np.sort(np.linalg.eigvalsh(M @ M.T if shape[0] <= shape[1] else M.T @ M))[::-1]
        np.testing.assert_allclose(s ** 2, ev, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("shape,seed", [((8, 12), 31), ((12, 8), 32), ((10, 16), 33)])
def test_tiny_output_singular_vectors_match_polar_factor(shape, seed):
    """Singular vectors of NS5(G) are those of G (U V^T direction) and the
    singular values are p^5 of the normalised ones, inside the page's band
    wherever p^5 of the input lies there."""
    rng = np.random.default_rng(seed)
    k = min(shape)
    U0, V0 = pins.orthogonal_pair(rng, *shape)
    s0 = np.linspace(1.0, 0.15, k)              # normalised values stay in [0.04, 0.3]
    G = ((U0 * s0) @ V0.T).astype(np.float32)
    out = ns5(G).astype(np.float64)
    U, s, Vt = jacobi_svd(G.astype(np.float64))
    polar = U @ Vt
    cos = np.sum(out * polar) / (np.linalg.norm(out) * np.linalg.norm(polar))
    assert cos > 0.98
    M = U.T @ out @ Vt.T
    assert np.linalg.norm(M - np.diag(np.diag(M))) < 0.05 * np.linalg.norm(M)
    facts = pins.page_facts()
    _, so, _ = jacobi_svd(out)
    assert so.min() >= facts["band_lo"] - 0.015 and so.max() <= facts["band_hi"] + 0.015


def test_single_64x128_band_after_momentum():
    # 64x128 Gaussian gradient, momentum from a zero buffer, then NS5: every
    # singular value of the update lies in the page's band (bf16 noise aside).
    G, buf = workloads.single_64x128()
    _, u = oracle.momentum_nesterov(G, buf, 0.95)
    for M in (u, np.ascontiguousarray(u.T)):
        s = np.linalg.svd(ns5(M).astype(np.float64), compute_uv=False)
        assert s.min() > 0.67 and s.max() < 1.14


# ---------------------------------------------------------------------------
# Planted mistakes: each copy of the oracle below carries one plausible error
# and must fail at least one pin.


def _ns5_variant(G, steps=5, eps=1e-7, *, coeffs=oracle.NS5_COEFFS, gram="XXt", transpose_rule=True,
                 transpose_back=True, norm="fro", extra_step=0, bx_order="BX"):
    a, b, c = (float(np.float32(v)) for v in coeffs)
    u = G.astype(np.float64)
    d = np.sqrt(np.sum(u * u)) if norm == "fro" else np.max(np.abs(u))
    X = round_bf16(round_bf16(u) / (d + float(np.float32(eps))))
    tall = G.shape[0] > G.shape[1]
    if tall and transpose_rule:
        X = X.T
    for _ in range(steps + extra_step):
        A = round_bf16(X @ X.T if gram == "XXt" else X.T @ X)
        B = round_bf16(b * A + c * (A @ A))
        X = round_bf16(a * X + (B @ X if bx_order == "BX" else X @ B))
    if tall and transpose_rule and transpose_back:
        X = X.T
    return np.ascontiguousarray(X).astype(np.float32)


MUTANTS = {
    "b_sign_flipped": dict(coeffs=(3.4445, 4.7750, 2.0315)),
    "b_and_c_swapped": dict(coeffs=(3.4445, 2.0315, -4.7750)),
    "a_dropped": dict(coeffs=(1.0, -4.7750, 2.0315)),
    "gram_transposed": dict(gram="XtX"),
    "no_transpose_rule": dict(transpose_rule=False),
    "no_transpose_back": dict(transpose_back=False),
    "max_norm": dict(norm="max"),
    "one_step_more": dict(extra_step=1),
    "XB_instead_of_BX": dict(bx_order="XB"),
}


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    kw = MUTANTS[name]

    def mutant(G, steps=5, eps=1e-7):
        return _ns5_variant(G, steps, eps, **kw)

    failed = []
    for check in pins.ALL_NS5_CHECKS:
        try:
            ok, _ = check(mutant)
        except Exception:
            ok = False
        if not ok:
            failed.append(check.__name__)
    assert failed, f"no pin caught mutant {name}"


def test_unmutated_variant_passes_all_pins():
    # the harness itself is sound: the variant with no mistake passes
    for check in pins.ALL_NS5_CHECKS:
        ok, detail = check(lambda G, steps=5, eps=1e-7: _ns5_variant(G, steps, eps))
        assert ok, (check.__name__, detail)


def test_grouped_is_each_matrix_alone():
    """oracle.ns5_grouped returns, in order, each matrix's own NS5 (the
    matrices of a group are independent), with the steps and coefficients
    passed through."""
    Gs = [workloads.gaussian(s, seed=k) for k, s in enumerate([(3, 5), (5, 3), (4, 4), (3, 5)])]
    for kw in ({}, {"steps": 2}, {"steps": 3, "coeffs": (1.5, -0.5, 0.0)}):
        got = oracle.ns5_grouped(Gs, **kw)
        assert len(got) == len(Gs)
        for G, o in zip(Gs, got):
            assert np.array_equal(o, ns5(G, **kw))
    assert not np.array_equal(oracle.ns5_grouped(Gs)[0], oracle.ns5_grouped(Gs)[3])
