"""Pins of the oracle's iteration with coefficients other than NS5's (the
variants the Muon section of the Synced report on Modded-NanoGPT implies when
it explains its quintic as coefficients chosen for the slope at zero, which
settle in a band instead of converging to 1): the classic cubic
Newton-Schulz iteration (a, b, c) = (1.5, -0.5, 0) and degenerate
coefficient sets whose result is known exactly."""

from fractions import Fraction

import numpy as np
import pytest

import oracle

from . import pins

CUBIC = (1.5, -0.5, 0.0)


def _scalar_recursion(s, norm, eps, coeffs, steps):
    """The iteration on one diagonal entry, with the bf16 rounding of every
    stored value (X0, A, B and each new X) done exactly with fractions."""
    a, b, c = (Fraction(float(np.float32(v))) for v in coeffs)
    x = pins.bf16_nearest_scalar(Fraction(pins.bf16_nearest_scalar(float(s))) / (Fraction(norm) + Fraction(eps)))
    for _ in range(steps):
        A = pins.bf16_nearest_scalar(Fraction(x) * Fraction(x))
        B = pins.bf16_nearest_scalar(b * Fraction(A) + c * Fraction(A) * Fraction(A))
        x = pins.bf16_nearest_scalar(a * Fraction(x) + Fraction(B) * Fraction(x))
    return x


@pytest.mark.parametrize("coeffs,steps", [(CUBIC, 8), ((2.0, -1.5, 0.5), 3), (oracle.NS5_COEFFS, 5)])
def test_diagonal_follows_the_scalar_recursion(coeffs, steps):
    d = np.array([1.0, 0.5, 0.1, 0.01, 1e-3, 0.0], dtype=np.float32)
    G = np.zeros((6, 9), dtype=np.float32)
    G[np.arange(6), np.arange(6)] = d
    out = oracle.ns5(G, steps=steps, coeffs=coeffs)
    off = out.copy()
    off[np.arange(6), np.arange(6)] = 0
    assert not np.any(off)
    norm = float(np.sqrt(sum(float(v) ** 2 for v in d)))
    want = [_scalar_recursion(s, norm, float(np.float32(1e-7)), coeffs, steps) for s in d]
    assert np.array_equal(out[np.arange(6), np.arange(6)].astype(np.float64), np.array(want))


def test_cubic_converges_to_the_polar_factor():
    """G = U diag(s) V^T with s in [0.2, 1]: the cubic's singular values
    converge to 1 (bf16 noise aside), so enough steps give U V^T."""
    rng = np.random.default_rng(3)
    U, V = pins.orthogonal_pair(rng, 32, 48)
    s = np.linspace(1.0, 0.2, 32)
    G = ((U * s) @ V.T).astype(np.float32)
    out = oracle.ns5(G, steps=14, coeffs=CUBIC).astype(np.float64)
    polar = U @ V.T
    assert np.linalg.norm(out - polar) / np.linalg.norm(polar) < 2e-2
    sv = np.linalg.svd(out, compute_uv=False)
    assert np.max(np.abs(sv - 1.0)) < 2e-2
    # the quintic's five steps settle in a band around 1 instead
    q = np.linalg.svd(oracle.ns5(G).astype(np.float64), compute_uv=False)
    assert np.max(np.abs(q - 1.0)) > 0.1


def test_identity_coefficients_return_the_normalised_input():
    rng = np.random.default_rng(4)
    G = rng.standard_normal((20, 33)).astype(np.float32)
    for Gi in (G, np.ascontiguousarray(G.T)):
        assert np.array_equal(oracle.ns5(Gi, steps=4, coeffs=(1.0, 0.0, 0.0)), oracle.ns5(Gi, steps=0))


def test_a_alone_scales_exactly():
    """(2, 0, 0): every step doubles X exactly (a power of two), so k steps
    give 2^k times the normalised input: a multiplies X, not A or B."""
    rng = np.random.default_rng(5)
    G = rng.standard_normal((17, 29)).astype(np.float32)
    assert np.array_equal(oracle.ns5(G, steps=3, coeffs=(2.0, 0.0, 0.0)), 8 * oracle.ns5(G, steps=0))
