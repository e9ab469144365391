"""Pins of oracle.polar_factor, U V^T of G = U S V^T: the orthogonalisation
the Muon section (Synced report on Modded-NanoGPT) says NS5 approximates.
Pinned against an independent SVD (the oracle's one-sided Jacobi, no
LAPACK), the defining properties of the polar decomposition, closed forms,
invariances, the classic cubic Newton-Schulz iteration (which converges to
it) and planted mistakes."""

import numpy as np
import pytest

import oracle
from oracle import jacobi_svd, polar_factor
from newton_schulz_09_amd import workloads


def _orthonormal(rng, n, k):
    q, _ = np.linalg.qr(rng.standard_normal((n, k)))
    return q


def test_matches_the_independent_jacobi_svd():
    for shape, seed in (((3, 5), 1), ((5, 3), 2), ((6, 6), 3), ((4, 9), 4)):
        G = workloads.gaussian(shape, seed=seed)
        U, s, Vt = jacobi_svd(G.astype(np.float64))
        want = U @ Vt
        assert np.max(np.abs(polar_factor(G).astype(np.float64) - want)) < 1e-6, shape


@pytest.mark.parametrize("shape", [(16, 40), (40, 16), (24, 24)])
def test_defining_properties(shape):
    """For full-rank G: Q has orthonormal rows (or columns, when tall) and
    G Q^T (or Q^T G) is symmetric positive definite - the polar decomposition,
    which fixes Q uniquely."""
    G = workloads.gaussian(shape, seed=sum(shape)).astype(np.float64)
    Q = polar_factor(G).astype(np.float64)
    m = min(shape)
    if shape[0] <= shape[1]:
        gram, H = Q @ Q.T, G @ Q.T
    else:
        gram, H = Q.T @ Q, Q.T @ G
    assert np.max(np.abs(gram - np.eye(m))) < 1e-6
    assert np.max(np.abs(H - H.T)) < 1e-5 * np.abs(H).max()
    assert np.linalg.eigvalsh((H + H.T) / 2).min() > 0


def test_closed_form_and_rank_deficiency():
    rng = np.random.default_rng(5)
    U, V = _orthonormal(rng, 20, 12), _orthonormal(rng, 50, 12)
    s = np.exp(rng.uniform(np.log(1e-3), 0, 12))
    G = (U * s) @ V.T
    assert np.max(np.abs(polar_factor(G) - U @ V.T)) < 1e-5
    s[[1, 4, 7]] = 0.0                       # rank 9: U_r V_r^T over the nonzero ones
    G = (U * s) @ V.T
    keep = s > 0
    assert np.max(np.abs(polar_factor(G) - U[:, keep] @ V[:, keep].T)) < 1e-5
    assert not polar_factor(np.zeros((3, 4))).any()


def test_invariances():
    rng = np.random.default_rng(6)
    G = rng.standard_normal((12, 30))
    Q = polar_factor(G).astype(np.float64)
    O = _orthonormal(rng, 12, 12)
    assert np.max(np.abs(polar_factor(G.T) - Q.T)) < 1e-6           # transpose
    assert np.max(np.abs(polar_factor(-G) + Q)) < 1e-6              # odd
    assert np.max(np.abs(polar_factor(3.5 * G) - Q)) < 1e-6         # scale-free
    assert np.max(np.abs(polar_factor(O @ G) - O @ Q)) < 1e-5       # left orthogonal equivariance


def test_cubic_newton_schulz_converges_to_it():
    """The classic cubic iteration X <- 1.5 X - 0.5 X X^T X, which NS5's
    quintic was tuned away from, converges to U V^T (float32 iteration of the
    oracle, many steps)."""
    G = workloads.gaussian((24, 48), seed=7)
    X = oracle.ns5(G, steps=60, coeffs=(1.5, -0.5, 0.0), precision="f32")
    assert np.max(np.abs(X - polar_factor(G))) < 1e-4


@pytest.mark.parametrize("mistake", ["no_transpose_back", "keep_sigma", "full_null_space"])
def test_pins_catch_planted_mistakes(mistake):
    rng = np.random.default_rng(8)
    G = rng.standard_normal((10, 6))          # tall
    U, s, Vt = np.linalg.svd(G, full_matrices=False)
    if mistake == "no_transpose_back":
        bad = (U @ Vt).T.copy()
        ok = bad.shape == G.shape and np.allclose(bad, polar_factor(G), atol=1e-5)
    elif mistake == "keep_sigma":
        bad = U @ np.diag(s / s.max()) @ Vt
        ok = np.allclose(bad, polar_factor(G), atol=1e-5)
    else:                                      # rank-deficient G, null space kept
        s2 = s.copy()
        s2[-2:] = 0.0
        G2 = (U * s2) @ Vt
        bad = U @ Vt
        ok = np.allclose(bad, polar_factor(G2), atol=1e-5)
    assert not ok
