"""Pins of the CPU model of the GPU's U V^T through an SVD
(tests/svd_model.py): its pair schedule, its small eigensolver, and the
distance from the float64 oracle that float32 storage leaves it at on
Gaussian, ill-conditioned (singular values over three decades) and
rank-deficient inputs.  That distance (at most 2.4e-7 here) is the basis of
the GPU parity bar for this method, 1e-5."""

import numpy as np
import pytest

import oracle
from newton_schulz_09_amd import workloads

from . import parity, svd_model

#: The GPU parity bar of U V^T through the SVD (relative Frobenius against
#: oracle.polar_factor): more than 40 times the model's largest distance.
POLAR_TOL = 1e-5


@pytest.mark.parametrize("P", [2, 4, 6, 24, 48])
def test_round_robin_meets_every_pair_once(P):
    seen = set()
    for r in range(P - 1):
        i, j = svd_model.round_robin(P, r)
        assert len(set(i) | set(j)) == P          # disjoint, every player once
        seen |= {(a, b) for a, b in zip(i, j)}
        assert np.all(i < j)
    assert len(seen) == P * (P - 1) // 2


def test_diagonalise_gives_an_orthogonal_eigenbasis():
    rng = np.random.default_rng(1)
    A = rng.standard_normal((64, 300))
    M = A @ A.T
    R = svd_model.diagonalise(M)
    D = R @ M @ R.T
    assert np.max(np.abs(R @ R.T - np.eye(64))) < 1e-12
    assert np.max(np.abs(D - np.diag(np.diag(D)))) < 1e-10 * np.abs(D).max()
    assert np.allclose(np.sort(np.diag(D)), np.linalg.eigvalsh(M), rtol=1e-10)


def _inputs():
    rng = np.random.default_rng(9)
    U, _ = np.linalg.qr(rng.standard_normal((64, 64)))
    V, _ = np.linalg.qr(rng.standard_normal((160, 64)))
    s = np.exp(rng.uniform(np.log(1e-3), 0, 64))
    s2 = s.copy()
    s2[rng.permutation(64)[:16]] = 0.0
    return {"64x128": workloads.gaussian((64, 128), 1), "128x64": workloads.gaussian((128, 64), 2),
            "100x150": workloads.gaussian((100, 150), 3), "3x5": workloads.gaussian((3, 5), 4),
            "ill-conditioned": ((U * s) @ V.T).astype(np.float32),
            "rank-deficient": ((U * s2) @ V.T).astype(np.float32)}


@pytest.mark.parametrize("name", list(_inputs()))
def test_float32_storage_lands_near_the_oracle(name):
    G = _inputs()[name]
    Q, sweeps = svd_model.polar_svd(G)
    d = parity.rel_fro(Q, oracle.polar_factor(G))
    assert d <= 2.5e-7, (name, d)
    assert d * 40 <= POLAR_TOL
    assert sweeps <= 12
