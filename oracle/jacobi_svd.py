"""One-sided (Hestenes) Jacobi SVD for tiny matrices, in float64.

TEST INFRASTRUCTURE ONLY (same import rule as ``muon_oracle``).

The Muon section (Synced report on Modded-NanoGPT) characterises NS5 by the
SVD: it approximately replaces G = U S V^T with U V^T.  The tests check the
oracle's output against that characterisation with this brute-force SVD, which
is independent of LAPACK: it rotates pairs of columns until all of them are
mutually orthogonal, so the column norms are the singular values.
"""

import numpy as np


def jacobi_svd(M, tol=1e-15, max_sweeps=60):
    """Thin SVD ``M = U @ diag(s) @ Vt`` of a small real matrix.

    Works on the orientation with at least as many rows as columns; the
    columns of W = M V are rotated pairwise (plane rotations chosen to zero
    their inner product) until every pair is orthogonal to ``tol``.
    Singular values come back sorted in decreasing order.  Zero singular
    values get an arbitrary unit left vector completed by Gram-Schmidt.
    """
    M = np.array(M, dtype=np.float64)
    flip = M.shape[0] < M.shape[1]
    W = M.T.copy() if flip else M.copy()
    rows, k = W.shape
    V = np.eye(k)
    for _ in range(max_sweeps):
        off = 0.0
        for p in range(k - 1):
            for q in range(p + 1, k):
                alpha = W[:, p] @ W[:, p]
                beta = W[:, q] @ W[:, q]
                gamma = W[:, p] @ W[:, q]
                if gamma == 0.0:
                    continue
                off = max(off, abs(gamma) / np.sqrt(alpha * beta))
                zeta = (beta - alpha) / (2.0 * gamma)
                t = np.sign(zeta) / (abs(zeta) + np.sqrt(1.0 + zeta * zeta)) if zeta != 0 else 1.0
                cs = 1.0 / np.sqrt(1.0 + t * t)
                sn = cs * t
                wp, wq = W[:, p].copy(), W[:, q].copy()
                W[:, p] = cs * wp - sn * wq
                W[:, q] = sn * wp + cs * wq
                vp, vq = V[:, p].copy(), V[:, q].copy()
                V[:, p] = cs * vp - sn * vq
                V[:, q] = sn * vp + cs * vq
        if off < tol:
            break
    s = np.sqrt(np.sum(W * W, axis=0))
    order = np.argsort(-s)
    s, W, V = s[order], W[:, order], V[:, order]
    U = np.zeros((rows, k))
    for j in range(k):
        if s[j] > 1e-300 and s[j] > 1e-12 * s[0]:
            U[:, j] = W[:, j] / s[j]
        else:
            # complete an orthonormal basis for a (numerically) zero direction
            v = np.zeros(rows)
            for trial in range(rows):
                v[:] = 0.0
                v[(j + trial) % rows] = 1.0
                v -= U[:, :j] @ (U[:, :j].T @ v)
                if np.linalg.norm(v) > 1e-6:
                    break
            U[:, j] = v / np.linalg.norm(v)
    if flip:
        return V, s, U.T
    return U, s, V.T
