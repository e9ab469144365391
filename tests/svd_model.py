"""A model of the GPU's U V^T through an SVD (block one-sided Jacobi with
float32 storage and float64 arithmetic), evaluated in numpy.

TEST INFRASTRUCTURE: it shares no code with the HIP library.  It follows the
same algorithm (blocks of 32 rows paired round-robin, each pair's 64 x 64
Gram matrix diagonalised by cyclic Jacobi and applied to the pair's rows of
[W | J], rows rounded to float32 after every application, the same
tolerances) so that the distance it lands from the float64 oracle pins, on
the CPU, what float32 storage costs this method; that distance is what the
GPU parity bar of the method is set against.
"""

import numpy as np

ROWS_PER_BLOCK = 32
TOL = 1e-6
RANK_TOL = 1e-6


def round_robin(P, r):
    """Round r (0 .. P-2) of the circle method on P players: P/2 disjoint
    pairs (i < j); over P - 1 rounds every two players meet once."""
    ks = np.arange(1, P // 2)
    a, b = (r + ks) % (P - 1), (r - ks + (P - 1)) % (P - 1)
    return np.concatenate([[r], np.minimum(a, b)]), np.concatenate([[P - 1], np.maximum(a, b)])


def diagonalise(M, max_sweeps=16):
    """R with R M R^T diagonal, by cyclic Jacobi in rounds of disjoint
    rotations (row_p <- c row_p - s row_q, row_q <- s row_p + c row_q)."""
    M = M.copy()
    n = M.shape[0]
    R = np.eye(n)
    iu = np.triu_indices(n, 1)
    for _ in range(max_sweeps):
        for r in range(n - 1):
            p, q = round_robin(n, r)
            mpq, mpp, mqq = M[p, q], M[p, p], M[q, q]
            rot = (np.abs(mpq) > 1e-300) & (np.abs(mpq) > 1e-17 * np.sqrt(np.abs(mpp * mqq)))
            tau = np.where(rot, (mqq - mpp) / np.where(rot, 2.0 * mpq, 1.0), 0.0)
            t = np.where(tau >= 0, 1.0, -1.0) / (np.abs(tau) + np.sqrt(1.0 + tau * tau))
            c = np.where(rot, 1.0 / np.sqrt(1.0 + t * t), 1.0)
            s = np.where(rot, t * c, 0.0)
            for A in (M, R):
                ap, aq = A[p].copy(), A[q].copy()
                A[p] = c[:, None] * ap - s[:, None] * aq
                A[q] = s[:, None] * ap + c[:, None] * aq
            mp, mq = M[:, p].copy(), M[:, q].copy()
            M[:, p] = mp * c - mq * s
            M[:, q] = mp * s + mq * c
        d = np.sqrt(np.abs(np.outer(np.diag(M), np.diag(M))))[iu]
        off = np.abs(M[iu])
        ratio = np.where(d > 0, off / np.where(d > 0, d, 1.0), np.where(off > 1e-300, 1.0, 0.0))
        if ratio.max() <= 1e-15:
            break
    return R


def polar_svd(G, max_sweeps=12):
    """U V^T of G by the GPU's method; returns (float32 Q, sweeps run)."""
    G = np.asarray(G, dtype=np.float32)
    tall = G.shape[0] > G.shape[1]
    W0 = G.T if tall else G
    m, n = W0.shape
    m_pad = -(-max(m, 64) // 64) * 64
    n_pad = -(-n // 64) * 64
    P = m_pad // ROWS_PER_BLOCK
    WJ = np.zeros((m_pad, n_pad + m_pad), dtype=np.float32)
    WJ[:m, :n] = W0
    WJ[:, n_pad:] = np.eye(m_pad, dtype=np.float32)
    iu = np.triu_indices(2 * ROWS_PER_BLOCK, 1)
    sweeps = 0
    for _ in range(max_sweeps):
        sweeps += 1
        rotated = 0
        for r in range(P - 1):
            bi, bj = round_robin(P, r)
            for i, j in zip(bi, bj):
                rows = np.r_[i * ROWS_PER_BLOCK:(i + 1) * ROWS_PER_BLOCK, j * ROWS_PER_BLOCK:(j + 1) * ROWS_PER_BLOCK]
                Wp = WJ[rows, :n_pad].astype(np.float64)
                M = Wp @ Wp.T
                d = np.sqrt(np.outer(np.diag(M), np.diag(M)))[iu]
                worst = np.max(np.where(d > 0, np.abs(M[iu]) / np.where(d > 0, d, 1.0), 0.0))
                if worst <= TOL:
                    continue
                rotated += 1
                R = diagonalise(M)
                WJ[rows] = (R @ WJ[rows].astype(np.float64)).astype(np.float32)
        if rotated == 0:
            break
    lens = np.sqrt(np.sum(WJ[:, :n_pad].astype(np.float64) ** 2, axis=1))
    inv = np.where((lens > 0) & (lens > RANK_TOL * lens.max()), 1.0 / np.where(lens > 0, lens, 1.0), 0.0)
    N = (inv[:, None] * WJ[:, :n_pad].astype(np.float64)).astype(np.float32).astype(np.float64)
    Q = (WJ[:, n_pad:].astype(np.float64).T @ N)[:m, :n]
    return (Q.T if tall else Q).astype(np.float32), sweeps
