"""Permuted block-diagonal inputs, for NS5 checks at sizes the oracle cannot
run whole (Muon section of the Modded-NanoGPT report: the quintic iteration).

For permutation matrices P, Q and G = P diag(G_1, ..., G_k) Q^T, every product
of the iteration keeps the block pattern: an entry of X X^T, A A or B X whose
row and column fall in different blocks is a sum of products that each have a
zero factor, so it is exactly zero, and the permutations only reorder rows and
columns (P X Q^T (P X Q^T)^T = P X X^T P^T).  Hence NS5(G) = P diag(O_1, ...,
O_k) Q^T, where O_k is block k iterated on its own but normalised by the norm
of the whole of G.  O_k is the leading block of NS5 of the augmented matrix
[[G_k, 0], [0, c_k]] with c_k^2 = ||G||_F^2 - ||G_k||_F^2: that matrix has G's
norm, and its extra 1 x 1 block never meets G_k.  The oracle runs that
augmented matrix at the block's size.
"""

import numpy as np


def permuted_block_diagonal(n, nblocks, seed):
    """G (n x n, float32) with nblocks Gaussian blocks of n / nblocks, block b
    scaled by 0.5 + b / nblocks, on rows rows[b] and columns cols[b] of two
    seeded permutations.  Returns (G, rows, cols, blocks)."""
    if n % nblocks:
        raise ValueError("n must be a multiple of nblocks")
    bs = n // nblocks
    rng = np.random.default_rng(seed)
    rows = rng.permutation(n).reshape(nblocks, bs)
    cols = rng.permutation(n).reshape(nblocks, bs)
    G = np.zeros((n, n), np.float32)
    blocks = []
    for b in range(nblocks):
        Gb = (rng.standard_normal((bs, bs)) * (0.5 + b / nblocks)).astype(np.float32)
        G[np.ix_(rows[b], cols[b])] = Gb
        blocks.append(Gb)
    return G, rows, cols, blocks


def augmented(blocks, b):
    """[[G_b, 0], [0, c_b]] with c_b^2 = sum of all blocks' squares - G_b's
    (float64 sums of the float32 values; c_b rounded once to float32)."""
    total = sum(float(np.sum(np.square(x, dtype=np.float64))) for x in blocks)
    own = float(np.sum(np.square(blocks[b], dtype=np.float64)))
    bs = blocks[b].shape[0]
    M = np.zeros((bs + 1, bs + 1), np.float32)
    M[:bs, :bs] = blocks[b]
    M[bs, bs] = np.float32(np.sqrt(total - own))
    return M


def off_block_is_zero(O, rows, cols):
    """True when every entry of O outside the blocks (rows[b], cols[b]) is
    zero (either sign): O has no more nonzeros than its blocks hold."""
    inside = sum(int(np.count_nonzero(O[np.ix_(r, c)])) for r, c in zip(rows, cols))
    return int(np.count_nonzero(O)) == inside
