"""The permuted block-diagonal construction (tests/blockdiag.py) against the
oracle run whole, at a size it finishes at once: NS5 of the whole matrix is
zero off the blocks and, on block b, NS5 of the augmented matrix for b.  The
GPU checks at the largest accepted short side rest on this."""

import numpy as np

import oracle

from . import blockdiag, parity


def test_whole_matrix_equals_augmented_blocks():
    G, rows, cols, blocks = blockdiag.permuted_block_diagonal(96, 3, seed=5)
    O = oracle.ns5(G)
    assert blockdiag.off_block_is_zero(O, rows, cols)
    for b in range(3):
        Ob = oracle.ns5(blockdiag.augmented(blocks, b))[:32, :32]
        got = O[np.ix_(rows[b], cols[b])]
        assert parity.rel_fro(got, Ob) <= 1e-3, b
    # the normalisation by the whole of G matters: block 0 iterated with its
    # own norm is far off
    assert parity.rel_fro(O[np.ix_(rows[0], cols[0])], oracle.ns5(blocks[0])) > 0.05


def test_off_block_check_sees_a_stray_entry():
    G, rows, cols, _ = blockdiag.permuted_block_diagonal(64, 4, seed=6)
    assert blockdiag.off_block_is_zero(G, rows, cols)
    r, c = rows[0][0], cols[1][0]
    G[r, c] = 1e-30
    assert not blockdiag.off_block_is_zero(G, rows, cols)


def test_whole_matrix_equals_augmented_blocks_float32_iteration():
    G, rows, cols, blocks = blockdiag.permuted_block_diagonal(96, 3, seed=5)
    O = oracle.ns5(G, precision="f32")
    assert blockdiag.off_block_is_zero(O, rows, cols)
    for b in range(3):
        Ob = oracle.ns5(blockdiag.augmented(blocks, b), precision="f32")[:32, :32]
        assert parity.rel_fro(O[np.ix_(rows[b], cols[b])], Ob) <= 1e-5, b
