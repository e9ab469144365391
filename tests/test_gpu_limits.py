"""GPU parity at the largest shapes the library accepts on either side: a long
side of 2^20 (16 x 2^20 and its transpose, against the oracle run whole), and
a short side of 16384 (16384 x 16384, a permuted block-diagonal input whose
blocks the oracle checks one by one, with every entry off the blocks exactly
zero).  These run the grids, K loops and 64-bit offsets at their extremes,
for the bf16 iteration and for the iteration carried in float32."""

import numpy as np
import pytest
import torch

import oracle
from newton_schulz_09_amd import workloads

from . import blockdiag, parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def muon():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from newton_schulz_09_amd import muon as m
    return m


@pytest.fixture(scope="module")
def longest():
    """16 x 2^20 and the oracle's NS5 of it (the oracle of the transpose is
    its transpose, by the tall rule the oracle's pins cover)."""
    G = workloads.gaussian((16, 1 << 20), seed=71)
    return G, oracle.ns5(G)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("tall", [False, True], ids=["16x2^20", "2^20x16"])
def test_longest_side(muon, longest, tall):
    G, want = longest
    assert G.shape[1] == muon.MAX_LONG
    if tall:
        G, want = np.ascontiguousarray(G.T), np.ascontiguousarray(want.T)
    print(f"ns5 {G.shape}", flush=True)
    out = parity.to_np(muon.ns5(torch.from_numpy(G).cuda()))
    torch.cuda.synchronize()
    parity.assert_ns5_parity(out, want, f"{G.shape}")
    assert parity.is_bf16_valued(out)


@pytest.mark.timeout(300)
def test_shortest_side_at_its_limit(muon):
    n, nb = muon.MAX_SHORT, 32
    G, rows, cols, blocks = blockdiag.permuted_block_diagonal(n, nb, seed=72)
    print(f"ns5 {G.shape}, {nb} permuted blocks", flush=True)
    out = parity.to_np(muon.ns5(torch.from_numpy(G).cuda()))
    torch.cuda.synchronize()
    del G
    assert np.all(np.isfinite(out))
    assert blockdiag.off_block_is_zero(out, rows, cols)
    bs = n // nb
    for b in range(nb):
        want = oracle.ns5(blockdiag.augmented(blocks, b))[:bs, :bs]
        parity.assert_ns5_parity(out[np.ix_(rows[b], cols[b])], want, f"block {b}")


# The float32 products sum a K beyond 4096 in blocks of 1024 values, each
# block's sum added with one float32 rounding; tests/test_fp32_model.py pins
# on the CPU that this keeps even K = 2^20 within a tenth of the float32 bar,
# so the bar is the same at every K.  16 x K for K = 2^16, 2^18 and 2^20, and the transpose
# at 2^20.
@pytest.mark.timeout(600)
@pytest.mark.parametrize("K,tall", [(1 << 16, False), (1 << 18, False), (1 << 20, False), (1 << 20, True)],
                         ids=["16x2^16", "16x2^18", "16x2^20", "2^20x16"])
def test_float32_iteration_long_sums(muon, longest, K, tall):
    G = np.ascontiguousarray(longest[0][:, :K])
    want = oracle.ns5(G, precision="f32")
    bf16_dist = parity.rel_fro(longest[1], want) if K == muon.MAX_LONG else None
    if tall:
        G, want = np.ascontiguousarray(G.T), np.ascontiguousarray(want.T)
    print(f"float32 iteration {G.shape}", flush=True)
    out = parity.to_np(muon.newton_schulz_f32([torch.from_numpy(G).cuda()])[0])
    torch.cuda.synchronize()
    r = parity.assert_f32_parity(out, want, f"{G.shape}")
    print(f"relative Frobenius {r:.3g}" + (f", bf16 iteration {bf16_dist:.3g}" if bf16_dist else ""), flush=True)


@pytest.mark.timeout(600)
def test_float32_iteration_shortest_side_at_its_limit(muon):
    n, nb = muon.MAX_SHORT, 32
    G, rows, cols, blocks = blockdiag.permuted_block_diagonal(n, nb, seed=73)
    print(f"float32 iteration {G.shape}, {nb} permuted blocks", flush=True)
    out = parity.to_np(muon.newton_schulz_f32([torch.from_numpy(G).cuda()])[0])
    torch.cuda.synchronize()
    del G
    assert np.all(np.isfinite(out))
    assert blockdiag.off_block_is_zero(out, rows, cols)
    bs = n // nb
    for b in range(nb):
        want = oracle.ns5(blockdiag.augmented(blocks, b), precision="f32")[:bs, :bs]
        parity.assert_f32_parity(out[np.ix_(rows[b], cols[b])], want, f"block {b}")
