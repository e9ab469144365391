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


# The float32 matrix cores' accumulator departs from round-to-nearest by an
# amount that grows with the length of the sum: on 16 x K Gaussian inputs the
# float32 iteration lands 1.9e-6, 5.1e-6, 1.8e-5, 8.9e-5 and 7.3e-4 from the
# oracle (float64 accumulation) at K = 2^12, 2^14, 2^16, 2^18 and 2^20, where a
# sequential round-to-nearest float32 accumulator lands 1.8e-6 .. 5.3e-5.  The
# float32 bar (1e-4, from the workloads' K <= 6400) therefore does not carry to
# K = 2^20; there the bar is 2e-3, and the float32 iteration must still sit at
# least five times closer to its oracle than the bf16 iteration does (measured:
# 7.3e-4 against 7.6e-3).
F32_LONG_K_TOL = 2e-3


@pytest.mark.timeout(600)
@pytest.mark.parametrize("tall", [False, True], ids=["16x2^20", "2^20x16"])
def test_float32_iteration_longest_side(muon, longest, tall):
    G = longest[0]
    want = oracle.ns5(G, precision="f32")
    bf16_dist = parity.rel_fro(longest[1], want)
    if tall:
        G, want = np.ascontiguousarray(G.T), np.ascontiguousarray(want.T)
    print(f"float32 iteration {G.shape}", flush=True)
    out = parity.to_np(muon.newton_schulz_f32([torch.from_numpy(G).cuda()])[0])
    torch.cuda.synchronize()
    assert np.all(np.isfinite(out))
    r = parity.rel_fro(out, want)
    d = np.max(np.abs(parity.svals(out) - parity.svals(want)))
    print(f"relative Frobenius {r:.3g}, singular values {d:.3g}, bf16 iteration {bf16_dist:.3g}", flush=True)
    assert r <= F32_LONG_K_TOL and d <= F32_LONG_K_TOL, (r, d)
    assert r * 5 <= bf16_dist, (r, bf16_dist)


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
