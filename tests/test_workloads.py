"""The seeded synthetic inputs (newton_schulz_09_amd/workloads.py) against
their stated recipes: shapes and order, determinism per seed, the rank-16 plus
noise structure of the GPT-2 hidden sets, the orthogonal factors and singular
value ranges of the U diag(s) V^T workloads, and the quarter of exactly-zero
singular values of the extreme-aspect batch.  Small sizes where the generators
take them; the full-size generators are the same code."""

import numpy as np

from newton_schulz_09_amd import workloads


def test_single_64x128():
    G, buf = workloads.single_64x128()
    assert G.shape == (64, 128) and G.dtype == np.float32
    assert not buf.any() and buf.shape == G.shape
    assert abs(float(G.mean())) < 0.05 and 0.95 < float(G.std()) < 1.05
    G2, _ = workloads.single_64x128()
    assert np.array_equal(G, G2)                       # seeded


def test_gpt2_hidden_sets_shapes_and_order():
    assert workloads.GPT2_124M_SHAPES == [(768, 2304), (768, 768), (768, 3072), (3072, 768)]
    assert workloads.GPT2_1P5B_SHAPES == [(1600, 4800), (1600, 1600), (1600, 6400), (6400, 1600)]
    assert (workloads.GPT2_124M_LAYERS, workloads.GPT2_1P5B_LAYERS) == (12, 48)
    # the generator both sets use, on small shapes: layer-major, per-matrix seeds
    shapes = [(24, 72), (24, 24), (72, 24)]
    items = workloads.gpt_hidden_set(shapes, 3, seed=1)
    assert [it[2].shape for it in items] == shapes * 3
    assert [(it[0], it[1]) for it in items[:4]] == [(0, 0), (0, 1), (0, 2), (1, 0)]
    assert all(it[2].dtype == np.float32 and it[3].dtype == np.float32 for it in items)
    one = workloads.gpt_hidden_set(shapes, 3, seed=1, only_shape=2)
    assert [it[1] for it in one] == [2, 2, 2]
    assert np.array_equal(one[1][2], items[1 * 3 + 2][2])    # any subset, same matrices


def test_gpt2_matrix_is_rank16_plus_noise():
    layer, si, G, buf = workloads.gpt_hidden_set([(768, 2304)], 1, seed=1)[0]
    assert np.array_equal(G, workloads.gpt2_124m(only_shape=0)[0][2])   # the 124M set's first matrix
    s = np.linalg.svd(G.astype(np.float64), compute_uv=False)
    # a rank-16 signal (L R / 4, singular values ~ sqrt(768 * 2304) / 4 ~ 330)
    # over 0.1 N(0,1) noise (largest singular value ~ 0.1 (sqrt(768) + sqrt(2304)) ~ 7.6)
    assert s[15] > 100 and s[16] < 10
    assert 0.095 < float(buf.std()) < 0.105               # momentum buffer: std 0.1


def test_u_diag_s_vt_recipe():
    G, U, s, V = workloads.square_4096(n=128)
    n = 128
    assert np.allclose(U.T @ U, np.eye(n), atol=1e-10) and np.allclose(V.T @ V, np.eye(n), atol=1e-10)
    assert s.min() >= 1e-3 and s.max() <= 1.0
    assert np.allclose(G, (U * s) @ V.T, atol=1e-6)
    sv = np.linalg.svd(G.astype(np.float64), compute_uv=False)
    assert np.allclose(np.sort(sv)[::-1], np.sort(s)[::-1], atol=1e-6)


def test_extreme_aspect_recipe():
    items = workloads.extreme_aspect(wide=(64, 256), count=2)
    assert [it[0].shape for it in items] == [(64, 256), (64, 256), (256, 64), (256, 64)]
    for G, U, s, V in items:
        k = 64
        assert np.count_nonzero(s == 0.0) == k // 4       # a quarter exactly zero
        nz = s[s > 0]
        assert nz.min() >= 1e-4 and nz.max() <= 1.0
        assert np.allclose(U.T.astype(np.float64) @ U, np.eye(k), atol=1e-5)
        assert np.allclose(V.T.astype(np.float64) @ V, np.eye(k), atol=1e-5)
        sv = np.linalg.svd(G.astype(np.float64), compute_uv=False)
        assert np.sum(sv < 1e-6) == k // 4                # rank-deficient by exactly that quarter
    again = workloads.extreme_aspect(wide=(64, 256), count=2, which="tall", indices=[1])
    assert np.array_equal(again[0][0], items[3][0])       # any subset, same matrices
