"""Seeded synthetic inputs for the Muon hot path (numpy only).

This module holds input generation and nothing of the method's arithmetic:
it is the one piece that both the GPU tests and the CPU oracle are fed from.
Every draw uses ``numpy.random.default_rng`` (PCG64).  Where a workload has
many matrices, each matrix has its own generator seeded with the tuple
(seed, layer, shape index) or (seed, index), so any subset can be generated
on its own and the workload is fully defined by its seed.

Workloads (shapes are rows x cols of the fp32 gradient G):

* ``single_64x128``   - seed 0.  G ~ N(0,1), 64x128, float64 draws cast to
  float32; the momentum buffer starts at zero; its 128x64 transpose exercises
  the tall path.
* ``gpt2_124m``       - seed 1.  12 layers x (768x2304, 768x768, 768x3072,
  3072x768), the hidden matrices of GPT-2 124M.  Per matrix, from
  default_rng((seed, layer, shape_index)), in this order:
  L (m x 16), R (16 x n), N (m x n) ~ N(0,1) and a momentum buffer
  0.1 * N(0,1), all drawn as float32; G = L R / 4 + 0.1 N in float32 (a rank-16
  signal plus noise, standing in for a training gradient).
* ``square_4096``     - seed 3.  G = U diag(s) V^T, U and V the Q factors of
  QR of 4096x4096 N(0,1) matrices (float64), s log-uniform on [1e-3, 1].
* ``gpt2_1p5b``       - seed 4.  As ``gpt2_124m`` with 48 layers x (1600x4800,
  1600x1600, 1600x6400, 6400x1600), the hidden matrices of GPT-2 1.5B.
  Per matrix generator: default_rng((seed, layer, shape_index)).
* ``extreme_aspect``  - seed 5.  Eight 2048x8192 then eight 8192x2048 matrices
  G = U diag(s) V^T with U, V from reduced QR of float32 N(0,1) draws,
  s log-uniform on [1e-4, 1] and a random quarter of s set to exactly 0;
  matrix i (0..15) draws from default_rng((seed, i)).
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GPT2_124M_SHAPES = [(768, 2304), (768, 768), (768, 3072), (3072, 768)]
GPT2_124M_LAYERS = 12
GPT2_1P5B_SHAPES = [(1600, 4800), (1600, 1600), (1600, 6400), (6400, 1600)]
GPT2_1P5B_LAYERS = 48
MU = 0.95


def single_64x128(seed=0):
    """G (64x128, float32) and a zero momentum buffer."""
    rng = np.random.default_rng(seed)
    G = rng.standard_normal((64, 128)).astype(np.float32)
    return G, np.zeros_like(G)


def _lowrank_plus_noise(rng, rows, cols, rank=16):
    L = rng.standard_normal((rows, rank), dtype=np.float32)
    R = rng.standard_normal((rank, cols), dtype=np.float32)
    N = rng.standard_normal((rows, cols), dtype=np.float32)
    G = (L @ R) * np.float32(0.25) + np.float32(0.1) * N
    buf = np.float32(0.1) * rng.standard_normal((rows, cols), dtype=np.float32)
    return G.astype(np.float32), buf.astype(np.float32)


def _workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def gpt_hidden_set(shapes, layers, seed, only_shape=None):
    """Gradients and momentum buffers for ``layers`` x ``shapes``.

    Returns a list of ``(layer, shape_index, G, buf)``, layer-major.
    ``only_shape`` (a shape index) generates just that class.  Matrices are
    drawn on a few threads; each has its own generator, so the values do not
    depend on the order in which they are drawn.
    """
    keys = [(layer, si) for layer in range(layers) for si in range(len(shapes))
            if only_shape is None or si == only_shape]

    def one(key):
        layer, si = key
        r, c = shapes[si]
        G, buf = _lowrank_plus_noise(np.random.default_rng((seed, layer, si)), r, c)
        return (layer, si, G, buf)

    with ThreadPoolExecutor(_workers()) as ex:
        return list(ex.map(one, keys))


def gpt2_124m(seed=1, only_shape=None):
    return gpt_hidden_set(GPT2_124M_SHAPES, GPT2_124M_LAYERS, seed, only_shape)


def gpt2_1p5b(seed=4, only_shape=None):
    return gpt_hidden_set(GPT2_1P5B_SHAPES, GPT2_1P5B_LAYERS, seed, only_shape)


def square_4096(seed=3, n=4096):
    """G = U diag(s) V^T (float32) and its factors (float64)."""
    rng = np.random.default_rng(seed)
    U, _ = np.linalg.qr(rng.standard_normal((n, n)))
    V, _ = np.linalg.qr(rng.standard_normal((n, n)))
    s = np.exp(rng.uniform(np.log(1e-3), 0.0, n))
    G = ((U * s) @ V.T).astype(np.float32)
    return G, U, s, V


def extreme_aspect_one(rng, rows, cols):
    k = min(rows, cols)
    U, _ = np.linalg.qr(rng.standard_normal((rows, k), dtype=np.float32))
    V, _ = np.linalg.qr(rng.standard_normal((cols, k), dtype=np.float32))
    s = np.exp(rng.uniform(np.log(1e-4), 0.0, k))
    s[rng.permutation(k)[: k // 4]] = 0.0
    G = ((U.astype(np.float64) * s) @ V.T.astype(np.float64)).astype(np.float32)
    return G, U, s, V


def extreme_aspect(seed=5, wide=(2048, 8192), count=8, which=None, indices=None):
    """``count`` wide then ``count`` tall matrices as ``(G, U, s, V)``;
    ``which`` ('wide' or 'tall') keeps one half, ``indices`` (within the half
    or the whole list) a subset."""
    idx = list(range(2 * count))
    if which == "wide":
        idx = idx[:count]
    elif which == "tall":
        idx = idx[count:]
    if indices is not None:
        idx = [idx[i] for i in indices]
    out = []
    for i in idx:
        shape = wide if i < count else (wide[1], wide[0])
        out.append(extreme_aspect_one(np.random.default_rng((seed, i)), *shape))
    return out


def gaussian(shape, seed, scale=1.0):
    """A plain N(0, scale^2) float32 matrix for edge-shape tests."""
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_normal(shape)).astype(np.float32)
