"""A model of NS5 evaluated with float32 accumulation: the oracle's algorithm
(the steps of zeroth_power_via_newtonschulz5, Muon section of the Synced
report on Modded-NanoGPT, with the same bf16 rounding points) in which every
matrix product is summed in float32 instead of float64.

TEST INFRASTRUCTURE: it shares no code with the HIP library (nor with the
oracle, whose float64 arithmetic it is measured against).  It exists to pin,
on the CPU, how far any float32-accumulating evaluation of the algorithm can
land from the float64 oracle on a given input: the iteration amplifies the
few bf16 roundings that float32 partial sums flip, and on some inputs that
alone approaches or exceeds the parity bar.

Accumulation model: the products of bf16 values are exact in float32; they
are added to a float32 accumulator ``block`` at a time, each block's sum
formed exactly and added with one round-to-nearest-even rounding (block = 1:
a plain sequential float32 sum; block = 16: one rounding per 16-deep matrix
core instruction).  The same model serves the iteration carried in float32
(``precision="f32"``), where a block's sum of float32 products is formed in
float64 (close to exact) before its one rounding.  The fused updates round as a float32 fused multiply-add
would: B = bf16(fl32(c * (A A) + fl32(b * A))), X = bf16(fl32(a * X + B X)).
"""

import numpy as np


def _bf16(x):
    """Round finite float64 values to bfloat16, ties to even: scale to the
    bf16 quantum of each value's binade, rint (half to even), scale back."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e - 8, -133)
    return np.ldexp(np.rint(np.ldexp(x, -q)), q)


def _fl32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def matmul_f32(P, Q, block=1):
    """P @ Q summed over k in float32: the running sum is rounded to float32
    after every ``block`` terms (each block summed exactly in float64, which
    holds for bf16 x bf16 products of moderate exponent spread).
    ``block=None``: no float32 rounding at all (a float64 sum)."""
    P = np.asarray(P, dtype=np.float64)
    Q = np.asarray(Q, dtype=np.float64)
    if block is None:
        return P @ Q
    K = P.shape[1]
    acc = np.zeros((P.shape[0], Q.shape[1]), dtype=np.float64)
    for k0 in range(0, K, block):
        acc = _fl32(acc + P[:, k0:k0 + block] @ Q[k0:k0 + block, :])
    return acc


def ns5_f32acc(G, steps=5, eps=1e-7, coeffs=(3.4445, -4.7750, 2.0315), block=1, precision="bf16"):
    """NS5 of one matrix with float32 accumulation (see the module
    docstring); returns float32 in G's shape.  ``block=None`` carries sums
    and updates in float64 instead, which is the oracle's arithmetic.
    ``precision="f32"``: the iteration carried in float32 (no bf16 cast; X0,
    A, B and X each rounded once to float32), as the oracle's f32 mode."""
    fl = _fl32 if block is not None else (lambda x: np.asarray(x, dtype=np.float64))
    rnd = _bf16 if precision == "bf16" else _fl32
    a, b, c = (float(np.float32(v)) for v in coeffs)
    eps = float(np.float32(eps))
    u = np.asarray(G, dtype=np.float32).astype(np.float64)
    d = np.sqrt(np.sum(u * u)) + eps
    X = _bf16(_bf16(u) / d) if precision == "bf16" else _fl32(u / d)
    tall = u.shape[0] > u.shape[1]
    if tall:
        X = X.T
    for _ in range(steps):
        A = rnd(matmul_f32(X, X.T, block))
        B = rnd(fl(c * matmul_f32(A, A, block) + fl(b * A)))
        X = rnd(fl(a * X + matmul_f32(B, X, block)))
    if tall:
        X = X.T
    return np.ascontiguousarray(X).astype(np.float32)
