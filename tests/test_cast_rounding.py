"""The bf16 cast computes X0 = bf16(fl64(v / d)) (v a bf16 value, d the norm
plus eps) without a float64 division for almost every element: q =
v * fl32(1/d) in float32 is within about 2 float32 ulps of v / d, so the
hardware round-to-nearest-even of q to bf16 is the same unless q lies within
8 ulps of a bf16 rounding midpoint or is not a normal float32; only those
elements take the float64 quotient.  These CPU checks pin that criterion
(written here with numpy, independently of the kernel) against the direct
definition, on random inputs and on inputs built to sit next to a midpoint.
"""
import numpy as np


def bf16_from_f64(q):
    """Round float64 values to bf16 once (nearest, ties to even)."""
    m, e = np.frexp(np.asarray(q, np.float64))
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)


def bf16_from_f32(x):
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def fast_cast(v, d, fallback=True):
    r32 = (1.0 / d).astype(np.float32)
    q = (v.astype(np.float32) * r32).astype(np.float32)
    bits = q.view(np.uint32)
    mag = bits & 0x7FFFFFFF
    near = ((bits & 0xFFFF).astype(np.int64) - 0x8000) ** 2 <= 64
    slow = ((mag != 0) & (mag < 0x01000000)) | (mag >= 0x7F800000)
    if fallback:
        slow |= near
    return np.where(slow, bf16_from_f64(v / d), bf16_from_f32(q))


def near_midpoint_inputs(rng, n, max_rel):
    v = bf16_from_f64(rng.standard_normal(n) * 3)
    m = bf16_from_f64(rng.uniform(1e-3, 1.0, n))
    _, e = np.frexp(m)
    mid = m + np.ldexp(1.0, e - 9)                      # halfway to the next bf16 value
    rel = rng.choice([-1.0, 1.0], n) * np.exp(rng.uniform(np.log(2.0 ** -30), np.log(max_rel), n))
    d = np.abs(v / mid) * (1 + rel)
    return v, np.where(d == 0, 1.0, d)


def test_random_inputs_match_the_definition():
    rng = np.random.default_rng(0)
    for _ in range(4):
        d = np.float64(np.exp(rng.uniform(-16, 30)))
        v = bf16_from_f64(rng.standard_normal(500_000) * np.exp(rng.uniform(-20, 20, 500_000)) * d)
        v[:100] = 0.0
        assert np.array_equal(fast_cast(v, np.full_like(v, d)), bf16_from_f64(v / d))


def test_near_midpoint_inputs_match_the_definition():
    rng = np.random.default_rng(1)
    v, d = near_midpoint_inputs(rng, 500_000, 2.0 ** -16)
    assert np.array_equal(fast_cast(v, d), bf16_from_f64(v / d))


def test_the_fallback_is_needed():
    """Without the near-midpoint fallback the float32 quotient rounds the
    wrong way on such inputs: the check above has teeth."""
    rng = np.random.default_rng(1)
    v, d = near_midpoint_inputs(rng, 500_000, 2.0 ** -16)
    assert np.sum(fast_cast(v, d, fallback=False) != bf16_from_f64(v / d)) > 1000
