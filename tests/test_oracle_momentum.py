"""Pins for the oracle's Nesterov momentum (Muon section of the Synced report
on Modded-NanoGPT, summary paragraph, where the momentum output is the
matrix that gets orthogonalised).  Reading: buf <- mu*buf + g, u <- g + mu*buf, one float32 rounding per
result.  Pinned by closed forms of the linear recurrence and exact arithmetic."""

from fractions import Fraction

import numpy as np

from oracle import momentum_nesterov
from newton_schulz_09_amd import workloads


def _ulp_diff32(a, b):
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def test_zero_buffer_closed_form_bitwise():
    # From a zero buffer: buf' = g exactly and u = (1 + mu) g rounded once.
    G, buf = workloads.single_64x128()
    b, u = momentum_nesterov(G, buf, 0.95)
    assert np.array_equal(b, G)
    mu = float(np.float32(0.95))
    # (1 + mu) has 25 significant bits, g 24: the product is exact in float64
    want = (G.astype(np.float64) * (1.0 + mu)).astype(np.float32)
    assert np.array_equal(u, want)


def test_constant_gradient_geometric_closed_form():
    rng = np.random.default_rng(2)
    g = rng.standard_normal(1000).astype(np.float32)
    buf = np.zeros_like(g)
    mu = float(np.float32(0.9))
    for t in range(1, 31):
        buf, u = momentum_nesterov(g, buf, 0.9)
        geo = (1.0 - mu ** t) / (1.0 - mu)
        np.testing.assert_allclose(buf, g * geo, rtol=3e-6 * t, atol=0)
        np.testing.assert_allclose(u, g * (1.0 + mu * geo), rtol=3e-6 * t, atol=0)


def test_varying_gradient_is_discounted_sum():
    # buf_t = sum_s mu^(t-s) g_s : no dampening factor (1 - mu), no lookahead error
    rng = np.random.default_rng(3)
    gs = rng.standard_normal((12, 500)).astype(np.float32)
    mu = float(np.float32(0.95))
    buf = np.zeros(500, dtype=np.float32)
    for t in range(12):
        buf, u = momentum_nesterov(gs[t], buf, 0.95)
        want_buf = sum(mu ** (t - s) * gs[s].astype(np.float64) for s in range(t + 1))
        np.testing.assert_allclose(buf, want_buf, rtol=1e-5, atol=1e-5)
        np.testing.assert_allclose(u, gs[t] + mu * want_buf, rtol=1e-5, atol=1e-5)


def test_single_rounding_against_exact_rationals():
    rng = np.random.default_rng(4)
    g = (rng.standard_normal(400) * 10 ** rng.uniform(-3, 3, 400)).astype(np.float32)
    buf = (rng.standard_normal(400) * 10 ** rng.uniform(-3, 3, 400)).astype(np.float32)
    b, u = momentum_nesterov(g, buf, 0.95)
    mu = Fraction(float(np.float32(0.95)))
    exact_b = [mu * Fraction(float(x)) + Fraction(float(y)) for x, y in zip(buf, g)]
    want_b = np.array([np.float32(float(v)) for v in exact_b], dtype=np.float32)
    # float(Fraction) rounds once to float64, np.float32 once more: the two
    # can differ from a single rounding only at a float64-made tie
    d = _ulp_diff32(b, want_b)
    assert d.max() <= 1 and np.mean(d == 0) >= 0.99
    exact_u = [Fraction(float(y)) + mu * Fraction(float(x)) for x, y in zip(b, g)]
    want_u = np.array([np.float32(float(v)) for v in exact_u], dtype=np.float32)
    d = _ulp_diff32(u, want_u)
    assert d.max() <= 1 and np.mean(d == 0) >= 0.99
