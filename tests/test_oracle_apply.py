"""Pins of the oracle's parameter update p <- p - lr * O (the reading taken
where the Muon section of the Synced report on Modded-NanoGPT orders the step
as momentum, orthogonalisation, update, but its formula did not survive)."""

from fractions import Fraction

import numpy as np

import oracle


def _ulp_diff32(a, b):
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def test_zero_learning_rate_leaves_the_parameters():
    rng = np.random.default_rng(1)
    p = rng.standard_normal((17, 23)).astype(np.float32)
    O = oracle.round_bf16(rng.standard_normal((17, 23))).astype(np.float32)
    assert np.array_equal(oracle.apply_update(p, O, 0.0), p)


def test_unit_update_subtracts_the_learning_rate():
    """O = 1 everywhere: the result is p - lr, elementwise, rounded once."""
    p = np.linspace(-3, 3, 101, dtype=np.float32)
    got = oracle.apply_update(p, np.ones_like(p), 0.25)
    assert np.array_equal(got, (p.astype(np.float64) - 0.25).astype(np.float32))
    got = oracle.apply_update(p, -np.ones_like(p), 0.25)
    assert np.array_equal(got, (p.astype(np.float64) + 0.25).astype(np.float32))


def test_single_rounding_against_exact_rationals():
    rng = np.random.default_rng(2)
    p = (rng.standard_normal(400) * 10 ** rng.uniform(-2, 2, 400)).astype(np.float32)
    O = oracle.round_bf16(rng.standard_normal(400)).astype(np.float32)
    lr = np.float32(0.02)
    got = oracle.apply_update(p, O, float(lr))
    exact = [Fraction(float(x)) - Fraction(float(lr)) * Fraction(float(o)) for x, o in zip(p, O)]
    want = np.array([np.float32(float(v)) for v in exact], dtype=np.float32)
    d = _ulp_diff32(got, want)
    assert d.max() <= 1 and np.mean(d == 0) >= 0.99


def test_step_with_update_composes_momentum_ns5_and_update():
    rng = np.random.default_rng(3)
    g = rng.standard_normal((12, 20)).astype(np.float32)
    b = (0.1 * rng.standard_normal((12, 20))).astype(np.float32)
    p = rng.standard_normal((12, 20)).astype(np.float32)
    bufs, ps = oracle.muon_step_apply([g], [b], [p], mu=0.9, lr=0.05)
    nb, u = oracle.momentum_nesterov(g, b, 0.9)
    assert np.array_equal(bufs[0], nb)
    assert np.array_equal(ps[0], oracle.apply_update(p, oracle.ns5(u), 0.05))
