"""Pins for the oracle's float64 -> bfloat16 rounding (round to nearest, ties to
even), which the Muon section's listing relies on through ``G.bfloat16()``
and the bf16 iteration.  Checked by brute force over the bf16 value table and
against torch's float32 -> bfloat16 conversion for float32 inputs."""

import numpy as np
import pytest
import torch

from oracle import round_bf16

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _bf16_table():
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    vals = (bits << 16).view(np.float32).astype(np.float64)
    ok = np.isfinite(vals)
    return bits[ok], vals[ok]


def _brute_nearest(x, bits, vals):
    """Nearest finite bf16 (ties to the even bit pattern) by search over the
    whole table; values beyond the largest finite bf16 by half an ulp or more
    round to infinity."""
    order = np.argsort(vals, kind="stable")
    sv, sb = vals[order], bits[order]
    # drop -0 duplicate: keep +0 and -0 both (they compare equal); search works
    out = np.empty_like(x)
    bmax = float.fromhex("0x1.fep127")
    for i, xi in enumerate(x):
        if abs(xi) >= bmax + 2.0 ** 119:      # at or past the overflow midpoint
            out[i] = np.copysign(np.inf, xi)
            continue
        j = np.searchsorted(sv, xi)
        cand = []
        for t in (j - 1, j, j + 1):
            if 0 <= t < len(sv):
                cand.append((abs(sv[t] - xi), int(sb[t]) & 1, sv[t]))
        cand.sort(key=lambda c: (c[0], c[1]))
        r = cand[0][2]
        if r == 0.0:
            r = np.copysign(0.0, xi)
        out[i] = r
    return out


def test_round_bf16_matches_brute_force_table():
    bits, vals = _bf16_table()
    rng = np.random.default_rng(0)
    n = 3000
    mags = np.exp2(rng.uniform(-140, 128, n))
    x = mags * rng.choice([-1.0, 1.0], n)
    # exact midpoints between neighbouring bf16 values (ties), both signs
    pos = np.sort(vals[(vals > 0)])
    idx = rng.integers(0, len(pos) - 1, 800)
    mids = (pos[idx] + pos[idx + 1]) / 2.0          # exact in float64
    x = np.concatenate([x, mids, -mids, [0.0, -0.0, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135,
                                         float.fromhex("0x1.fep127"), float.fromhex("0x1.ff8p127"),
                                         float.fromhex("0x1.ff7ffp127"), 1.0 + 2.0 ** -8,
                                         1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -40]])
    got = round_bf16(x)
    want = _brute_nearest(x, bits, vals)
    assert np.array_equal(np.signbit(got[got == 0]), np.signbit(want[got == 0]))
    assert np.array_equal(got, want)


def test_round_bf16_agrees_with_torch_on_float32_inputs():
    rng = np.random.default_rng(1)
    x32 = (rng.standard_normal(200000) * np.exp2(rng.uniform(-30, 30, 200000))).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    got = round_bf16(x32.astype(np.float64))
    assert np.array_equal(got, want)


def test_round_bf16_special_values():
    x = np.array([np.inf, -np.inf, np.nan, 1.0, -1.0, 0.5])
    r = round_bf16(x)
    assert r[0] == np.inf and r[1] == -np.inf and np.isnan(r[2])
    assert list(r[3:]) == [1.0, -1.0, 0.5]
    # ties to even at 1: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert round_bf16(1.0 + 2.0 ** -8) == 1.0
    assert round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2 * 2.0 ** -7
