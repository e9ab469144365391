"""Comparison helpers for GPU-vs-oracle parity.

Tolerances (stated for the NS5 output of every matrix): relative Frobenius
error <= 1e-2 against the oracle, and every sorted singular value within 0.02
of the oracle's.  The oracle accumulates in float64 and the GPU in float32,
which flips a few bf16 roundings that the iteration then amplifies; the
measured spread of that effect on these workloads is 5e-4 .. 7e-3, so the
bound is the accumulation difference with margin, not slack for errors.
Momentum is float32 arithmetic with one rounding per result: at most 1 ulp
apart (the oracle rounds float64 -> float32, which can differ from a single
fused rounding only at a float64-made tie).
"""

import numpy as np
import torch

REL_FRO_TOL = 1e-2
SIGMA_TOL = 0.02


def to_np(t):
    return t.detach().to("cpu").numpy()


def rel_fro(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    num = np.linalg.norm(got - want)
    return num / den if den > 0 else num


def svals(M):
    """Singular values, float64, descending (LAPACK through torch on the CPU)."""
    t = torch.from_numpy(np.ascontiguousarray(M, dtype=np.float64))
    return torch.linalg.svdvals(t).numpy()


def assert_ns5_parity(got, want, name="", check_sigma=True, bar=(REL_FRO_TOL, SIGMA_TOL)):
    """The parity bar; ``bar`` (relative Frobenius, singular value) is the
    stated one unless a CPU model of float32 accumulation (``model_bar``)
    widens it for this input."""
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    r = rel_fro(got, want)
    assert r <= bar[0], f"{name}: relative Frobenius error {r:.3g} > {bar[0]:.3g}"
    if check_sigma:
        d = np.max(np.abs(svals(got) - svals(want)))
        assert d <= bar[1], f"{name}: singular values differ by {d:.3g} > {bar[1]:.3g}"
    return r


#: Bar of the iteration carried in float32 against the oracle's float32
#: iteration: the GPU accumulates the products in float32 (MFMA), the oracle in
#: float64, which alone lands 0.5e-6 .. 3.3e-6 apart (numpy, float32 against
#: float64 accumulation), so the bar leaves a 30-fold margin and is 100 times
#: tighter than the distance between the bf16 and float32 iterations.
F32_REL_FRO_TOL = 1e-4
F32_SIGMA_TOL = 1e-4


def assert_f32_parity(got, want, name=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    r = rel_fro(got, want)
    assert r <= F32_REL_FRO_TOL, f"{name}: relative Frobenius error {r:.3g} > {F32_REL_FRO_TOL}"
    d = np.max(np.abs(svals(got) - svals(want)))
    assert d <= F32_SIGMA_TOL, f"{name}: singular values differ by {d:.3g} > {F32_SIGMA_TOL}"
    return r


def ulp_diff32(a, b):
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def bf16_ulp_diff(a, b):
    """Distance in bf16 steps between two arrays of bf16-valued float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    ia = (a.view(np.uint32) >> 16).astype(np.int64)
    ib = (b.view(np.uint32) >> 16).astype(np.int64)
    ia = np.where(ia >= 0x8000, -(ia & 0x7FFF), ia)
    ib = np.where(ib >= 0x8000, -(ib & 0x7FFF), ib)
    return np.abs(ia - ib)


def is_bf16_valued(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return bool(np.all((a.view(np.uint32) & 0xFFFF) == 0))


def model_bar(G, margin=1.25):
    """The (relative Frobenius, singular value) bar for NS5 of ``G``: the
    stated bar, or ``margin`` times the distance from the oracle of the
    oracle's algorithm evaluated with float32 accumulation (tests/fp32_model,
    one rounding per term), whichever is larger.  Only tiny inputs afford the
    model; on the workloads it lands inside the stated bar."""
    import oracle
    from . import fp32_model
    want = oracle.ns5(G)
    got = fp32_model.ns5_f32acc(G, block=1)
    r = rel_fro(got, want)
    d = float(np.max(np.abs(svals(got) - svals(want))))
    return max(REL_FRO_TOL, margin * r), max(SIGMA_TOL, margin * d)
