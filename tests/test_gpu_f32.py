"""GPU parity of the iteration carried in float32 (muon_newton_schulz_f32_batched)
against the oracle's float32 iteration (``ns5(..., precision="f32")``), through
the C ABI.

Bar: relative Frobenius error <= 1e-4 per matrix and every sorted singular
value within 1e-4.  The GPU accumulates the products in float32 (MFMA), the
oracle in float64; that difference alone lands 0.5e-6 .. 3.3e-6 apart on these
inputs (numpy, float32 against float64 accumulation), so the bar leaves a
30-fold margin and is 100 times tighter than the distance between the bf16
and float32 iterations (1.4e-2 on the 64 x 128 case)."""

import numpy as np
import pytest
import torch

import oracle
from newton_schulz_09_amd import workloads

from . import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def muon():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from newton_schulz_09_amd import muon as m
    return m


def cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def check(got, want, name):
    parity.assert_f32_parity(got, want, name)


SHAPES = [(1, 1), (3, 5), (5, 3), (64, 64), (65, 130), (130, 65), (100, 1000), (257, 300), (640, 700),
          (700, 640), (768, 768), (96, 4000)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_shapes(muon, shape):
    G = workloads.gaussian(shape, seed=2000 + shape[0] + 3 * shape[1])
    out = parity.to_np(muon.newton_schulz_f32([cuda(G)])[0])
    check(out, oracle.ns5(G, precision="f32"), f"{shape}")


def test_single_64x128_after_momentum_and_transpose(muon):
    G, buf = workloads.single_64x128()
    _, u = oracle.momentum_nesterov(G, buf, 0.95)
    u_d = muon.momentum_nesterov(cuda(G), cuda(buf), mu=0.95)
    o, oT = (parity.to_np(x) for x in muon.newton_schulz_f32([u_d, u_d.t().contiguous()]))
    want = oracle.ns5(u, precision="f32")
    check(o, want, "64x128")
    check(oT, np.ascontiguousarray(want.T), "128x64")
    # the float32 and bf16 iterations differ by bf16 error, not more
    r = parity.rel_fro(o, parity.to_np(muon.ns5(u_d)))
    assert 1e-3 < r < 5e-2


@pytest.mark.parametrize("steps", [0, 1, 3, 7])
def test_step_counts(muon, steps):
    G = workloads.gaussian((200, 520), seed=60 + steps)
    out = parity.to_np(muon.newton_schulz_f32([cuda(G)], steps=steps)[0])
    want = oracle.ns5(G, steps=steps, precision="f32")
    if steps == 0:  # X0 = fl32(G / d): the same float64 quotient on both sides
        assert parity.ulp_diff32(out, want).max() <= 1
    else:
        check(out, want, f"steps={steps}")


def test_cubic_coefficients(muon):
    G = workloads.gaussian((130, 300), seed=71)
    cubic = muon.CUBIC_COEFFS
    out = parity.to_np(muon.newton_schulz_f32([cuda(G)], steps=12, coeffs=cubic)[0])
    check(out, oracle.ns5(G, steps=12, coeffs=cubic, precision="f32"), "cubic")


def test_zero_input_and_alias(muon):
    z = torch.zeros(70, 90, device="cuda")
    assert torch.count_nonzero(muon.newton_schulz_f32([z])[0]).item() == 0
    G = workloads.gaussian((90, 70), seed=6)
    g_d = cuda(G)
    muon.newton_schulz_f32([g_d], outs=[g_d])     # out aliases G
    check(parity.to_np(g_d), oracle.ns5(G, precision="f32"), "aliased")


def test_diagonal_input_stays_diagonal(muon):
    G = np.zeros((6, 9), dtype=np.float32)
    G[np.arange(6), np.arange(6)] = [1.0, 0.5, 0.1, 0.01, 1e-3, 0.0]
    out = parity.to_np(muon.newton_schulz_f32([cuda(G)])[0])
    off = out.copy()
    off[np.arange(6), np.arange(6)] = 0
    assert not off.any()
    want = oracle.ns5(G, precision="f32")
    # each step's roundings differ by under an ulp and the iteration's slope
    # (up to |p'| = a = 3.4445) amplifies them over five steps: measured 11
    # float32 ulps, 6e-7 relative
    check(out, want, "diagonal")
    d = np.abs(out.astype(np.float64) - want.astype(np.float64))
    assert np.all(d <= 1e-5 * np.abs(want.astype(np.float64)))


def test_mixed_shape_batch(muon):
    shapes = [(64, 128), (128, 64), (65, 130), (3, 5), (300, 768), (768, 300), (64, 128), (200, 520), (1, 1)]
    rng = np.random.default_rng(321)
    host = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    outs = muon.newton_schulz_f32([cuda(h) for h in host])
    for h, o, s in zip(host, outs, shapes):
        check(parity.to_np(o), oracle.ns5(h, precision="f32"), f"batch {s}")


def test_gpt2_124m_set_sampled(muon):
    """The GPT-2 124M hidden set (48 matrices, one call): one matrix of each
    shape against the oracle, every output finite."""
    items = workloads.gpt2_124m()
    Gs = [cuda(it[2]) for it in items]
    outs = muon.newton_schulz_f32(Gs)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.isfinite(o).all()
    seen = set()
    for k, it in enumerate(items):
        shape = it[2].shape
        if shape in seen:
            continue
        seen.add(shape)
        check(parity.to_np(outs[k]), oracle.ns5(it[2], precision="f32"), f"124M {shape} #{k}")


def test_passes_over_one_workspace(muon):
    """130 same-shaped matrices plus another shape: passes of at most 128 that
    reuse the workspace from its start, each matrix as in a call of its own."""
    rng = np.random.default_rng(99)
    shapes = [(40, 96)] * 130 + [(96, 40)] * 2
    host = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    Gs = [cuda(h) for h in host]
    outs = muon.newton_schulz_f32(Gs)
    for k in (0, 127, 128, 129, 130, 131):
        single = parity.to_np(muon.newton_schulz_f32([Gs[k]])[0])
        assert np.array_equal(parity.to_np(outs[k]), single), k
    for k in (129, 131):
        check(parity.to_np(outs[k]), oracle.ns5(host[k], precision="f32"), f"pass {k}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cap", [1, 7])
def test_scale_several_tiles_per_workgroup(muon, tmp_path, cap):
    """The float32 scale kernel walks its 32 x 32 tiles grid-stride; a tiny
    workgroup cap (MUON_F32_SCALE_WG_CAP, read once per process, so set in a
    child process) makes each workgroup take many tiles (as the largest
    shapes do), with the same results as one tile per workgroup."""
    from . import cap_child, capped
    rng = np.random.default_rng(cap)
    shapes = [(70, 150), (150, 70), (33, 40)]
    arrays = {"n": np.int64(len(shapes))}
    for k, s in enumerate(shapes):
        arrays[f"G{k}"] = rng.standard_normal(s).astype(np.float32)
    want = cap_child.run("f32scale", arrays)
    got = capped.run_capped(tmp_path, "f32scale", arrays, "MUON_F32_SCALE_WG_CAP", cap)
    assert len(got) == len(want) == 2 * len(shapes)
    for a, b in zip(got, want):
        assert np.array_equal(a, b)
