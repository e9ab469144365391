"""GPU parity at sizes the oracle finishes in seconds: momentum, the norm and
bf16 cast, NS5 over edge and ragged shapes, step counts, invariants and the
grouped launch.  Every call goes through the C ABI (libmuon.so)."""

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


# ---------------------------------------------------------------- momentum

def test_momentum_single_64x128(muon):
    G, buf = workloads.single_64x128()
    g_d, b_d = cuda(G), cuda(buf)
    u_d = muon.momentum_nesterov(g_d, b_d, mu=0.95)
    torch.cuda.synchronize()
    want_b, want_u = oracle.momentum_nesterov(G, buf, 0.95)
    assert np.array_equal(parity.to_np(b_d), want_b)
    assert parity.ulp_diff32(parity.to_np(u_d), want_u).max() <= 1


@pytest.mark.parametrize("numel,offset", [(1, 0), (7, 0), (1000003, 0), (1000003, 1), (4096 * 1031, 3)])
def test_momentum_ragged_misaligned_inplace(muon, numel, offset):
    rng = np.random.default_rng(numel + offset)
    g = rng.standard_normal(numel + offset).astype(np.float32)
    b = (0.1 * rng.standard_normal(numel + offset)).astype(np.float32)
    g_d, b_d = cuda(g), cuda(b)
    gv, bv = g_d[offset:], b_d[offset:]          # views: misaligned by `offset` floats
    muon.momentum_nesterov(gv, bv, u=gv, mu=0.9)  # u aliases g
    torch.cuda.synchronize()
    want_b, want_u = oracle.momentum_nesterov(g[offset:], b[offset:], 0.9)
    assert parity.ulp_diff32(parity.to_np(bv), want_b).max() <= 1
    assert parity.ulp_diff32(parity.to_np(gv), want_u).max() <= 1
    if offset:
        assert parity.to_np(g_d)[:offset].tolist() == g[:offset].tolist()   # untouched prefix


def test_momentum_empty(muon):
    e = torch.empty(0, device="cuda")
    out = muon.momentum_nesterov(e, e.clone())
    assert out.numel() == 0


def test_momentum_repeated_steps(muon):
    rng = np.random.default_rng(9)
    gs = rng.standard_normal((6, 50000)).astype(np.float32)
    buf = np.zeros(50000, dtype=np.float32)
    b_d = cuda(buf)
    for t in range(6):
        u_d = muon.momentum_nesterov(cuda(gs[t]), b_d, mu=0.95)
        buf, u = oracle.momentum_nesterov(gs[t], buf, 0.95)
        torch.cuda.synchronize()
        assert parity.ulp_diff32(parity.to_np(b_d), buf).max() <= 1
        assert parity.ulp_diff32(parity.to_np(u_d), u).max() <= 1


# ---------------------------------------------------------------- norm + cast

@pytest.mark.parametrize("shape", [(64, 128), (128, 64), (3, 5), (1, 1), (300, 1600), (1700, 90), (256, 256)])
def test_normalise_and_cast(muon, shape):
    """steps=0 returns X0 = bf16(bf16(G)/(||G||+eps)) in G's orientation.  The
    GPU forms the norm and the quotient in float64 like the oracle and rounds
    once to bf16, so the two agree bit for bit but for rare float64 ties."""
    G = workloads.gaussian(shape, seed=shape[0] * 7 + shape[1])
    out = parity.to_np(muon.ns5(cuda(G), steps=0))
    want = oracle.ns5(G, steps=0)
    d = parity.bf16_ulp_diff(out, want)
    assert d.max() <= 1 and np.mean(d == 0) >= 0.999
    assert parity.is_bf16_valued(out)


# ---------------------------------------------------------------- NS5

def test_single_64x128_after_momentum_and_transpose(muon):
    G, buf = workloads.single_64x128()
    _, u = oracle.momentum_nesterov(G, buf, 0.95)
    u_d = muon.momentum_nesterov(cuda(G), cuda(buf), mu=0.95)
    o = parity.to_np(muon.ns5(u_d))
    oT = parity.to_np(muon.ns5(u_d.t().contiguous()))
    want = oracle.ns5(u)
    parity.assert_ns5_parity(o, want, "64x128")
    parity.assert_ns5_parity(oT, np.ascontiguousarray(want.T), "128x64")
    # tall rule: NS5(G^T) = NS5(G)^T (same X after the transpose rule)
    assert np.max(parity.bf16_ulp_diff(oT, np.ascontiguousarray(o.T))) <= 1
    s = parity.svals(o)
    assert s.min() > 0.67 and s.max() < 1.14          # the page's band, bf16 noise aside
    assert parity.is_bf16_valued(o)


# (1000, 1600), (500, 1024) and (1024, 500) pad m to a multiple of 256, so
# X X^T runs on 256 x 256 tiles with padding inside its diagonal tiles
SHAPES = [(1, 1), (1, 9), (9, 1), (3, 5), (5, 3), (64, 64), (65, 130), (130, 65), (100, 1000),
          (257, 300), (640, 700), (700, 640), (768, 768), (1000, 1600), (96, 4000), (500, 1024), (1024, 500)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_ns5_shapes(muon, shape):
    G = workloads.gaussian(shape, seed=1000 + shape[0] + 3 * shape[1])
    out = parity.to_np(muon.ns5(cuda(G)))
    parity.assert_ns5_parity(out, oracle.ns5(G), f"{shape}")
    assert parity.is_bf16_valued(out)


@pytest.mark.parametrize("steps", [1, 2, 3, 7])
def test_ns5_step_counts(muon, steps):
    G = workloads.gaussian((200, 520), seed=40 + steps)
    out = parity.to_np(muon.ns5(cuda(G), steps=steps))
    parity.assert_ns5_parity(out, oracle.ns5(G, steps=steps), f"steps={steps}")


def test_ns5_zero_input_and_alias(muon):
    z = torch.zeros(70, 90, device="cuda")
    assert torch.count_nonzero(muon.ns5(z)).item() == 0
    G = workloads.gaussian((70, 90), seed=5)
    g_d = cuda(G)
    muon.ns5(g_d, out=g_d)                       # out aliases G
    parity.assert_ns5_parity(parity.to_np(g_d), oracle.ns5(G), "aliased")


def test_ns5_sign_symmetry_and_determinism(muon):
    G = workloads.gaussian((300, 500), seed=77)
    g_d = cuda(G)
    o1 = parity.to_np(muon.ns5(g_d))
    o2 = parity.to_np(muon.ns5(g_d))
    o3 = parity.to_np(muon.ns5(-g_d))
    assert np.array_equal(o1, o2)                # no atomics, no races
    # p is odd and the roundings to bf16 are symmetric, but the matrix cores'
    # float32 accumulation is not exactly sign-symmetric (a few sums differ in
    # the last bit), so the odd symmetry holds to the parity bar, not bitwise
    parity.assert_ns5_parity(o3, -o1, "sign")
    assert np.mean(parity.bf16_ulp_diff(o3, -o1) == 0) > 0.9


@pytest.mark.parametrize("shape,count", [((64, 128), 3), ((130, 65), 5), ((768, 768), 4), ((200, 900), 130)])
def test_grouped_equals_single(muon, shape, count):
    """One grouped launch per kernel (and passes of 128 beyond that) gives
    each matrix exactly what the single-matrix call gives."""
    rng = np.random.default_rng(shape[0] + count)
    Gs = [rng.standard_normal(shape).astype(np.float32) for _ in range(count)]
    g_d = [cuda(G) for G in Gs]
    outs = [parity.to_np(o) for o in muon.ns5_grouped(g_d)]
    singles = [parity.to_np(muon.ns5(g)) for g in (g_d[0], g_d[-1], g_d[count // 2])]
    assert np.array_equal(outs[0], singles[0])
    assert np.array_equal(outs[-1], singles[1])
    assert np.array_equal(outs[count // 2], singles[2])
    parity.assert_ns5_parity(outs[-1], oracle.ns5(Gs[-1]), "grouped last")


def test_diagonal_input(muon):
    """A diagonal G stays exactly diagonal; the entries follow the scalar
    recursion (the oracle's diagonal pin) up to float32-vs-float64
    accumulation of a single term, i.e. exactly."""
    G = np.zeros((6, 9), dtype=np.float32)
    G[np.arange(6), np.arange(6)] = [1.0, 0.5, 0.1, 0.01, 1e-3, 0.0]
    out = parity.to_np(muon.ns5(cuda(G)))
    want = oracle.ns5(G)
    off = out.copy()
    off[np.arange(6), np.arange(6)] = 0
    assert not off.any()
    assert np.max(parity.bf16_ulp_diff(out, want)) <= 1


# ---------------------------------------------------------------- batched (mixed shapes)

def _bitwise_equal_to_single(muon, Gs, outs):
    for k, (G, o) in enumerate(zip(Gs, outs)):
        single = parity.to_np(muon.ns5(G))
        got = parity.to_np(o)
        assert np.array_equal(got, single), f"matrix {k} {tuple(G.shape)} differs from the single call"


def test_batched_mixed_shapes_equal_single_calls(muon):
    """Every matrix of a mixed-shape batch gets exactly what muon_ns5 gives it
    alone (same tile, same kernels, independent matrices)."""
    shapes = [(64, 128), (128, 64), (65, 130), (130, 65), (3, 5), (768, 300), (300, 768), (64, 128),
              (200, 520), (200, 520), (1, 1), (96, 4000)]
    rng = np.random.default_rng(123)
    host = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    Gs = [cuda(h) for h in host]
    outs = muon.ns5_batched(Gs)
    _bitwise_equal_to_single(muon, Gs, outs)
    for k in (2, 6, 11):
        parity.assert_ns5_parity(parity.to_np(outs[k]), oracle.ns5(host[k]), f"batched {shapes[k]}")


def test_a_x_is_added_at_the_same_point_on_every_engine(muon):
    """a X + B X adds a X[i][j] inside its K loop once the K values below the
    end of row i's 64 block are summed, a point fixed by the row alone, so the
    engine a matrix runs on does not change its result.  Alone, (256, 768),
    (768, 256) and (768, 2304) run on 256 x 256 tiles (a X read from the stage
    and added in the same K step) and (200, 520) (columns padded to 640) on
    256 x 128 (a X copied out and added by the 64 x 64 wave sub-tiles); next to
    (300, 768), whose rows pad to 384, all of them run on 128 x 128 tiles."""
    shapes = [(256, 768), (768, 256), (768, 2304), (200, 520), (300, 768)]
    rng = np.random.default_rng(2024)
    host = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    Gs = [cuda(h) for h in host]
    outs = muon.ns5_batched(Gs)
    _bitwise_equal_to_single(muon, Gs, outs)
    for k in (0, 3):
        parity.assert_ns5_parity(parity.to_np(outs[k]), oracle.ns5(host[k]), f"{shapes[k]} next to (300, 768)")


def test_batched_many_shapes_and_passes(muon):
    """More than 8 distinct shapes and more than 128 matrices: the batch runs
    in several launch groups and passes over one workspace."""
    rng = np.random.default_rng(7)
    shapes = [(40 + 3 * i, 90 + 5 * i) for i in range(11)] * 13 + [(257, 90)] * 3
    Gs = [cuda(rng.standard_normal(s).astype(np.float32)) for s in shapes]
    outs = muon.ns5_batched(Gs)
    assert len(outs) == len(shapes) > 128
    _bitwise_equal_to_single(muon, Gs[:11] + Gs[-4:], outs[:11] + outs[-4:])
    _bitwise_equal_to_single(muon, Gs[100:104], outs[100:104])


@pytest.mark.parametrize("shapes", [
    # 120 x 3 + 8 x 3 = 384 tiles of 256 x 256 in one a X + B X launch: more
    # than one round on 256 CUs, a partial last round that holds every tall
    # matrix (the final step writes those transposed)
    [(256, 768)] * 120 + [(768, 256)] * 8,
    # 8 x 36 = 288 tiles
    [(768, 3072)] * 8,
])
def test_batched_large_launches_equal_single_calls(muon, shapes):
    """Launches of several rounds of 256 x 256 tiles give every matrix exactly
    what a single call (a few tiles) gives it, and match the oracle."""
    rng = np.random.default_rng(31)
    host = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    Gs = [cuda(h) for h in host]
    outs = muon.ns5_batched(Gs)
    _bitwise_equal_to_single(muon, Gs, outs)
    for k in sorted({len(shapes) * 7 // 8, len(shapes) - 1}):  # tiles of the last round
        parity.assert_ns5_parity(parity.to_np(outs[k]), oracle.ns5(host[k]), f"{shapes[k]} #{k}")


def test_batched_zero_steps_and_aliasing(muon):
    rng = np.random.default_rng(11)
    host = [rng.standard_normal(s).astype(np.float32) for s in [(70, 90), (90, 70), (33, 33)]]
    Gs = [cuda(h) for h in host]
    x0 = muon.ns5_batched(Gs, steps=0)
    for h, o in zip(host, x0):
        d = parity.bf16_ulp_diff(parity.to_np(o), oracle.ns5(h, steps=0))
        assert d.max() <= 1 and np.mean(d == 0) >= 0.999
    muon.ns5_batched(Gs, outs=Gs)            # in place
    for h, g in zip(host, Gs):
        parity.assert_ns5_parity(parity.to_np(g), oracle.ns5(h), "batched in place")



@pytest.mark.timeout(600)
@pytest.mark.parametrize("cap", [1, 7, 100])
def test_cast_several_tiles_per_workgroup(muon, tmp_path, cap):
    """Very large inputs make each cast workgroup handle several 64x64 tiles of
    one matrix; a low cap (MUON_CAST_WG_CAP, read once per process, so set in
    a child process) forces that path here.  X0, the NS5 result and the fused
    step's outputs and buffers are bitwise those of the one-tile path, for
    wide, tall, ragged and tile-aligned shapes."""
    from . import cap_child, capped
    shapes = [(200, 520), (520, 200), (64, 128), (3, 5), (768, 768), (130, 65)]
    rng = np.random.default_rng(31)
    arrays = {"n": np.int64(len(shapes))}
    for k, s in enumerate(shapes):
        arrays[f"G{k}"] = rng.standard_normal(s).astype(np.float32)
        arrays[f"B{k}"] = (0.1 * rng.standard_normal(s)).astype(np.float32)
    want = cap_child.run("cast", arrays)
    got = capped.run_capped(tmp_path, "cast", arrays, "MUON_CAST_WG_CAP", cap)
    assert len(got) == len(want) == 4 * len(shapes)
    for k, (w, g) in enumerate(zip(want, got)):
        part = ("X0", "NS5", "fused", "buffers")[k // len(shapes)]
        assert np.array_equal(w, g), f"{part} of matrix {k % len(shapes)} {shapes[k % len(shapes)]} differs with cap {cap}"


# ---------------------------------------------------------------- fused Muon step

def test_fused_step_matches_momentum_then_ns5(muon):
    """muon_momentum_ns5_batched = momentum, then NS5 of u: the new buffers are
    exact (<= 1 fp32 ulp vs the oracle), the updates meet the parity bar and
    agree with the unfused path but for rare bf16 ties of the norm."""
    from newton_schulz_09_amd import step as step_mod
    shapes = [(64, 128), (128, 64), (65, 130), (130, 65), (3, 5), (300, 768), (768, 300), (1, 7)]
    rng = np.random.default_rng(21)
    gs = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    bs = [(0.1 * rng.standard_normal(s)).astype(np.float32) for s in shapes]
    fused = step_mod.MuonStep(shapes)
    plain = step_mod.MuonStep(shapes)
    for st in (fused, plain):
        for k in range(len(shapes)):
            st.grads[k].copy_(torch.from_numpy(gs[k]))
            st.bufs[k].copy_(torch.from_numpy(bs[k]))
    for _ in range(2):                      # two steps: the buffer carries over
        fused.fused_step()
        plain.step()
    torch.cuda.synchronize()
    for k, s in enumerate(shapes):
        b1, u1 = oracle.momentum_nesterov(gs[k], bs[k], 0.95)
        b2, u2 = oracle.momentum_nesterov(gs[k], b1, 0.95)
        assert parity.ulp_diff32(parity.to_np(fused.bufs[k]), b2).max() <= 1
        assert np.array_equal(parity.to_np(fused.bufs[k]), parity.to_np(plain.bufs[k]))
        got = parity.to_np(fused.outs[k])
        parity.assert_ns5_parity(got, oracle.ns5(u2), f"fused {s}")
        d = parity.bf16_ulp_diff(got, parity.to_np(plain.outs[k]))
        assert np.mean(d == 0) > 0.99, f"{s}: fused and unfused differ in {np.mean(d != 0):.3%} of entries"


def test_fused_step_misaligned_and_ragged(muon):
    """Buffers that are not 16-byte aligned or not a multiple of 4 long take
    the scalar path of the fused pass."""
    rng = np.random.default_rng(5)
    shapes = [(7, 9), (33, 17)]
    g_host = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    b_host = [(0.1 * rng.standard_normal(s)).astype(np.float32) for s in shapes]
    flat_g = torch.zeros(1 + sum(r * c for r, c in shapes), device="cuda")
    flat_b = torch.zeros_like(flat_g)
    views_g, views_b, off = [], [], 1       # offset 1 float: 4-byte aligned only
    for (r, c), gh, bh in zip(shapes, g_host, b_host):
        vg = flat_g[off:off + r * c].view(r, c)
        vb = flat_b[off:off + r * c].view(r, c)
        vg.copy_(torch.from_numpy(gh))
        vb.copy_(torch.from_numpy(bh))
        views_g.append(vg)
        views_b.append(vb)
        off += r * c
    outs = muon.ns5_batched(views_g, bufs=views_b, mu=0.9)
    torch.cuda.synchronize()
    for k in range(len(shapes)):
        nb, u = oracle.momentum_nesterov(g_host[k], b_host[k], 0.9)
        assert parity.ulp_diff32(parity.to_np(views_b[k]), nb).max() <= 1
        parity.assert_ns5_parity(parity.to_np(outs[k]), oracle.ns5(u), f"ragged {shapes[k]}")


# ---------------------------------------------------------------- other coefficients

def test_newton_schulz_with_ns5_coefficients_is_ns5(muon):
    """muon_newton_schulz_batched with NS5's coefficients gives exactly what
    muon_ns5_batched gives."""
    rng = np.random.default_rng(41)
    shapes = [(64, 128), (130, 65), (300, 768), (3, 5)]
    Gs = [cuda(rng.standard_normal(s).astype(np.float32)) for s in shapes]
    want = muon.ns5_batched(Gs)
    got = muon.ns5_batched(Gs, coeffs=muon.NS5_COEFFS)
    torch.cuda.synchronize()
    for k, (w, g) in enumerate(zip(want, got)):
        assert torch.equal(w, g), f"matrix {k} {shapes[k]}"


@pytest.mark.parametrize("coeffs,steps", [((1.5, -0.5, 0.0), 12), ((2.0, -1.5, 0.5), 3)],
                         ids=["cubic", "other"])
def test_newton_schulz_coefficients_parity(muon, coeffs, steps):
    """Other coefficients meet the parity bar against the oracle run with the
    same coefficients, for wide, tall and tile-ragged shapes."""
    rng = np.random.default_rng(43)
    shapes = [(64, 128), (128, 64), (200, 520), (520, 200), (768, 768)]
    host = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    outs = muon.ns5_batched([cuda(h) for h in host], steps=steps, coeffs=coeffs)
    torch.cuda.synchronize()
    for h, o, s in zip(host, outs, shapes):
        want = oracle.ns5(h, steps=steps, coeffs=coeffs)
        parity.assert_ns5_parity(parity.to_np(o), want, f"{coeffs} {s}")


def test_newton_schulz_identity_coefficients(muon):
    """(1, 0, 0) leaves the normalised input unchanged, bit for bit."""
    rng = np.random.default_rng(47)
    Gs = [cuda(rng.standard_normal(s).astype(np.float32)) for s in [(70, 90), (90, 70), (256, 256)]]
    want = muon.ns5_batched(Gs, steps=0)
    got = muon.ns5_batched(Gs, steps=3, coeffs=(1.0, 0.0, 0.0))
    torch.cuda.synchronize()
    for w, g in zip(want, got):
        assert torch.equal(w, g)


# ---------------------------------------------------------------- the step with its update

def _apply_reference(p, O, lr):
    """p - lr*O with one float32 rounding, from the GPU's own O: lr*O is exact
    in float64 (O is bf16-valued) and so is the difference at these
    magnitudes, so rounding it to float32 is the fused multiply-add."""
    return (p.astype(np.float64) - np.float64(np.float32(lr)) * O.astype(np.float64)).astype(np.float32)


def _ulp32(x):
    x = np.abs(np.asarray(x, dtype=np.float32))
    return (np.nextafter(x, np.float32(np.inf)) - x).astype(np.float64)


@pytest.mark.parametrize("steps", [5, 0])
def test_apply_step_updates_parameters(muon, steps):
    """muon_momentum_ns5_apply_batched against the oracle's whole step
    (oracle.muon_step_apply): the buffers within 1 float32 ulp and the
    parameters within lr times the NS5 parity bar plus one float32 ulp per
    entry.  Against the step without the update, the buffers are bitwise
    equal and the parameters are p - lr * O with that step's O (one float32
    rounding)."""
    rng = np.random.default_rng(51)
    shapes = [(64, 128), (128, 64), (200, 520), (520, 200), (3, 5), (768, 768), (33, 17)]
    gs = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    bs = [(0.1 * rng.standard_normal(s)).astype(np.float32) for s in shapes]
    ps = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    lr = 0.02
    b1 = [cuda(b) for b in bs]
    outs = muon.ns5_batched([cuda(g) for g in gs], steps=steps, bufs=b1, mu=0.9)
    b2 = [cuda(b) for b in bs]
    p2 = [cuda(p) for p in ps]
    muon.ns5_batched([cuda(g) for g in gs], p2, steps=steps, bufs=b2, mu=0.9, lr=lr)
    torch.cuda.synchronize()
    want_b, want_p = oracle.muon_step_apply(gs, bs, ps, mu=0.9, lr=lr, steps=steps)
    _, want_o = oracle.muon_step(gs, bs, mu=0.9, steps=steps)
    for k, s in enumerate(shapes):
        assert torch.equal(b1[k], b2[k]), f"buffers {s}"
        assert parity.ulp_diff32(parity.to_np(b2[k]), want_b[k]).max() <= 1, f"buffers {s}"
        got = parity.to_np(p2[k]).astype(np.float64)
        err = np.linalg.norm(got - want_p[k])
        tol = parity.REL_FRO_TOL if steps else 2.0 ** -8  # steps = 0: X0, within one bf16 ulp
        bound = lr * tol * np.linalg.norm(want_o[k].astype(np.float64)) + np.linalg.norm(_ulp32(want_p[k]))
        assert err <= bound, f"update {s}: {err:.4g} > {bound:.4g}"
        O = parity.to_np(outs[k])
        d = parity.ulp_diff32(parity.to_np(p2[k]), _apply_reference(ps[k], O, lr))
        assert d.max() <= 1 and np.mean(d == 0) >= 0.999, f"update {s}"
        if steps:
            parity.assert_ns5_parity(O, want_o[k], f"O {s}")


# ---------------------------------------------------------------- bfloat16 in, bfloat16 out

@pytest.mark.parametrize("steps", [5, 0])
def test_bf16_inputs_give_bf16_outputs(muon, steps):
    """muon_ns5_batched_bf16: the output is the last iterate in G's dtype.  It
    agrees with the float32 entry point on the same values but for rare ties
    of the norm's summation order, is no further from the oracle than that
    path is, and meets the parity bar; odd widths take the unaligned paths.
    The bar of each small input is the stated one unless the oracle's
    algorithm evaluated with float32 accumulation (tests/fp32_model.py) lands
    beyond it on the CPU: then 1.25 times that distance (the 33 x 17 input,
    where the model lands 1.49e-2 from the oracle)."""
    from .test_fp32_model import bf16_io_inputs
    inputs = bf16_io_inputs()
    shapes, host = list(inputs), list(inputs.values())
    G16 = [torch.from_numpy(h).to("cuda").to(torch.bfloat16) for h in host]
    out16 = muon.ns5_batched(G16, steps=steps)
    out32 = muon.ns5_batched([cuda(h) for h in host], steps=steps)
    torch.cuda.synchronize()
    for h, o16, o32, s in zip(host, out16, out32, shapes):
        assert o16.dtype == torch.bfloat16 and tuple(o16.shape) == s
        got = o16.float().cpu().numpy()
        d = parity.bf16_ulp_diff(got, parity.to_np(o32))
        assert np.mean(d == 0) >= 0.999, f"{s}: {np.mean(d != 0):.3%} differ from the float32 path"
        want = oracle.ns5(h, steps=steps)
        if steps:
            assert parity.rel_fro(got, want) <= parity.rel_fro(parity.to_np(o32), want) + 1e-3, s
            bar = parity.model_bar(h) if h.size <= 20000 else (parity.REL_FRO_TOL, parity.SIGMA_TOL)
            r = parity.assert_ns5_parity(got, want, f"bf16 {s}", bar=bar)
            print(f"bf16 {s}: relative Frobenius {r:.3g} (bar {bar[0]:.3g})", flush=True)
        else:
            d = parity.bf16_ulp_diff(got, want)
            assert d.max() <= 1 and np.mean(d == 0) >= 0.999


def test_single_and_grouped_calls_take_bf16(muon):
    """muon_ns5 and muon_ns5_grouped with MUON_BF16: bitwise what the batched
    bf16 entry point (checked against the oracle above) gives the same
    matrices, with bf16 outputs; in place too."""
    rng = np.random.default_rng(16)
    one = torch.from_numpy(rng.standard_normal((96, 200)).astype(np.float32)).to("cuda").to(torch.bfloat16)
    got = muon.ns5(one)
    assert got.dtype == torch.bfloat16
    assert torch.equal(got, muon.ns5_batched([one])[0])
    group = [torch.from_numpy(rng.standard_normal((300, 130)).astype(np.float32)).to("cuda").to(torch.bfloat16)
             for _ in range(5)]
    outs = muon.ns5_grouped(group)
    want = muon.ns5_batched(group)
    for k in range(len(group)):
        assert outs[k].dtype == torch.bfloat16 and torch.equal(outs[k], want[k]), k
    inplace = [g.clone() for g in group]
    muon.ns5_grouped(inplace, outs=inplace)
    for k in range(len(group)):
        assert torch.equal(inplace[k], want[k]), k


# ---------------------------------------------------------------- grouped momentum

def test_momentum_grouped_ragged_misaligned_and_passes(muon):
    """Nesterov momentum over 70 arrays of ragged sizes in one call (two
    launches of at most 64): misaligned views, an empty entry, u aliasing g;
    every result within 1 float32 ulp of the oracle, the rest untouched."""
    rng = np.random.default_rng(77)
    sizes = [int(x) for x in rng.integers(1, 5000, size=70)]
    sizes[5] = 0
    sizes[9] = 768 * 768
    offs = [k % 3 for k in range(70)]
    gh = [rng.standard_normal(n + o).astype(np.float32) for n, o in zip(sizes, offs)]
    bh = [(0.1 * rng.standard_normal(n + o)).astype(np.float32) for n, o in zip(sizes, offs)]
    gd = [cuda(x) for x in gh]
    bd = [cuda(x) for x in bh]
    gv = [t[o:] for t, o in zip(gd, offs)]
    bv = [t[o:] for t, o in zip(bd, offs)]
    us = [g if k % 4 == 0 else torch.empty_like(g) for k, g in enumerate(gv)]   # every 4th in place
    muon.momentum_nesterov_grouped(gv, bv, us, mu=0.9)
    torch.cuda.synchronize()
    for k, (n, o) in enumerate(zip(sizes, offs)):
        want_b, want_u = oracle.momentum_nesterov(gh[k][o:], bh[k][o:], 0.9)
        assert parity.ulp_diff32(parity.to_np(bv[k]), want_b).max(initial=0) <= 1, k
        assert parity.ulp_diff32(parity.to_np(us[k]), want_u).max(initial=0) <= 1, k
        if o:
            assert parity.to_np(bd[k])[:o].tolist() == bh[k][:o].tolist()


def test_large_matrices_deterministic_and_equal_single_calls(muon):
    """m >= 2048 (256 tiles throughout): the result is the same on every call
    and for every batch a matrix is part of, and matches the oracle."""
    shapes = [(2048, 2048), (2048, 2304), (2304, 2048), (2048, 2048)]
    rng = np.random.default_rng(2048)
    host = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    Gs = [cuda(h) for h in host]
    outs = [parity.to_np(o) for o in muon.ns5_batched(Gs)]
    again = [parity.to_np(o) for o in muon.ns5_batched(Gs)]
    for a, b in zip(outs, again):
        assert np.array_equal(a, b)
    _bitwise_equal_to_single(muon, Gs[:3], [cuda(o) for o in outs[:3]])
    parity.assert_ns5_parity(outs[0], oracle.ns5(host[0]), "2048x2048")
    parity.assert_ns5_parity(outs[2], oracle.ns5(host[2]), "2304x2048")


def test_two_4096_matrices_equal_single_calls(muon):
    """Two 4096 x 4096 matrices in one call (symmetric products on 192 tiles
    over m padded to 4224, two matrices per launch) give bitwise what each
    gets alone."""
    g = torch.Generator(device="cuda").manual_seed(4096)
    Gs = [torch.randn(4096, 4096, device="cuda", generator=g) for _ in range(2)]
    outs = muon.ns5_batched(Gs)
    for k, G in enumerate(Gs):
        assert torch.equal(outs[k], muon.ns5(G)), k
        assert torch.isfinite(outs[k]).all()


# The one-launch path of small matrices at the edges of its range (short side
# up to 64, long side up to 256: four 32-wide blocks of X per wave at 256) and
# just past them (the tiled path), in one batch and one by one.
SMALL_EDGE_SHAPES = [(64, 256), (256, 64), (33, 250), (1, 256), (64, 225), (64, 257), (65, 256), (2, 1)]


def test_small_range_edges(muon):
    rng = np.random.default_rng(2024)
    host = [rng.standard_normal(sh).astype(np.float32) for sh in SMALL_EDGE_SHAPES]
    bufs = [(0.1 * rng.standard_normal(sh)).astype(np.float32) for sh in SMALL_EDGE_SHAPES]
    Gs = [cuda(h) for h in host]
    bd = [cuda(b) for b in bufs]
    outs = muon.ns5_batched(Gs, bufs=bd, mu=0.95)
    torch.cuda.synchronize()
    for k, sh in enumerate(SMALL_EDGE_SHAPES):
        b1 = cuda(bufs[k])
        single = muon.ns5_batched([Gs[k]], bufs=[b1], mu=0.95)[0]
        assert torch.equal(single, outs[k]) and torch.equal(b1, bd[k]), f"{sh}: batched differs from single"
        want_b, want_u = oracle.momentum_nesterov(host[k], bufs[k], 0.95)
        assert parity.ulp_diff32(parity.to_np(bd[k]), want_b).max() <= 1, sh
        got = parity.to_np(outs[k])
        bar = parity.model_bar(want_u) if want_u.size <= 20000 else (parity.REL_FRO_TOL, parity.SIGMA_TOL)
        parity.assert_ns5_parity(got, oracle.ns5(want_u), f"{sh}", check_sigma=min(sh) > 1, bar=bar)
        assert parity.is_bf16_valued(got)


# Batches the library runs as several parts on several streams (one launch
# group, at least 5e11 nominal flops), with segments that the parts cannot
# share evenly (tests/test_split_plan.py checks on the CPU that these batches
# are split and how).
SPLIT_BATCHES = {
    # 20 matrices of the 768 class, 7.6e11 nominal flops, 5.7e-5 elements per
    # flop: three parts; segments of 13, 5 and 2 go 5/4/4, 1/2/2 and 1/1/0
    "three-parts-uneven": [(768, 3072)] * 13 + [(3072, 768)] * 5 + [(768, 768)] * 2,
    # eight shapes of one matrix each, 5.9e11 nominal flops: three parts of
    # 3, 3 and 2 (the round-robin runs on across segments)
    "three-parts-one-per-shape": [(768, n) for n in range(4096, 8192, 512)],
    # five 2048^2 matrices, 1.3e12 nominal flops, 1.6e-5 elements per flop:
    # two parts of 3 and 2
    "two-parts-uneven": [(2048, 2048)] * 5,
}


@pytest.mark.parametrize("name", sorted(SPLIT_BATCHES))
def test_split_batches_equal_single_calls(muon, name):
    """The fused step over a batch that runs as parts on several streams:
    every matrix's update and new momentum buffer are bitwise what a call on
    that matrix alone gives, and a second call gives the same again."""
    shapes = SPLIT_BATCHES[name]
    rng = np.random.default_rng(91)
    host_g = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    host_b = [(0.1 * rng.standard_normal(s)).astype(np.float32) for s in shapes]
    Gs = [cuda(h) for h in host_g]
    bufs = [cuda(h) for h in host_b]
    outs = muon.ns5_batched(Gs, bufs=bufs, mu=0.95)
    bufs2 = [cuda(h) for h in host_b]
    again = muon.ns5_batched(Gs, bufs=bufs2, mu=0.95)
    torch.cuda.synchronize()
    for k, G in enumerate(Gs):
        assert torch.equal(outs[k], again[k]) and torch.equal(bufs[k], bufs2[k]), f"{name}: matrix {k} differs between calls"
        b = cuda(host_b[k])
        o = muon.ns5_batched([G], bufs=[b], mu=0.95)[0]
        assert torch.equal(o, outs[k]), f"{name}: update {k} {tuple(G.shape)} differs from its single call"
        assert torch.equal(b, bufs[k]), f"{name}: buffer {k} {tuple(G.shape)} differs from its single call"
        assert torch.isfinite(o).all().item(), k


@pytest.mark.parametrize("shapes", [
    # 16 x 36 upper 256 tiles in X X^T and b A + c A A (2.25 rounds of 256
    # CUs); alone, a 2048^2 matrix takes 192 tiles for them
    [(2048, 2048)] * 16,
    # three segments, two K lengths in X X^T (2048 and 4096), tall matrices
    [(2048, 2048)] * 12 + [(2048, 4096)] * 6 + [(4096, 2048)] * 6,
], ids=["16x2048^2", "mixed-K"])
def test_batches_of_2048_class_matrices_equal_single_calls(muon, shapes):
    """Batches of 2048-class matrices, whose symmetric products run several
    rounds of 256 x 256 tiles, give every matrix bitwise what a single call
    (192 tiles for a lone 2048^2) gives it, the same on every call."""
    rng = np.random.default_rng(77)
    host = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    Gs = [cuda(h) for h in host]
    outs = muon.ns5_batched(Gs)
    again = muon.ns5_batched(Gs)
    for k, (a, b) in enumerate(zip(outs, again)):
        assert torch.equal(a, b), f"matrix {k} differs between two calls"
        assert torch.isfinite(a).all(), k
    _bitwise_equal_to_single(muon, Gs, outs)
