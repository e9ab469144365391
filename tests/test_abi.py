"""The C ABI without a GPU: libmuon.so loads, exports every function that
include/muon.h declares, sizes workspaces, and rejects invalid arguments
before it touches the HIP runtime (no kernel is launched here)."""

import ctypes
import os
import re

import pytest

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "muon.h")


@pytest.fixture(scope="module")
def muon():
    from newton_schulz_09_amd import muon as m
    return m


def _declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(muon_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for need in ("muon_momentum_nesterov", "muon_ns5", "muon_ns5_grouped", "muon_ns5_workspace_size"):
        assert need in names


def test_library_exports_every_declared_symbol(muon):
    declared = _declared_functions()
    assert sorted(muon.EXPORTS) == declared
    for name in declared:
        assert hasattr(muon.lib, name), name


def test_workspace_size(muon):
    # X twice (bf16, padded to the tile) + A, B + norm partials
    s = muon.workspace_size(64, 128, 1)
    assert s >= 2 * 64 * 128 * 2 + 2 * 64 * 64 * 2
    assert muon.workspace_size(128, 64, 1) == s               # orientation-independent
    assert muon.workspace_size(768, 2304, 12) > 12 * (2 * 768 * 2304 + 2 * 768 * 768) * 2
    assert muon.workspace_size(768, 2304, 500) == muon.workspace_size(768, 2304, 128)
    assert muon.workspace_size(0, 5, 1) == 0
    assert muon.workspace_size(5, 5, 0) == 0
    assert muon.workspace_size(20000, 20000, 1) == 0           # short side beyond the limit
    assert muon.workspace_size(1, 1, 1) > 0


def test_shape_limits(muon):
    S, L = muon.MAX_SHORT, muon.MAX_LONG
    for rows, cols in ((S, S), (16, L), (L, 16), (S, L), (L, S)):
        assert muon.workspace_size(rows, cols, 1) > 0, (rows, cols)
    for rows, cols in ((S + 1, S + 1), (16, L + 1), (L + 1, 16), (S + 1, L)):
        assert muon.workspace_size(rows, cols, 1) == 0, (rows, cols)
    # the largest accepted shape: two copies of X (bf16, 16384 x >= 2^20) alone
    # pass 2^36 bytes, so every size on the way is 64-bit
    big = muon.workspace_size(S, L, 1)
    assert big >= 2 * S * L * 2 + 2 * S * S * 2
    assert big < 2 * (2 * S * (L + 1024) * 2 + 2 * (S + 1024) ** 2 * 2)
    assert muon.workspace_size(S, L, 2) >= 2 * big - 256


def test_validation_errors_before_any_launch(muon):
    lib = muon.lib
    fake = ctypes.c_void_p(0x100000)            # never dereferenced: calls fail validation first
    ws_small = ctypes.c_void_p(0x200000)
    # momentum
    assert lib.muon_momentum_nesterov(None, None, None, 0, 0.95, None) == muon.MUON_OK
    assert lib.muon_momentum_nesterov(None, fake, fake, 4, 0.95, None) == muon.MUON_ERR_INVALID_ARG
    assert lib.muon_momentum_nesterov(fake, fake, fake, -1, 0.95, None) == muon.MUON_ERR_INVALID_ARG
    assert lib.muon_momentum_nesterov(fake, fake, fake, 8, 0.95, None) == muon.MUON_ERR_INVALID_ARG  # u == buf
    assert b"alias" in lib.muon_last_error()
    # ns5
    need = muon.workspace_size(64, 128, 1)
    assert lib.muon_ns5(None, fake, 64, 128, muon.MUON_F32, 5, 1e-7, ws_small, need, None) == muon.MUON_ERR_INVALID_ARG
    assert lib.muon_ns5(fake, fake, 0, 128, muon.MUON_F32, 5, 1e-7, ws_small, need, None) == muon.MUON_ERR_INVALID_ARG
    assert lib.muon_ns5(fake, fake, 64, 128, muon.MUON_F32, -1, 1e-7, ws_small, need, None) == muon.MUON_ERR_INVALID_ARG
    assert lib.muon_ns5(fake, fake, 64, 128, muon.MUON_F32, 5, float("nan"), ws_small, need, None) == muon.MUON_ERR_INVALID_ARG
    assert lib.muon_ns5(fake, fake, 64, 128, muon.MUON_F32, 5, 1e-7, None, need, None) == muon.MUON_ERR_WORKSPACE
    assert lib.muon_ns5(fake, fake, 64, 128, muon.MUON_F32, 5, 1e-7, ctypes.c_void_p(0x200010), need, None) \
        == muon.MUON_ERR_WORKSPACE
    assert lib.muon_ns5(fake, fake, 64, 128, muon.MUON_F32, 5, 1e-7, ws_small, need - 1, None) == muon.MUON_ERR_WORKSPACE
    assert b"needed" in lib.muon_last_error()
    assert lib.muon_ns5(fake, fake, 64, 128, 2, 5, 1e-7, ws_small, need, None) == muon.MUON_ERR_INVALID_ARG
    assert b"dtype" in lib.muon_last_error()
    # a bf16 matrix needs the same workspace
    assert lib.muon_ns5(fake, fake, 64, 128, muon.MUON_BF16, 5, 1e-7, ws_small, need - 1, None) \
        == muon.MUON_ERR_WORKSPACE
    assert lib.muon_ns5(fake, fake, 1 << 15, 1 << 15, muon.MUON_F32, 5, 1e-7, ws_small, 1 << 40, None) \
        == muon.MUON_ERR_UNSUPPORTED
    # grouped
    arr = (ctypes.c_void_p * 2)(0x100000, 0)
    ok = (ctypes.c_void_p * 2)(0x100000, 0x100100)
    need2 = muon.workspace_size(64, 128, 2)
    assert lib.muon_ns5_grouped(ok, arr, 2, 64, 128, muon.MUON_F32, 5, 1e-7, ws_small, need2, None) == muon.MUON_ERR_INVALID_ARG
    assert lib.muon_ns5_grouped(ok, ok, 0, 64, 128, muon.MUON_F32, 5, 1e-7, ws_small, need2, None) == muon.MUON_ERR_INVALID_ARG
    assert lib.muon_ns5_grouped(None, ok, 2, 64, 128, muon.MUON_F32, 5, 1e-7, ws_small, need2, None) == muon.MUON_ERR_INVALID_ARG
    assert lib.muon_ns5_grouped(ok, ok, 2, 64, 128, muon.MUON_F32, 5, 1e-7, ws_small, need2 - 256, None) \
        == muon.MUON_ERR_WORKSPACE


def test_status_strings(muon):
    for code in range(5):
        assert muon.lib.muon_status_string(code)
    assert muon.lib.muon_status_string(99) == b"unknown status"


def test_binding_rejects_cpu_tensors(muon):
    import torch
    g = torch.zeros(4)
    with pytest.raises(ValueError):
        muon.momentum_nesterov(g, g.clone())
    with pytest.raises(ValueError):
        muon.ns5(torch.zeros(4, 4))


def test_batched_workspace_size(muon):
    shapes = [(768, 2304), (768, 768), (768, 3072), (3072, 768)] * 12
    s = muon.batched_workspace_size(shapes)
    # the four shape classes share one pass: at least the sum of their grouped needs
    assert s >= sum(muon.workspace_size(r, c, 12) for r, c in shapes[:4]) - 4 * 256
    assert muon.batched_workspace_size([(64, 128)]) == muon.workspace_size(64, 128, 1)
    assert muon.batched_workspace_size([(0, 5)]) == 0
    assert muon.batched_workspace_size([(64, 128), (20000, 20000)]) == 0
    i64 = ctypes.c_int64
    assert muon.lib.muon_ns5_batched_workspace_size(None, None, 1) == 0
    assert muon.lib.muon_ns5_batched_workspace_size((i64 * 1)(4), (i64 * 1)(4), 0) == 0


def test_batched_validation_errors_before_any_launch(muon):
    lib = muon.lib
    i64 = ctypes.c_int64
    fake = ctypes.c_void_p(0x100000)
    ws = ctypes.c_void_p(0x200000)
    g = (ctypes.c_void_p * 2)(0x100000, 0x100100)
    o = (ctypes.c_void_p * 2)(0x300000, 0x300100)
    rows, cols = (i64 * 2)(64, 130), (i64 * 2)(128, 65)
    need = lib.muon_ns5_batched_workspace_size(rows, cols, 2)
    assert need > 0
    assert lib.muon_ns5_batched(None, o, rows, cols, 2, 5, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert lib.muon_ns5_batched(g, o, None, cols, 2, 5, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert lib.muon_ns5_batched(g, o, rows, cols, 0, 5, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert lib.muon_ns5_batched(g, o, rows, cols, 2, -1, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    bad = (i64 * 2)(64, 0)
    assert lib.muon_ns5_batched(g, o, bad, cols, 2, 5, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert b"matrix 1" in lib.muon_last_error()
    nullo = (ctypes.c_void_p * 2)(0x300000, 0)
    assert lib.muon_ns5_batched(g, nullo, rows, cols, 2, 5, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert lib.muon_ns5_batched(g, o, rows, cols, 2, 5, 1e-7, ws, need - 256, None) == muon.MUON_ERR_WORKSPACE
    assert lib.muon_ns5_batched(g, o, rows, cols, 2, 5, 1e-7, None, need, None) == muon.MUON_ERR_WORKSPACE
    huge = (i64 * 2)(64, 1 << 15)
    assert lib.muon_ns5_batched(g, o, huge, (i64 * 2)(128, 1 << 15), 2, 5, 1e-7, ws, 1 << 40, None) \
        == muon.MUON_ERR_UNSUPPORTED
    ev = (ctypes.c_void_p * 1)()
    rec = ctypes.c_int(7)
    assert lib.muon_ns5_batched_timed(g, o, None, 0.95, rows, cols, 2, 5, 1e-7, ws, need, None, None, 1,
                                      ctypes.byref(rec)) == muon.MUON_ERR_INVALID_ARG
    assert rec.value == 0
    del fake, ev


def test_fused_step_validation_errors_before_any_launch(muon):
    lib = muon.lib
    i64 = ctypes.c_int64
    ws = ctypes.c_void_p(0x200000)
    g = (ctypes.c_void_p * 2)(0x100000, 0x100100)
    b = (ctypes.c_void_p * 2)(0x400000, 0x400100)
    o = (ctypes.c_void_p * 2)(0x300000, 0x300100)
    rows, cols = (i64 * 2)(64, 130), (i64 * 2)(128, 65)
    need = lib.muon_ns5_batched_workspace_size(rows, cols, 2)
    call = lib.muon_momentum_ns5_batched
    assert call(g, None, o, rows, cols, 2, 0.95, 5, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    nullb = (ctypes.c_void_p * 2)(0x400000, 0)
    assert call(g, nullb, o, rows, cols, 2, 0.95, 5, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert b"momentum buffer" in lib.muon_last_error()
    alias = (ctypes.c_void_p * 2)(0x400000, 0x300100)       # out[1] == buf[1]
    assert call(g, alias, o, rows, cols, 2, 0.95, 5, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert b"alias" in lib.muon_last_error()
    assert call(g, b, o, rows, cols, 2, 0.95, 5, 1e-7, ws, need - 256, None) == muon.MUON_ERR_WORKSPACE
    assert call(g, b, o, rows, cols, 0, 0.95, 5, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG


def test_static_workspace_validation_errors_before_any_device_call(muon):
    """muon_momentum_ns5_batched_static validates every argument, and checks
    that each matrix fits in the library's static workspace, before it looks
    up that workspace on the device: these run on a host with no GPU."""
    lib = muon.lib
    i64 = ctypes.c_int64
    g = (ctypes.c_void_p * 2)(0x100000, 0x100100)
    b = (ctypes.c_void_p * 2)(0x400000, 0x400100)
    o = (ctypes.c_void_p * 2)(0x300000, 0x300100)
    rows, cols = (i64 * 2)(64, 130), (i64 * 2)(128, 65)
    call = lib.muon_momentum_ns5_batched_static
    assert call(g, None, o, rows, cols, 2, 0.95, 5, 1e-7, None) == muon.MUON_ERR_INVALID_ARG
    nullb = (ctypes.c_void_p * 2)(0x400000, 0)
    assert call(g, nullb, o, rows, cols, 2, 0.95, 5, 1e-7, None) == muon.MUON_ERR_INVALID_ARG
    alias = (ctypes.c_void_p * 2)(0x400000, 0x300100)       # out[1] == buf[1]
    assert call(g, alias, o, rows, cols, 2, 0.95, 5, 1e-7, None) == muon.MUON_ERR_INVALID_ARG
    assert call(g, b, o, rows, cols, 0, 0.95, 5, 1e-7, None) == muon.MUON_ERR_INVALID_ARG
    assert call(g, b, o, rows, cols, 2, 0.95, -1, 1e-7, None) == muon.MUON_ERR_INVALID_ARG
    assert call(g, b, o, rows, cols, 2, 0.95, 5, float("inf"), None) == muon.MUON_ERR_INVALID_ARG
    # the largest square that fits, and the next step up, which does not
    assert muon.workspace_size(5632, 5632, 1) <= muon.STATIC_WORKSPACE_BYTES < muon.workspace_size(5648, 5648, 1)
    big = (i64 * 2)(5648, 130)
    assert call(g, b, o, big, big, 2, 0.95, 5, 1e-7, None) == muon.MUON_ERR_UNSUPPORTED
    assert b"the library holds" in lib.muon_last_error()
    huge = (i64 * 2)(1 << 15, 64)                           # beyond MUON_NS5_MAX_SHORT
    assert call(g, b, o, huge, huge, 2, 0.95, 5, 1e-7, None) == muon.MUON_ERR_UNSUPPORTED


def test_polar_svd_validation_errors_before_any_launch(muon):
    lib = muon.lib
    ws = ctypes.c_void_p(0x200000)
    g = (ctypes.c_void_p * 2)(0x100000, 0x100100)
    o = (ctypes.c_void_p * 2)(0x300000, 0x300100)
    need = lib.muon_polar_svd_workspace_size(64, 128, 2)
    assert need > 0 and lib.muon_polar_svd_workspace_size(64, 128, 200) == lib.muon_polar_svd_workspace_size(64, 128, 128)
    assert lib.muon_polar_svd_workspace_size(4097, 5000, 1) == 0          # beyond MUON_POLAR_MAX_SHORT
    assert lib.muon_polar_svd_workspace_size(0, 5, 1) == 0
    call = lib.muon_polar_svd_grouped
    assert call(None, o, 2, 64, 128, 12, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert call(g, o, 0, 64, 128, 12, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert call(g, o, 2, 64, 128, 0, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert call(g, o, 2, 64, 128, 65, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert call(g, o, 2, 5000, 5000, 12, ws, 1 << 40, None) == muon.MUON_ERR_UNSUPPORTED
    assert call(g, o, 2, 64, 128, 12, ws, need - 256, None) == muon.MUON_ERR_WORKSPACE


def test_coefficient_validation_errors_before_any_launch(muon):
    lib = muon.lib
    i64 = ctypes.c_int64
    ws = ctypes.c_void_p(0x200000)
    g = (ctypes.c_void_p * 2)(0x100000, 0x100100)
    o = (ctypes.c_void_p * 2)(0x300000, 0x300100)
    rows, cols = (i64 * 2)(64, 130), (i64 * 2)(128, 65)
    need = lib.muon_ns5_batched_workspace_size(rows, cols, 2)
    call = lib.muon_newton_schulz_batched
    ok = (ctypes.c_float * 3)(1.5, -0.5, 0.0)
    assert call(g, o, rows, cols, 2, 5, None, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert b"coefficient" in lib.muon_last_error()
    nan = (ctypes.c_float * 3)(1.5, float("nan"), 0.0)
    assert call(g, o, rows, cols, 2, 5, nan, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert b"coefficient 1" in lib.muon_last_error()
    assert call(g, o, rows, cols, 2, 5, ok, 1e-7, ws, need - 256, None) == muon.MUON_ERR_WORKSPACE
    assert call(g, o, rows, cols, 2, -1, ok, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert call(None, o, rows, cols, 2, 5, ok, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG


def test_apply_validation_errors_before_any_launch(muon):
    lib = muon.lib
    i64 = ctypes.c_int64
    ws = ctypes.c_void_p(0x200000)
    g = (ctypes.c_void_p * 2)(0x100000, 0x100100)
    b = (ctypes.c_void_p * 2)(0x400000, 0x400100)
    p = (ctypes.c_void_p * 2)(0x300000, 0x300100)
    rows, cols = (i64 * 2)(64, 130), (i64 * 2)(128, 65)
    need = lib.muon_ns5_batched_workspace_size(rows, cols, 2)
    call = lib.muon_momentum_ns5_apply_batched
    assert call(g, b, None, rows, cols, 2, 0.95, 0.02, 5, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert call(g, None, p, rows, cols, 2, 0.95, 0.02, 5, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert call(g, b, p, rows, cols, 2, 0.95, float("inf"), 5, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert b"lr" in lib.muon_last_error()
    alias_g = (ctypes.c_void_p * 2)(0x300000, 0x100100)     # p[1] == g[1]
    assert call(g, b, alias_g, rows, cols, 2, 0.95, 0.02, 5, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert b"gradient" in lib.muon_last_error()
    alias_b = (ctypes.c_void_p * 2)(0x400000, 0x300100)     # p[0] == buf[0]
    assert call(g, b, alias_b, rows, cols, 2, 0.95, 0.02, 5, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    nullp = (ctypes.c_void_p * 2)(0x300000, 0)
    assert call(g, b, nullp, rows, cols, 2, 0.95, 0.02, 5, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert call(g, b, p, rows, cols, 2, 0.95, 0.02, 5, 1e-7, ws, need - 256, None) == muon.MUON_ERR_WORKSPACE


def test_bf16_validation_errors_before_any_launch(muon):
    lib = muon.lib
    i64 = ctypes.c_int64
    ws = ctypes.c_void_p(0x200000)
    g = (ctypes.c_void_p * 2)(0x100000, 0x100100)
    o = (ctypes.c_void_p * 2)(0x300000, 0x300100)
    rows, cols = (i64 * 2)(64, 130), (i64 * 2)(128, 65)
    need = lib.muon_ns5_batched_workspace_size(rows, cols, 2)
    call = lib.muon_ns5_batched_bf16
    assert call(None, o, rows, cols, 2, 5, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert call(g, o, rows, None, 2, 5, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert call(g, o, rows, cols, 2, -1, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert call(g, o, rows, cols, 2, 5, float("nan"), ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert call(g, o, rows, cols, 2, 5, 1e-7, ws, need - 256, None) == muon.MUON_ERR_WORKSPACE


def test_f32_workspace_size(muon):
    # X twice + A, B in float32, padded to the 128 tile with a 32-float row skew
    s = muon.f32_workspace_size([(64, 128)])
    assert s >= 2 * 128 * 160 * 4 + 2 * 128 * 160 * 4
    assert muon.f32_workspace_size([(128, 64)]) == s            # orientation-independent
    one = muon.f32_workspace_size([(768, 2304)])
    assert muon.f32_workspace_size([(768, 2304)] * 12) > 11 * one
    # shapes run one after another: the largest pass sets the size
    assert muon.f32_workspace_size([(768, 2304)] * 12 + [(64, 128)]) == muon.f32_workspace_size([(768, 2304)] * 12)
    assert muon.f32_workspace_size([(768, 2304)] * 500) == muon.f32_workspace_size([(768, 2304)] * 128)
    assert muon.f32_workspace_size([(0, 5)]) == 0
    assert muon.f32_workspace_size([(20000, 20000)]) == 0


def test_f32_validation_errors_before_any_launch(muon):
    lib = muon.lib
    i64 = ctypes.c_int64
    ws = ctypes.c_void_p(0x200000)
    g = (ctypes.c_void_p * 2)(0x100000, 0x100100)
    o = (ctypes.c_void_p * 2)(0x300000, 0x300100)
    rows, cols = (i64 * 2)(64, 130), (i64 * 2)(128, 65)
    need = lib.muon_newton_schulz_f32_workspace_size(rows, cols, 2)
    assert need > 0
    call = lib.muon_newton_schulz_f32_batched
    ok = (ctypes.c_float * 3)(1.5, -0.5, 0.0)
    nan = (ctypes.c_float * 3)(1.5, float("inf"), 0.0)
    assert call(g, o, rows, cols, 2, 5, nan, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert b"coefficient 1" in lib.muon_last_error()
    assert call(g, o, rows, cols, 2, 5, ok, 1e-7, ws, need - 256, None) == muon.MUON_ERR_WORKSPACE
    assert call(g, o, rows, cols, 2, 5, None, 1e-7, ctypes.c_void_p(0x200010), need, None) == muon.MUON_ERR_WORKSPACE
    assert call(g, o, rows, cols, 2, 5, None, 1e-7, None, need, None) == muon.MUON_ERR_WORKSPACE
    assert call(g, o, rows, cols, 2, -1, None, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert call(g, o, rows, cols, 2, 5, None, float("nan"), ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert call(None, o, rows, cols, 2, 5, None, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    assert call(g, o, rows, cols, 0, 5, None, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    bad = (i64 * 2)(64, 0)
    assert call(g, o, bad, cols, 2, 5, None, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    null_o = (ctypes.c_void_p * 2)(0x300000, None)
    assert call(g, null_o, rows, cols, 2, 5, None, 1e-7, ws, need, None) == muon.MUON_ERR_INVALID_ARG
    big = (i64 * 1)(20000)
    assert call(g, o, big, big, 1, 5, None, 1e-7, ws, need, None) == muon.MUON_ERR_UNSUPPORTED


def test_grouped_momentum_validation_errors_before_any_launch(muon):
    lib = muon.lib
    i64 = ctypes.c_int64
    vp = ctypes.c_void_p
    g = (vp * 2)(0x100000, 0x100100)
    b = (vp * 2)(0x200000, 0x200100)
    u = (vp * 2)(0x300000, 0x300100)
    n = (i64 * 2)(16, 7)
    call = lib.muon_momentum_nesterov_grouped
    assert call(None, None, None, None, 0, 0.95, None) == muon.MUON_OK          # nothing to do
    assert call(g, b, u, n, -1, 0.95, None) == muon.MUON_ERR_INVALID_ARG
    assert call(None, b, u, n, 2, 0.95, None) == muon.MUON_ERR_INVALID_ARG
    assert call(g, b, u, None, 2, 0.95, None) == muon.MUON_ERR_INVALID_ARG
    assert call(g, b, u, (i64 * 2)(16, -3), 2, 0.95, None) == muon.MUON_ERR_INVALID_ARG
    assert b"numel[1]" in lib.muon_last_error()
    assert call(g, b, (vp * 2)(0x300000, 0x200100), n, 2, 0.95, None) == muon.MUON_ERR_INVALID_ARG
    assert b"alias" in lib.muon_last_error()
    assert call((vp * 2)(0x100000, None), b, u, n, 2, 0.95, None) == muon.MUON_ERR_INVALID_ARG
    # an empty entry may carry null pointers; with every entry empty nothing is launched
    assert call((vp * 2)(None, None), (vp * 2)(None, None), (vp * 2)(None, None), (i64 * 2)(0, 0), 2, 0.95,
                None) == muon.MUON_OK
