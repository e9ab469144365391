"""Python binding of libmuon.so (C ABI in include/muon.h).

Argument marshalling only: every step of momentum and NS5 runs in the HIP
kernels of the library.  PyTorch supplies device memory (the tensors and a
cached workspace) and the current HIP stream.  Importing this module raises
if the library has not been built (``python -m newton_schulz_09_amd.build``);
there is no fallback.
"""

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmuon.so")

MUON_OK = 0
MUON_ERR_INVALID_ARG = 1
MUON_ERR_UNSUPPORTED = 2
MUON_ERR_WORKSPACE = 3
MUON_ERR_HIP = 4
# muon_dtype: the element type of muon_ns5 / muon_ns5_grouped
MUON_F32 = 0
MUON_BF16 = 1

NS5_STEPS = 5
NS5_EPS = 1e-7
#: (a, b, c) of NS5 (MUON_NS5_A/B/C) and of the classic cubic Newton-Schulz
#: iteration X <- 1.5 X - 0.5 X X^T X, whose singular values converge to 1.
NS5_COEFFS = (3.4445, -4.7750, 2.0315)
CUBIC_COEFFS = (1.5, -0.5, 0.0)
MAX_GROUP = 128
#: Accepted shapes (MUON_NS5_MAX_SHORT / MUON_NS5_MAX_LONG): short side <=
#: MAX_SHORT and long side <= MAX_LONG.
MAX_SHORT = 16384
MAX_LONG = 1 << 20

#: Every symbol include/muon.h declares.
EXPORTS = ("muon_momentum_nesterov", "muon_momentum_nesterov_grouped", "muon_ns5_workspace_size", "muon_ns5", "muon_ns5_grouped",
           "muon_ns5_batched_workspace_size", "muon_ns5_batched", "muon_newton_schulz_batched",
           "muon_ns5_batched_bf16", "muon_momentum_ns5_batched", "muon_momentum_ns5_apply_batched",
           "muon_ns5_batched_timed", "muon_newton_schulz_f32_workspace_size", "muon_newton_schulz_f32_batched",
           "muon_momentum_ns5_batched_static", "muon_polar_svd_workspace_size", "muon_polar_svd_grouped",
           "muon_status_string", "muon_last_error")
#: Largest short side of polar_svd_grouped (MUON_POLAR_MAX_SHORT).
POLAR_MAX_SHORT = 4096
#: Bytes of the device array muon_momentum_ns5_batched_static uses as its
#: workspace (MUON_STATIC_WORKSPACE_BYTES).
STATIC_WORKSPACE_BYTES = 256 << 20


class MuonError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m newton_schulz_09_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    lib.muon_momentum_nesterov.argtypes = [vp, vp, vp, i64, ctypes.c_float, vp]
    lib.muon_momentum_nesterov.restype = ctypes.c_int
    lib.muon_momentum_nesterov_grouped.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                                   ctypes.POINTER(i64), i64, ctypes.c_float, vp]
    lib.muon_momentum_nesterov_grouped.restype = ctypes.c_int
    lib.muon_ns5_workspace_size.argtypes = [i64, i64, i64]
    lib.muon_ns5_workspace_size.restype = sz
    lib.muon_ns5.argtypes = [vp, vp, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_float, vp, sz, vp]
    lib.muon_ns5.restype = ctypes.c_int
    lib.muon_ns5_grouped.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), i64, i64, i64, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_float, vp, sz, vp]
    lib.muon_ns5_grouped.restype = ctypes.c_int
    pi64 = ctypes.POINTER(i64)
    lib.muon_ns5_batched_workspace_size.argtypes = [pi64, pi64, i64]
    lib.muon_ns5_batched_workspace_size.restype = sz
    lib.muon_ns5_batched.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), pi64, pi64, i64, ctypes.c_int,
                                     ctypes.c_float, vp, sz, vp]
    lib.muon_ns5_batched.restype = ctypes.c_int
    lib.muon_newton_schulz_batched.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), pi64, pi64, i64,
                                               ctypes.c_int, ctypes.POINTER(ctypes.c_float), ctypes.c_float, vp,
                                               sz, vp]
    lib.muon_newton_schulz_batched.restype = ctypes.c_int
    lib.muon_ns5_batched_bf16.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), pi64, pi64, i64, ctypes.c_int,
                                          ctypes.c_float, vp, sz, vp]
    lib.muon_ns5_batched_bf16.restype = ctypes.c_int
    lib.muon_momentum_ns5_batched.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp), pi64,
                                              pi64, i64, ctypes.c_float, ctypes.c_int, ctypes.c_float, vp, sz, vp]
    lib.muon_momentum_ns5_batched.restype = ctypes.c_int
    lib.muon_momentum_ns5_apply_batched.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                                    pi64, pi64, i64, ctypes.c_float, ctypes.c_float, ctypes.c_int,
                                                    ctypes.c_float, vp, sz, vp]
    lib.muon_momentum_ns5_apply_batched.restype = ctypes.c_int
    lib.muon_ns5_batched_timed.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                           ctypes.c_float, pi64, pi64, i64, ctypes.c_int, ctypes.c_float, vp, sz,
                                           vp, ctypes.POINTER(vp), ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.muon_ns5_batched_timed.restype = ctypes.c_int
    lib.muon_newton_schulz_f32_workspace_size.argtypes = [pi64, pi64, i64]
    lib.muon_newton_schulz_f32_workspace_size.restype = sz
    lib.muon_newton_schulz_f32_batched.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), pi64, pi64, i64,
                                                   ctypes.c_int, ctypes.POINTER(ctypes.c_float), ctypes.c_float,
                                                   vp, sz, vp]
    lib.muon_newton_schulz_f32_batched.restype = ctypes.c_int
    lib.muon_momentum_ns5_batched_static.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                                     pi64, pi64, i64, ctypes.c_float, ctypes.c_int, ctypes.c_float,
                                                     vp]
    lib.muon_momentum_ns5_batched_static.restype = ctypes.c_int
    lib.muon_polar_svd_workspace_size.argtypes = [i64, i64, i64]
    lib.muon_polar_svd_workspace_size.restype = sz
    lib.muon_polar_svd_grouped.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), i64, i64, i64, ctypes.c_int, vp,
                                           sz, vp]
    lib.muon_polar_svd_grouped.restype = ctypes.c_int
    lib.muon_status_string.argtypes = [ctypes.c_int]
    lib.muon_status_string.restype = ctypes.c_char_p
    lib.muon_last_error.argtypes = []
    lib.muon_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


def _check(status):
    if status != MUON_OK:
        msg = lib.muon_status_string(status).decode()
        detail = lib.muon_last_error().decode()
        raise MuonError(status, f"{msg}: {detail}" if detail else msg)


def _stream_handle(device):
    return torch.cuda.current_stream(device).cuda_stream


def _require_f32_cuda(t, name, dtype=torch.float32):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def momentum_nesterov(g, buf, u=None, mu=0.95):
    """buf <- mu*buf + g ; u <- g + mu*buf (new buf), in one kernel.
    ``u`` may be ``g`` (in-place); returns ``u``."""
    _require_f32_cuda(g, "g")
    _require_f32_cuda(buf, "buf")
    if buf.numel() != g.numel() or buf.device != g.device:
        raise ValueError("g and buf must have the same size and device")
    if u is None:
        u = torch.empty_like(g)
    _require_f32_cuda(u, "u")
    if u.numel() != g.numel() or u.device != g.device:
        raise ValueError("u must have the size and device of g")
    _check(lib.muon_momentum_nesterov(g.data_ptr(), buf.data_ptr(), u.data_ptr(), g.numel(), float(mu),
                                      _stream_handle(g.device)))
    return u


def momentum_nesterov_grouped(gs, bufs, us=None, mu=0.95):
    """Nesterov momentum on lists of float32 tensors (one launch per 64 of
    them): ``bufs`` are updated in place and ``us`` (new tensors unless
    given; ``us[i]`` may be ``gs[i]``) receive the momentum outputs."""
    gs, bufs = list(gs), list(bufs)
    if len(bufs) != len(gs):
        raise ValueError("bufs must match gs in length")
    us = [torch.empty_like(g) for g in gs] if us is None else list(us)
    if len(us) != len(gs):
        raise ValueError("us must match gs in length")
    if not gs:
        return us
    for i, (g, b, u) in enumerate(zip(gs, bufs, us)):
        for t, name in ((g, "gs"), (b, "bufs"), (u, "us")):
            _require_f32_cuda(t, f"{name}[{i}]")
        if b.numel() != g.numel() or u.numel() != g.numel():
            raise ValueError(f"entry {i}: gs, bufs and us must match in size")
        if any(t.device != gs[0].device for t in (g, b, u)):
            raise ValueError("all tensors must be on one device")
    n = len(gs)
    vp = ctypes.c_void_p
    arr = lambda ts: (vp * n)(*[t.data_ptr() for t in ts])  # noqa: E731
    numel = (ctypes.c_int64 * n)(*[g.numel() for g in gs])
    _check(lib.muon_momentum_nesterov_grouped(arr(gs), arr(bufs), arr(us), numel, n, float(mu),
                                              _stream_handle(gs[0].device)))
    return us


def workspace_size(rows, cols, count=1):
    return int(lib.muon_ns5_workspace_size(rows, cols, count))


_workspaces = {}


def _workspace(device, stream, nbytes):
    """A cached uint8 device buffer per (device, stream), grown on demand.
    Calls on one stream are ordered, so they can share it."""
    key = (device.index, stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _dtype_code(t):
    """muon_dtype of a float32 or bfloat16 tensor (others are rejected by
    the checks that follow)."""
    return MUON_BF16 if isinstance(t, torch.Tensor) and t.dtype == torch.bfloat16 else MUON_F32


def ns5(G, out=None, steps=NS5_STEPS, eps=NS5_EPS, workspace=None):
    """Quintic Newton-Schulz orthogonalisation of one 2-D float32 or
    bfloat16 matrix; ``out`` has G's type (bfloat16: the last iterate as is).
    Returns ``out`` (a new tensor unless given; may be ``G``)."""
    code = _dtype_code(G)
    dtype = torch.bfloat16 if code == MUON_BF16 else torch.float32
    _require_f32_cuda(G, "G", dtype)
    if G.dim() != 2:
        raise ValueError("G must be 2-D")
    rows, cols = G.shape
    if out is None:
        out = torch.empty_like(G)
    _require_f32_cuda(out, "out", dtype)
    if out.shape != G.shape or out.device != G.device:
        raise ValueError("out must have G's shape and device")
    need = workspace_size(rows, cols, 1)
    if need == 0:
        raise MuonError(MUON_ERR_UNSUPPORTED, f"shape {rows}x{cols} is not supported")
    stream = _stream_handle(G.device)
    ws = workspace if workspace is not None else _workspace(G.device, stream, need)
    _check(lib.muon_ns5(G.data_ptr(), out.data_ptr(), rows, cols, code, int(steps), float(eps), ws.data_ptr(),
                        ws.numel() * ws.element_size(), stream))
    return out


def ns5_grouped(Gs, outs=None, steps=NS5_STEPS, eps=NS5_EPS, workspace=None):
    """NS5 of a list of same-shaped matrices, all float32 or all bfloat16,
    batched per launch.  Returns the list of outputs (new tensors unless
    given), of the inputs' type."""
    Gs = list(Gs)
    if not Gs:
        return []
    code = _dtype_code(Gs[0])
    dtype = torch.bfloat16 if code == MUON_BF16 else torch.float32
    for i, G in enumerate(Gs):
        _require_f32_cuda(G, f"Gs[{i}]", dtype)
    shape, device = Gs[0].shape, Gs[0].device
    if len(shape) != 2 or any(G.shape != shape or G.device != device for G in Gs):
        raise ValueError("all matrices must be 2-D with the same shape and device")
    outs = _outputs(Gs, outs, dtype)
    rows, cols = shape
    count = len(Gs)
    need = workspace_size(rows, cols, count)
    if need == 0:
        raise MuonError(MUON_ERR_UNSUPPORTED, f"shape {rows}x{cols} is not supported")
    stream = _stream_handle(device)
    ws = workspace if workspace is not None else _workspace(device, stream, need)
    g_ptrs = (ctypes.c_void_p * count)(*[G.data_ptr() for G in Gs])
    o_ptrs = (ctypes.c_void_p * count)(*[o.data_ptr() for o in outs])
    _check(lib.muon_ns5_grouped(g_ptrs, o_ptrs, count, rows, cols, code, int(steps), float(eps), ws.data_ptr(),
                                ws.numel() * ws.element_size(), stream))
    return outs


def _outputs(Gs, outs, dtype=torch.float32):
    if outs is None:
        return [torch.empty_like(G) for G in Gs]
    outs = list(outs)
    if len(outs) != len(Gs):
        raise ValueError("outs must match Gs in length")
    for i, (G, o) in enumerate(zip(Gs, outs)):
        _require_f32_cuda(o, f"outs[{i}]", dtype)
        if o.shape != G.shape or o.device != G.device:
            raise ValueError(f"outs[{i}] must have the shape and device of Gs[{i}]")
    return outs


def batched_workspace_size(shapes):
    n = len(shapes)
    rows = (ctypes.c_int64 * n)(*[int(s[0]) for s in shapes])
    cols = (ctypes.c_int64 * n)(*[int(s[1]) for s in shapes])
    return int(lib.muon_ns5_batched_workspace_size(rows, cols, n))


def ns5_batched(Gs, outs=None, steps=NS5_STEPS, eps=NS5_EPS, workspace=None, events=None, bufs=None, mu=0.95,
                coeffs=None, lr=None):
    """NS5 of a list of float32 matrices of any shapes (one device), with one
    launch per product and NS5 step over all matrices that share a tile size.
    Returns the list of outputs (new tensors unless given).

    ``bufs`` (a list of float32 momentum buffers shaped like ``Gs``): run the
    whole Muon step instead: Gs are gradients, the buffers are updated in
    place (``buf <- mu*buf + g``) and the outputs are NS5 of
    ``u = g + mu*buf``, with momentum and the norm fused in one pass.

    ``events`` (measurement): a list of ``torch.cuda.Event(enable_timing=True)``
    pairs ``[start0, stop0, start1, stop1, ...]``; the library records them
    around the a X + B X launches of the non-final steps.  The number of
    pairs recorded is then available as ``ns5_batched.last_recorded``.

    ``coeffs`` (a, b, c): iterate X <- a X + (b A + c A A) X with these
    coefficients instead of NS5's (muon_newton_schulz_batched), e.g.
    ``CUBIC_COEFFS`` for the classic cubic Newton-Schulz iteration; not
    combined with ``bufs`` or ``events``.

    ``lr`` (with ``bufs``): the Muon step with its update
    (muon_momentum_ns5_apply_batched): ``outs`` are the parameters, updated
    in place to ``p - lr * NS5(u)``; not combined with ``events``.

    bfloat16 ``Gs`` (all of them): NS5 returning bfloat16, the last iterate as
    is (muon_ns5_batched_bf16); only ``outs``, ``steps``, ``eps`` and
    ``workspace`` apply."""
    Gs = list(Gs)
    if not Gs:
        return []
    dtype = Gs[0].dtype if isinstance(Gs[0], torch.Tensor) else torch.float32
    if dtype == torch.bfloat16 and (bufs is not None or events is not None or coeffs is not None or lr is not None):
        raise ValueError("bfloat16 inputs take only outs, steps, eps and workspace")
    if dtype != torch.bfloat16:
        dtype = torch.float32
    for i, G in enumerate(Gs):
        _require_f32_cuda(G, f"Gs[{i}]", dtype)
        if G.dim() != 2:
            raise ValueError(f"Gs[{i}] must be 2-D")
    device = Gs[0].device
    if any(G.device != device for G in Gs):
        raise ValueError("all matrices must be on one device")
    outs = _outputs(Gs, outs, dtype)
    count = len(Gs)
    shapes = [tuple(G.shape) for G in Gs]
    need = batched_workspace_size(shapes)
    if need == 0:
        raise MuonError(MUON_ERR_UNSUPPORTED, "a shape is not supported")
    stream = _stream_handle(device)
    ws = workspace if workspace is not None else _workspace(device, stream, need)
    rows = (ctypes.c_int64 * count)(*[s[0] for s in shapes])
    cols = (ctypes.c_int64 * count)(*[s[1] for s in shapes])
    g_ptrs = (ctypes.c_void_p * count)(*[G.data_ptr() for G in Gs])
    o_ptrs = (ctypes.c_void_p * count)(*[o.data_ptr() for o in outs])
    nbytes = ws.numel() * ws.element_size()
    b_ptrs = None
    if bufs is not None:
        bufs = list(bufs)
        if len(bufs) != count:
            raise ValueError("bufs must match Gs in length")
        for i, (G, b) in enumerate(zip(Gs, bufs)):
            _require_f32_cuda(b, f"bufs[{i}]")
            if b.shape != G.shape or b.device != G.device:
                raise ValueError(f"bufs[{i}] must have the shape and device of Gs[{i}]")
        b_ptrs = (ctypes.c_void_p * count)(*[b.data_ptr() for b in bufs])
    if dtype == torch.bfloat16:
        _check(lib.muon_ns5_batched_bf16(g_ptrs, o_ptrs, rows, cols, count, int(steps), float(eps), ws.data_ptr(),
                                         nbytes, stream))
    elif lr is not None:
        if b_ptrs is None or events is not None or coeffs is not None:
            raise ValueError("lr needs bufs, and is not combined with events or coeffs")
        _check(lib.muon_momentum_ns5_apply_batched(g_ptrs, b_ptrs, o_ptrs, rows, cols, count, float(mu), float(lr),
                                                   int(steps), float(eps), ws.data_ptr(), nbytes, stream))
    elif coeffs is not None:
        if b_ptrs is not None or events is not None:
            raise ValueError("coeffs is not combined with bufs or events")
        k = tuple(float(c) for c in coeffs)
        if len(k) != 3:
            raise ValueError("coeffs must be (a, b, c)")
        _check(lib.muon_newton_schulz_batched(g_ptrs, o_ptrs, rows, cols, count, int(steps), (ctypes.c_float * 3)(*k),
                                              float(eps), ws.data_ptr(), nbytes, stream))
    elif events is None:
        if b_ptrs is None:
            _check(lib.muon_ns5_batched(g_ptrs, o_ptrs, rows, cols, count, int(steps), float(eps), ws.data_ptr(),
                                        nbytes, stream))
        else:
            _check(lib.muon_momentum_ns5_batched(g_ptrs, b_ptrs, o_ptrs, rows, cols, count, float(mu), int(steps),
                                                 float(eps), ws.data_ptr(), nbytes, stream))
    else:
        if len(events) % 2:
            raise ValueError("events must come in (start, stop) pairs")
        ev = (ctypes.c_void_p * max(len(events), 1))(*[e.cuda_event for e in events])
        rec = ctypes.c_int(0)
        _check(lib.muon_ns5_batched_timed(g_ptrs, o_ptrs, b_ptrs, float(mu), rows, cols, count, int(steps),
                                          float(eps), ws.data_ptr(), nbytes, stream, ev, len(events) // 2,
                                          ctypes.byref(rec)))
        ns5_batched.last_recorded = rec.value
    return outs


def momentum_ns5_batched_static(gs, bufs, outs=None, mu=0.95, steps=NS5_STEPS, eps=NS5_EPS):
    """The whole Muon step over float32 matrices of any shapes, as
    ``ns5_batched(gs, outs, bufs=bufs, mu=mu)``, with no workspace argument:
    the library's own device array serves (muon_momentum_ns5_batched_static;
    for callers that cannot allocate, such as code under graph capture).
    ``bufs`` are updated in place; returns the outputs (new tensors unless
    given: pass ``outs`` to allocate nothing here either)."""
    gs, bufs = list(gs), list(bufs)
    if not gs:
        return []
    if len(bufs) != len(gs):
        raise ValueError("bufs must match gs in length")
    for i, (g, b) in enumerate(zip(gs, bufs)):
        _require_f32_cuda(g, f"gs[{i}]")
        _require_f32_cuda(b, f"bufs[{i}]")
        if g.dim() != 2 or b.shape != g.shape or b.device != gs[0].device or g.device != gs[0].device:
            raise ValueError(f"gs[{i}] and bufs[{i}] must be 2-D, of one shape, on one device")
    outs = _outputs(gs, outs)
    n = len(gs)
    vp = ctypes.c_void_p
    arr = lambda ts: (vp * n)(*[t.data_ptr() for t in ts])  # noqa: E731
    rows = (ctypes.c_int64 * n)(*[g.shape[0] for g in gs])
    cols = (ctypes.c_int64 * n)(*[g.shape[1] for g in gs])
    _check(lib.muon_momentum_ns5_batched_static(arr(gs), arr(bufs), arr(outs), rows, cols, n, float(mu), int(steps),
                                                float(eps), _stream_handle(gs[0].device)))
    return outs


def polar_svd_workspace_size(rows, cols, count=1):
    return int(lib.muon_polar_svd_workspace_size(rows, cols, count))


def polar_svd_grouped(Gs, outs=None, max_sweeps=16, workspace=None):
    """U V^T of each same-shaped float32 matrix through an SVD on the GPU
    (muon_polar_svd_grouped: block one-sided Jacobi), the orthogonalisation
    NS5 approximates.  Returns the list of outputs (new tensors unless
    given)."""
    Gs = list(Gs)
    if not Gs:
        return []
    for i, G in enumerate(Gs):
        _require_f32_cuda(G, f"Gs[{i}]")
    shape, device = Gs[0].shape, Gs[0].device
    if len(shape) != 2 or any(G.shape != shape or G.device != device for G in Gs):
        raise ValueError("all matrices must be 2-D with the same shape and device")
    outs = _outputs(Gs, outs)
    rows, cols = shape
    count = len(Gs)
    need = polar_svd_workspace_size(rows, cols, count)
    if need == 0:
        raise MuonError(MUON_ERR_UNSUPPORTED, f"shape {rows}x{cols} is not supported")
    stream = _stream_handle(device)
    ws = workspace if workspace is not None else _workspace(device, stream, need)
    g_ptrs = (ctypes.c_void_p * count)(*[G.data_ptr() for G in Gs])
    o_ptrs = (ctypes.c_void_p * count)(*[o.data_ptr() for o in outs])
    _check(lib.muon_polar_svd_grouped(g_ptrs, o_ptrs, count, rows, cols, int(max_sweeps), ws.data_ptr(),
                                      ws.numel() * ws.element_size(), stream))
    return outs


def f32_workspace_size(shapes):
    n = len(shapes)
    rows = (ctypes.c_int64 * n)(*[int(s[0]) for s in shapes])
    cols = (ctypes.c_int64 * n)(*[int(s[1]) for s in shapes])
    return int(lib.muon_newton_schulz_f32_workspace_size(rows, cols, n))


def newton_schulz_f32(Gs, outs=None, steps=NS5_STEPS, eps=NS5_EPS, coeffs=None, workspace=None):
    """The iteration carried in float32 (muon_newton_schulz_f32_batched): for
    each float32 matrix of ``Gs`` (any shapes, one device), X0 = G / (||G|| +
    eps) in float32 and ``steps`` steps X <- a X + (b A + c A A) X with every
    stored matrix in float32; ``coeffs`` (a, b, c) defaults to NS5's.  Returns
    the list of outputs (new tensors unless given)."""
    Gs = list(Gs)
    if not Gs:
        return []
    for i, G in enumerate(Gs):
        _require_f32_cuda(G, f"Gs[{i}]")
        if G.dim() != 2:
            raise ValueError(f"Gs[{i}] must be 2-D")
    device = Gs[0].device
    if any(G.device != device for G in Gs):
        raise ValueError("all matrices must be on one device")
    outs = _outputs(Gs, outs)
    count = len(Gs)
    shapes = [tuple(G.shape) for G in Gs]
    need = f32_workspace_size(shapes)
    if need == 0:
        raise MuonError(MUON_ERR_UNSUPPORTED, "a shape is not supported")
    stream = _stream_handle(device)
    ws = workspace if workspace is not None else _workspace(device, stream, need)
    rows = (ctypes.c_int64 * count)(*[s[0] for s in shapes])
    cols = (ctypes.c_int64 * count)(*[s[1] for s in shapes])
    g_ptrs = (ctypes.c_void_p * count)(*[G.data_ptr() for G in Gs])
    o_ptrs = (ctypes.c_void_p * count)(*[o.data_ptr() for o in outs])
    k = None
    if coeffs is not None:
        k = tuple(float(c) for c in coeffs)
        if len(k) != 3:
            raise ValueError("coeffs must be (a, b, c)")
        k = (ctypes.c_float * 3)(*k)
    _check(lib.muon_newton_schulz_f32_batched(g_ptrs, o_ptrs, rows, cols, count, int(steps), k, float(eps),
                                              ws.data_ptr(), ws.numel() * ws.element_size(), stream))
    return outs


def ns5_flops(rows, cols, steps=NS5_STEPS):
    """Nominal NS5 flop count (2 per multiply-add): steps * (4 m^2 n + 2 m^3),
    m = min(rows, cols), n = max(rows, cols)."""
    m, n = min(rows, cols), max(rows, cols)
    return steps * (4 * m * m * n + 2 * m ** 3)
