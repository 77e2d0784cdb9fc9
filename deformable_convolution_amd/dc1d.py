"""ctypes binding over libdc1d (declared in include/dc1d.h).

Argument marshalling only: this module turns torch tensors into
``dc1d_tensor`` descriptors, passes torch's current HIP stream, and maps
status codes to exceptions.  Every step of the computation runs in the
library's HIP kernels; there is no fallback of any kind -- if the library is
missing or the device is not a gfx950, calls raise.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdc1d.so")

DC1D_F32, DC1D_BF16 = 0, 1
_DTYPES = {torch.float32: DC1D_F32, torch.bfloat16: DC1D_BF16}

OK, ERR_NULL_PTR, ERR_BAD_ARG, ERR_BAD_SHAPE, ERR_BAD_DTYPE, ERR_ALIAS, ERR_WORKSPACE, ERR_DEVICE, ERR_LAUNCH = range(9)


class Dc1dError(RuntimeError):
    """A non-OK status from libdc1d."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))


class Dc1dValueError(Dc1dError, ValueError):
    """Argument, shape, dtype, alias or workspace errors."""


class _Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4)]


_lib = None
_lib_lock = threading.Lock()


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libdc1d.so (built in-tree); raise if it is not there."""
    global _lib
    with _lib_lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise ImportError("libdc1d.so is not built (expected at %s); run __graft_entry__.build()"
                                  % _LIB_PATH)
            lib = ctypes.CDLL(_LIB_PATH)
            i64, p, T = ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(_Tensor)
            lib.dc1d_output_length.restype = i64
            lib.dc1d_output_length.argtypes = [i64] * 5
            lib.dc1d_workspace_bytes.restype = ctypes.c_int
            lib.dc1d_workspace_bytes.argtypes = [T] * 5 + [i64] * 5 + [ctypes.POINTER(ctypes.c_size_t)]
            lib.dc1d_forward.restype = ctypes.c_int
            lib.dc1d_forward.argtypes = [T] * 6 + [i64] * 5 + [p, ctypes.c_size_t, p]
            lib.dc1d_debug_positions.restype = ctypes.c_int
            lib.dc1d_debug_positions.argtypes = [T, i64, i64, i64, i64, p, p, p, p]
            lib.dc1d_plan.restype = ctypes.c_int
            lib.dc1d_plan.argtypes = [T] * 5 + [i64] * 5 + [ctypes.POINTER(ctypes.c_char_p),
                                                         ctypes.POINTER(i64),
                                                         ctypes.POINTER(ctypes.c_int32),
                                                         ctypes.POINTER(ctypes.c_int32)]
            lib.dc1d_backward_workspace_bytes.restype = ctypes.c_int
            lib.dc1d_backward_workspace_bytes.argtypes = [T] * 5 + [ctypes.c_int] + [i64] * 5 + [
                ctypes.POINTER(ctypes.c_size_t)]
            lib.dc1d_backward.restype = ctypes.c_int
            lib.dc1d_backward.argtypes = [T] * 10 + [i64] * 5 + [p, ctypes.c_size_t, p]
            lib.dc1d_forward_noalloc.restype = ctypes.c_int
            lib.dc1d_forward_noalloc.argtypes = [T] * 6 + [i64] * 5 + [p]
            lib.dc1d_noalloc_scratch_bytes.restype = ctypes.c_size_t
            lib.dc1d_noalloc_scratch_bytes.argtypes = []
            lib.dc1d_set_kernel_events.restype = ctypes.c_int
            lib.dc1d_set_kernel_events.argtypes = [p, p]
            lib.dc1d_forward_constrained.restype = ctypes.c_int
            lib.dc1d_forward_constrained.argtypes = lib.dc1d_forward.argtypes
            lib.dc1d_backward_constrained.restype = ctypes.c_int
            lib.dc1d_backward_constrained.argtypes = lib.dc1d_backward.argtypes
            lib.dc1d_packed_workspace_bytes.restype = ctypes.c_int
            lib.dc1d_packed_workspace_bytes.argtypes = [T] * 5 + [i64] * 4 + [ctypes.POINTER(ctypes.c_size_t)]
            lib.dc1d_packed_forward.restype = ctypes.c_int
            lib.dc1d_packed_forward.argtypes = [T] * 12 + [i64] * 4 + [p, ctypes.c_size_t, p]
            lib.dc1d_packed_forward_constrained.restype = ctypes.c_int
            lib.dc1d_packed_forward_constrained.argtypes = lib.dc1d_packed_forward.argtypes
            lib.dc2d_workspace_bytes.restype = ctypes.c_int
            lib.dc2d_workspace_bytes.argtypes = [T] * 5 + [i64] * 8 + [ctypes.POINTER(ctypes.c_size_t)]
            lib.dc2d_forward.restype = ctypes.c_int
            lib.dc2d_forward.argtypes = [T] * 6 + [i64] * 8 + [p, ctypes.c_size_t, p]
            lib.dc2d_plan.restype = ctypes.c_int
            lib.dc2d_plan.argtypes = [T] * 5 + [i64] * 8 + [ctypes.POINTER(ctypes.c_char_p)]
            lib.dc1d_status_string.restype = ctypes.c_char_p
            lib.dc1d_status_string.argtypes = [ctypes.c_int]
            _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load_library().dc1d_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != OK:
        if status in (ERR_NULL_PTR, ERR_BAD_ARG, ERR_BAD_SHAPE, ERR_BAD_DTYPE, ERR_ALIAS, ERR_WORKSPACE):
            raise Dc1dValueError(status, where)
        raise Dc1dError(status, where)


def _desc(t):
    if t is None:
        return None
    d = _Tensor()
    d.data = t.data_ptr() if t.numel() > 0 else None
    d.dtype = _DTYPES.get(t.dtype, -1)
    d.ndim = t.dim()
    for i, s in enumerate(t.shape[:4]):
        d.shape[i] = s
    return d


def _ref(d):
    return None if d is None else ctypes.byref(d)


def output_length(L_in: int, K: int, stride: int = 1, padding: int = 0, dilation: int = 1) -> int:
    return int(load_library().dc1d_output_length(L_in, K, stride, padding, dilation))


def resolve_padding(padding, K: int, stride: int = 1, dilation: int = 1) -> int:
    """"valid" -> 0; "same" -> dilation*(K-1)/2 when that keeps the length
    with stride 1 and is symmetric; an int passes through (dc1d page, Usage:
    padding may be an int, "valid" or "same")."""
    if isinstance(padding, str):
        if padding == "valid":
            return 0
        if padding == "same":
            span = dilation * (K - 1)
            if stride != 1 or span % 2:
                raise ValueError('padding="same" needs stride 1 and an even dilation*(K-1)')
            return span // 2
        raise ValueError("padding must be an int, 'valid' or 'same'")
    return int(padding)


def _contig(t, name):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _args(x, offsets, weight, bias, mask, stride, padding, dilation, groups):
    K = weight.shape[-1] if weight.dim() == 3 else 0
    padding = resolve_padding(padding, K, stride, dilation)
    G = offsets.shape[1] if offsets.dim() == 4 else 0
    return padding, G


_ws_cache = {}
_ws_size_cache = {}


class _nullctx:
    def __enter__(self):
        return None

    def __exit__(self, *a):
        return False


def _device_ctx(device):
    """torch.cuda.device(device), or nothing when it is already current (the
    common case; entering the context costs more than the launch)."""
    if device.index is None or device.index == torch.cuda.current_device():
        return _nullctx()
    return torch.cuda.device(device)


def _workspace(nbytes: int, device):
    """A cached workspace per (device, stream), grown as needed (the library
    needs no initialisation of it; calls on one stream are ordered, so they
    can share it)."""
    if nbytes == 0:
        return None
    stream = torch.cuda.current_stream(device)
    key = (device.index, stream.cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def workspace_bytes(x, offsets, weight, bias=None, mask=None, stride=1, padding=0, dilation=1, groups=1) -> int:
    padding, G = _args(x, offsets, weight, bias, mask, stride, padding, dilation, groups)
    n = ctypes.c_size_t(0)
    dx, do, dm, dw, db = map(_desc, (x, offsets, mask, weight, bias))
    _check(load_library().dc1d_workspace_bytes(_ref(dx), _ref(do), _ref(dm), _ref(dw), _ref(db),
                                               stride, padding, dilation, groups, G, ctypes.byref(n)),
           "dc1d_workspace_bytes")
    return int(n.value)


def plan(x, offsets, weight, bias=None, mask=None, stride=1, padding=0, dilation=1, groups=1) -> dict:
    padding, G = _args(x, offsets, weight, bias, mask, stride, padding, dilation, groups)
    name = ctypes.c_char_p()
    grid = ctypes.c_int64()
    block = ctypes.c_int32()
    splits = ctypes.c_int32()
    dx, do, dm, dw, db = map(_desc, (x, offsets, mask, weight, bias))
    _check(load_library().dc1d_plan(_ref(dx), _ref(do), _ref(dm), _ref(dw), _ref(db), stride, padding,
                                    dilation, groups, G, ctypes.byref(name), ctypes.byref(grid),
                                    ctypes.byref(block), ctypes.byref(splits)), "dc1d_plan")
    return {"kernel": name.value.decode(), "grid": grid.value, "block": block.value, "splits": splits.value}


def forward_noalloc(x, offsets, weight, bias=None, mask=None, stride=1, padding=0, dilation=1, groups=1,
                    *, out):
    """dc1d_forward_noalloc: the forward with its workspace in the library's
    per-device scratch array (no device allocation in the call, none here
    either: ``out`` must be given).  Calls that may overlap on one device
    race on the scratch.  Enqueued on torch's current stream."""
    lib = load_library()
    x, offsets, weight, bias, mask, out = (_contig(t, n) for t, n in ((x, "x"), (offsets, "offsets"),
                                                                        (weight, "weight"), (bias, "bias"),
                                                                        (mask, "mask"), (out, "out")))
    padding, G = _args(x, offsets, weight, bias, mask, stride, padding, dilation, groups)
    dx, do, dm, dw, db, dout = map(_desc, (x, offsets, mask, weight, bias, out))
    with _device_ctx(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        _check(lib.dc1d_forward_noalloc(_ref(dx), _ref(do), _ref(dm), _ref(dw), _ref(db), _ref(dout), stride,
                                        padding, dilation, groups, G, stream), "dc1d_forward_noalloc")
    return out


def set_kernel_events(start=None, stop=None):
    """dc1d_set_kernel_events for this thread: torch.cuda.Event objects (already
    recorded once, so that their HIP events exist), or None, None."""
    h = (lambda e: None if e is None else ctypes.c_void_p(e.cuda_event))
    _check(load_library().dc1d_set_kernel_events(h(start), h(stop)), "dc1d_set_kernel_events")


def noalloc_scratch_bytes() -> int:
    return int(load_library().dc1d_noalloc_scratch_bytes())


def forward(x, offsets, weight, bias=None, mask=None, stride=1, padding=0, dilation=1, groups=1,
            out=None, workspace=None, constrained=False):
    """DeformConv1d forward on the GPU.  Tensors must be contiguous device
    tensors of one dtype (float32 or bfloat16); returns out [B, C_out, L_out]
    (allocated unless given).  constrained=True keeps every tap inside the
    undeformed kernel window of its output (dc1d_forward_constrained).
    Enqueued on torch's current stream."""
    lib = load_library()
    x, offsets, weight, bias, mask = (_contig(t, n) for t, n in ((x, "x"), (offsets, "offsets"),
                                                                   (weight, "weight"), (bias, "bias"),
                                                                   (mask, "mask")))
    padding, G = _args(x, offsets, weight, bias, mask, stride, padding, dilation, groups)
    if out is None:
        L_out = output_length(x.shape[-1], weight.shape[-1], stride, padding, dilation)
        if L_out < 1 or x.dim() != 3 or weight.dim() != 3:
            raise Dc1dValueError(ERR_BAD_SHAPE, "dc1d_forward")
        out = torch.empty((x.shape[0], weight.shape[0], L_out), dtype=x.dtype, device=x.device)
    dx, do, dm, dw, db, dout = map(_desc, (x, offsets, mask, weight, bias, out))
    if workspace is None:
        # the size depends on shapes and arguments only (cached per call signature)
        key = (x.device.index, x.dtype, tuple(x.shape), tuple(offsets.shape), mask is None, tuple(weight.shape),
               bias is None, stride, padding, dilation, groups)
        nbytes = _ws_size_cache.get(key)
        with _device_ctx(x.device):
            if nbytes is None:
                n = ctypes.c_size_t(0)
                _check(lib.dc1d_workspace_bytes(_ref(dx), _ref(do), _ref(dm), _ref(dw), _ref(db), stride, padding,
                                                dilation, groups, G, ctypes.byref(n)), "dc1d_workspace_bytes")
                nbytes = _ws_size_cache[key] = int(n.value)
            workspace = _workspace(nbytes, x.device)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with _device_ctx(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        fn = lib.dc1d_forward_constrained if constrained else lib.dc1d_forward
        _check(fn(_ref(dx), _ref(do), _ref(dm), _ref(dw), _ref(db), _ref(dout), stride, padding, dilation, groups,
                  G, ws_ptr, ws_len, stream), "dc1d_forward")
    return out


def backward(x, offsets, weight, grad_out, mask=None, stride=1, padding=0, dilation=1, groups=1,
             need=("x", "offsets", "mask", "weight", "bias"), workspace=None, constrained=False):
    """Gradients of sum(grad_out * forward(...)) on the GPU (float32 or
    bfloat16 tensors, all of one dtype; the gradients have it too, bf16 ones
    computed in fp32 and rounded once).  Returns a dict with the requested
    keys among x, offsets, mask (only with a mask), weight, bias; tensors are
    allocated here, the arithmetic runs in the library's kernels on torch's
    current stream.  constrained=True: the backward of the constrained
    forward."""
    lib = load_library()
    x, offsets, weight, grad_out, mask = (_contig(t, n) for t, n in ((x, "x"), (offsets, "offsets"),
                                                                      (weight, "weight"),
                                                                      (grad_out, "grad_out"),
                                                                      (mask, "mask")))
    padding, G = _args(x, offsets, weight, None, mask, stride, padding, dilation, groups)
    like = {"x": x, "offsets": offsets, "mask": mask, "weight": weight}
    grads = {}
    for k in need:
        if k == "mask" and mask is None:
            continue
        if k == "bias":
            grads[k] = torch.empty(weight.shape[0], dtype=weight.dtype, device=weight.device)
        else:
            grads[k] = torch.empty_like(like[k])
    dx, do, dm, dw, dg = map(_desc, (x, offsets, mask, weight, grad_out))
    gd = {k: _desc(v) for k, v in grads.items()}
    if workspace is None:
        n = ctypes.c_size_t(0)
        with torch.cuda.device(x.device):
            _check(lib.dc1d_backward_workspace_bytes(_ref(dx), _ref(do), _ref(dm), _ref(dw), _ref(dg),
                                                     int("weight" in grads), stride, padding, dilation,
                                                     groups, G, ctypes.byref(n)),
                   "dc1d_backward_workspace_bytes")
            workspace = _workspace(int(n.value), x.device)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        fn = lib.dc1d_backward_constrained if constrained else lib.dc1d_backward
        _check(fn(_ref(dx), _ref(do), _ref(dm), _ref(dw), _ref(dg), _ref(gd.get("x")), _ref(gd.get("offsets")),
                  _ref(gd.get("mask")), _ref(gd.get("weight")), _ref(gd.get("bias")), stride, padding, dilation,
                  groups, G, ws_ptr, ws_len, stream), "dc1d_backward")
    return grads


def packed_forward(x, trunk_weight, trunk_bias, off_weight, off_bias, weight, bias=None, mask_weight=None,
                   mask_bias=None, stride=1, padding=0, dilation=1, groups=1, with_offsets=False, out=None,
                   workspace=None, constrained=False):
    """The packed layer on the GPU (fp32): offsets (and, with mask_weight, the
    mask) generated from x by the depthwise trunk and pointwise heads, then
    the deformable forward (constrained=True: in the constrained mode, the
    generated offsets returned as generated).  trunk_weight [C_in, 1, K],
    off_weight and mask_weight [G*K, C_in, 1].  Returns out (allocated unless
    given), or with with_offsets (out, offsets) / (out, (offsets, mask)).
    Enqueued on torch's current stream."""
    lib = load_library()
    names = ("x", "trunk_weight", "trunk_bias", "off_weight", "off_bias", "weight", "bias", "mask_weight",
             "mask_bias")
    x, tw, tb, ow, ob, w, b, mw, mb = (_contig(t, n) for t, n in zip(
        (x, trunk_weight, trunk_bias, off_weight, off_bias, weight, bias, mask_weight, mask_bias), names))
    if x.dim() != 3 or w.dim() != 3 or ow.dim() != 3 or tw.dim() != 3 or tw.shape[2] < 1:
        raise Dc1dValueError(ERR_BAD_SHAPE, "dc1d_packed_forward")
    K = tw.shape[2]
    padding = resolve_padding(padding, K, stride, dilation)
    L_out = output_length(x.shape[-1], K, stride, padding, dilation)
    if L_out < 1 or ow.shape[0] % K:
        raise Dc1dValueError(ERR_BAD_SHAPE, "dc1d_packed_forward")
    G = ow.shape[0] // K
    if out is None:
        out = torch.empty((x.shape[0], w.shape[0], L_out), dtype=x.dtype, device=x.device)
    offs = msk = None
    if with_offsets:
        offs = torch.empty((x.shape[0], G, L_out, K), dtype=x.dtype, device=x.device)
        if mw is not None:
            msk = torch.empty_like(offs)
    d = [_desc(t) for t in (x, tw, tb, ow, ob, mw, mb, w, b, out, offs, msk)]
    if workspace is None:
        n = ctypes.c_size_t(0)
        with torch.cuda.device(x.device):
            _check(lib.dc1d_packed_workspace_bytes(_ref(d[0]), _ref(d[1]), _ref(d[3]), _ref(d[5]), _ref(d[7]),
                                                   stride, padding, dilation, groups, ctypes.byref(n)),
                   "dc1d_packed_workspace_bytes")
            workspace = _workspace(int(n.value), x.device)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        fn = lib.dc1d_packed_forward_constrained if constrained else lib.dc1d_packed_forward
        _check(fn(*[_ref(t) for t in d], stride, padding, dilation, groups, ws_ptr, ws_len, stream),
               "dc1d_packed_forward")
    if not with_offsets:
        return out
    return (out, (offs, msk)) if mw is not None else (out, offs)


def backward_workspace_bytes(x, offsets, weight, grad_out, mask=None, stride=1, padding=0, dilation=1, groups=1,
                             want_weight=True) -> int:
    """Device workspace (bytes) a backward call with these arguments needs."""
    padding, G = _args(x, offsets, weight, None, mask, stride, padding, dilation, groups)
    n = ctypes.c_size_t(0)
    dx, do, dm, dw, dg = map(_desc, (x, offsets, mask, weight, grad_out))
    with _device_ctx(x.device):
        _check(load_library().dc1d_backward_workspace_bytes(_ref(dx), _ref(do), _ref(dm), _ref(dw), _ref(dg),
                                                            int(want_weight), stride, padding, dilation, groups, G,
                                                            ctypes.byref(n)), "dc1d_backward_workspace_bytes")
    return int(n.value)


def packed_workspace_bytes(x, trunk_weight, off_weight, weight, mask_weight=None, stride=1, padding=0, dilation=1,
                           groups=1) -> int:
    """Device workspace (bytes) a packed-layer call with these arguments needs."""
    K = trunk_weight.shape[-1]
    padding = resolve_padding(padding, K, stride, dilation)
    n = ctypes.c_size_t(0)
    d = [_desc(t) for t in (x, trunk_weight, off_weight, mask_weight, weight)]
    with _device_ctx(x.device):
        _check(load_library().dc1d_packed_workspace_bytes(*[_ref(t) for t in d], stride, padding, dilation, groups,
                                                          ctypes.byref(n)), "dc1d_packed_workspace_bytes")
    return int(n.value)


def _pair(v):
    return (int(v[0]), int(v[1])) if isinstance(v, (tuple, list)) else (int(v), int(v))


def _args2d(x, offsets, weight, stride, padding, dilation):
    kh, kw = (weight.shape[2], weight.shape[3]) if weight.dim() == 4 else (1, 1)
    G = offsets.shape[1] // (2 * kh * kw) if offsets.dim() == 4 else 0
    return _pair(stride), _pair(padding), _pair(dilation), G


def workspace_bytes2d(x, offsets, weight, bias=None, mask=None, stride=1, padding=0, dilation=1, groups=1) -> int:
    """Device workspace (bytes) a 2D forward call with these arguments needs."""
    s, p, d, G = _args2d(x, offsets, weight, stride, padding, dilation)
    n = ctypes.c_size_t(0)
    dx, do, dm, dw, db = map(_desc, (x, offsets, mask, weight, bias))
    with _device_ctx(x.device):
        _check(load_library().dc2d_workspace_bytes(_ref(dx), _ref(do), _ref(dm), _ref(dw), _ref(db), s[0], s[1], p[0],
                                                   p[1], d[0], d[1], groups, G, ctypes.byref(n)),
               "dc2d_workspace_bytes")
    return int(n.value)


def plan2d(x, offsets, weight, bias=None, mask=None, stride=1, padding=0, dilation=1, groups=1) -> str:
    s, p, d, G = _args2d(x, offsets, weight, stride, padding, dilation)
    name = ctypes.c_char_p()
    dx, do, dm, dw, db = map(_desc, (x, offsets, mask, weight, bias))
    _check(load_library().dc2d_plan(_ref(dx), _ref(do), _ref(dm), _ref(dw), _ref(db), s[0], s[1], p[0], p[1], d[0],
                                    d[1], groups, G, ctypes.byref(name)), "dc2d_plan")
    return name.value.decode()


def forward2d(x, offsets, weight, bias=None, mask=None, stride=1, padding=0, dilation=1, groups=1, out=None,
              workspace=None):
    """2D modulated deformable convolution on the GPU (torchvision's offset
    layout: [B, 2*G*kh*kw, H_out, W_out], (row, column) per tap).  stride,
    padding, dilation: an int or a (row, column) pair.  Returns out
    [B, C_out, H_out, W_out] (allocated unless given), enqueued on torch's
    current stream."""
    lib = load_library()
    x, offsets, weight, bias, mask = (_contig(t, n) for t, n in ((x, "x"), (offsets, "offsets"), (weight, "weight"),
                                                                   (bias, "bias"), (mask, "mask")))
    s, p, d, G = _args2d(x, offsets, weight, stride, padding, dilation)
    if out is None:
        if x.dim() != 4 or weight.dim() != 4:
            raise Dc1dValueError(ERR_BAD_SHAPE, "dc2d_forward")
        Ho = output_length(x.shape[2], weight.shape[2], s[0], p[0], d[0])
        Wo = output_length(x.shape[3], weight.shape[3], s[1], p[1], d[1])
        if Ho < 1 or Wo < 1:
            raise Dc1dValueError(ERR_BAD_SHAPE, "dc2d_forward")
        out = torch.empty((x.shape[0], weight.shape[0], Ho, Wo), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace = _workspace(workspace_bytes2d(x, offsets, weight, bias, mask, s, p, d, groups), x.device)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    dx, do, dm, dw, db, dout = map(_desc, (x, offsets, mask, weight, bias, out))
    with _device_ctx(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        _check(lib.dc2d_forward(_ref(dx), _ref(do), _ref(dm), _ref(dw), _ref(db), _ref(dout), s[0], s[1], p[0], p[1],
                                d[0], d[1], groups, G, ws_ptr, ws_len, stream), "dc2d_forward")
    return out


def debug_positions(offsets, L_in, stride=1, padding=0, dilation=1):
    """(i0 int32, frac float32, valid uint8) device tensors shaped like offsets."""
    lib = load_library()
    _contig(offsets, "offsets")
    i0 = torch.empty(offsets.shape, dtype=torch.int32, device=offsets.device)
    fr = torch.empty(offsets.shape, dtype=torch.float32, device=offsets.device)
    va = torch.empty(offsets.shape, dtype=torch.uint8, device=offsets.device)
    d = _desc(offsets)
    with torch.cuda.device(offsets.device):
        stream = torch.cuda.current_stream(offsets.device).cuda_stream
        _check(lib.dc1d_debug_positions(ctypes.byref(d), L_in, stride, padding, dilation, i0.data_ptr(),
                                        fr.data_ptr(), va.data_ptr(), stream), "dc1d_debug_positions")
    return i0, fr, va
