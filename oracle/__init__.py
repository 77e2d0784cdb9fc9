"""CPU oracle for the 1D deformable convolution forward (double precision).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
path (``deformable_convolution_amd``) never imports it, and this package
imports nothing from the product.

Two independent formulations live here:

* ``forward`` / ``forward_points`` / ``positions`` / ``backward`` -- ctypes
  front end of ``dc1d_oracle.c``: the two-stage definition (sample, then
  contract) in plain C loops over doubles, and its term-by-term derivative.
* ``packed_heads`` / ``packed_forward`` -- the packed layer's offset (and
  mask) generator in the same C file, then ``forward``.
* ``forward2d`` -- 2D modulated deformable convolution (DCNv2 with
  torchvision's offset layout), same C file, same two stages.
* ``constrain_offsets`` and the ``constrained=True`` option of ``forward``,
  ``forward_points`` and ``backward`` -- the constrained mode: each offset
  clamped to its tap's window, then the unconstrained definition (and, for
  the offset gradient, the chain rule through the clamp).
* ``hat.forward`` -- a NumPy brute force that never splits a position into
  integer and fractional parts; it is the pin for the C oracle's
  floor/fraction logic and its zero-fill boundary.

Inputs may be NumPy arrays or CPU torch tensors of any floating dtype; they
are converted exactly to float64 before the call (bf16 and fp32 values are
representable in double).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dc1d_oracle.c")
_LIB = os.path.join(_HERE, "libdc1d_oracle.so")

# gcc flags: no contraction into FMA, no fast-math, so the C arithmetic is
# exactly the double-precision expression as written.
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-std=c11"]


def build(force: bool = False) -> str:
    """Compile ``dc1d_oracle.c`` into ``libdc1d_oracle.so`` next to it."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Lib:
    """ctypes handle on one build of ``dc1d_oracle.c`` (the default build, or a
    test's deliberately altered copy)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_output_length.restype = i64
        lib.oracle_output_length.argtypes = [i64] * 5
        lib.oracle_positions.restype = ctypes.c_int
        lib.oracle_positions.argtypes = [p, i64, i64, i64, i64, i64, i64, i64, p, p, p]
        lib.oracle_forward.restype = ctypes.c_int
        lib.oracle_forward.argtypes = [p] * 5 + [i64] * 10 + [p]
        lib.oracle_forward_points.restype = ctypes.c_int
        lib.oracle_forward_points.argtypes = [p] * 5 + [i64] * 10 + [p, i64, p]
        lib.oracle_backward.restype = ctypes.c_int
        lib.oracle_backward.argtypes = [p] * 5 + [i64] * 10 + [p] * 5
        lib.oracle_packed_heads.restype = ctypes.c_int
        lib.oracle_packed_heads.argtypes = [p] * 7 + [i64] * 7 + [p] * 2
        lib.oracle_forward2d.restype = ctypes.c_int
        lib.oracle_forward2d.argtypes = [p] * 5 + [i64] * 15 + [p]
        self.lib = lib


_default = None


def _load(lib=None):
    """The ctypes library to call: ``lib`` if given, else the default build."""
    global _default
    if lib is not None:
        return lib.lib
    if _default is None:
        _default = _Lib(build())
    return _default.lib


def load_variant(path: str) -> "_Lib":
    """Bind another build of the oracle source (used by the tests that check
    that the pins catch deliberately planted mistakes)."""
    return _Lib(path)


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor: exact widening to double on the CPU
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


_ERR = {1: "bad argument or shape", 2: "non-finite input", 3: "out of memory"}


def output_length(L_in: int, K: int, stride: int = 1, padding: int = 0, dilation: int = 1, lib=None) -> int:
    """conv1d closed form; -1 when out of range or not positive."""
    return int(_load(lib).oracle_output_length(L_in, K, stride, padding, dilation))


def _shapes(x, offsets, weight, groups):
    B, C_in, L_in = x.shape
    C_out, cpg, K = weight.shape
    G = offsets.shape[1]
    if cpg * groups != C_in:
        raise ValueError("weight shape does not match C_in / groups")
    return B, C_in, L_in, C_out, K, G


def constrain_offsets(offsets, dilation):
    """The constrained mode's offsets (dc1d page, section Usage /
    DeformConv1d: by default each tap stays inside its receptive field; the
    rule is not given there).  Reading: the receptive field of output l is
    the undeformed kernel's window [l*s - p, l*s - p + (K-1)*d], so tap k's
    position l*s - p + k*d + o must stay in it, i.e. o is clamped to
    [-k*d, (K-1-k)*d].  offsets [B, G, L_out, K] (float64)."""
    offsets = _f64(offsets)
    K = offsets.shape[-1]
    k = np.arange(K, dtype=np.float64)
    return np.clip(offsets, -k * dilation, (K - 1 - k) * dilation)


def forward(x, offsets, weight, bias=None, mask=None, stride=1, padding=0, dilation=1, groups=1, lib=None,
            constrained=False):
    """Deformable conv1d forward in float64; returns out [B, C_out, L_out].
    constrained=True: the constrained mode (offsets clamped per tap first)."""
    x, offsets, weight, bias, mask = map(_f64, (x, offsets, weight, bias, mask))
    if constrained:
        offsets = constrain_offsets(offsets, dilation)
    B, C_in, L_in, C_out, K, G = _shapes(x, offsets, weight, groups)
    L_out = output_length(L_in, K, stride, padding, dilation, lib)
    if L_out < 1 or offsets.shape != (B, G, L_out, K):
        raise ValueError("offsets must be [B, G, L_out, K] with L_out=%d" % L_out)
    if mask is not None and mask.shape != offsets.shape:
        raise ValueError("mask must have the offsets' shape")
    if bias is not None and bias.shape != (C_out,):
        raise ValueError("bias must be [C_out]")
    out = np.empty((B, C_out, L_out), dtype=np.float64)
    st = _load(lib).oracle_forward(_ptr(x), _ptr(offsets), _ptr(mask), _ptr(weight), _ptr(bias),
                                B, C_in, L_in, C_out, K, stride, padding, dilation, groups, G,
                                _ptr(out))
    if st:
        raise ValueError("oracle_forward: " + _ERR.get(st, str(st)))
    return out


def forward_points(x, offsets, weight, points, bias=None, mask=None, stride=1, padding=0,
                   dilation=1, groups=1, lib=None, constrained=False):
    """Oracle outputs at the given (b, co, l) triples only (array [n, 3])."""
    x, offsets, weight, bias, mask = map(_f64, (x, offsets, weight, bias, mask))
    if constrained:
        offsets = constrain_offsets(offsets, dilation)
    B, C_in, L_in, C_out, K, G = _shapes(x, offsets, weight, groups)
    L_out = output_length(L_in, K, stride, padding, dilation, lib)
    if L_out < 1 or offsets.shape != (B, G, L_out, K):
        raise ValueError("offsets must be [B, G, L_out, K] with L_out=%d" % L_out)
    pts = np.ascontiguousarray(np.asarray(points, dtype=np.int64).reshape(-1, 3))
    out = np.empty(len(pts), dtype=np.float64)
    st = _load(lib).oracle_forward_points(_ptr(x), _ptr(offsets), _ptr(mask), _ptr(weight),
                                       _ptr(bias), B, C_in, L_in, C_out, K, stride, padding,
                                       dilation, groups, G, _ptr(pts), len(pts), _ptr(out))
    if st:
        raise ValueError("oracle_forward_points: " + _ERR.get(st, str(st)))
    return out


def positions(offsets, L_in, K, stride=1, padding=0, dilation=1, lib=None):
    """(i0 int64, frac float64, valid uint8) for offsets [B, G, L_out, K]."""
    offsets = _f64(offsets)
    B, G, L_out, Ko = offsets.shape
    if Ko != K or L_out != output_length(L_in, K, stride, padding, dilation, lib):
        raise ValueError("offsets shape disagrees with L_out")
    i0 = np.empty(offsets.shape, dtype=np.int64)
    fr = np.empty(offsets.shape, dtype=np.float64)
    va = np.empty(offsets.shape, dtype=np.uint8)
    st = _load(lib).oracle_positions(_ptr(offsets), B, G, L_in, K, stride, padding, dilation,
                                  _ptr(i0), _ptr(fr), _ptr(va))
    if st:
        raise ValueError("oracle_positions: " + _ERR.get(st, str(st)))
    return i0, fr, va


def backward(x, offsets, weight, dout, mask=None, stride=1, padding=0, dilation=1, groups=1, lib=None,
             constrained=False):
    """Gradients of sum(dout * forward(...)) in float64, as a dict with keys
    x, offsets, mask (None without a mask), weight, bias.  constrained=True:
    the chain rule through the per-tap clamp -- every gradient taken at the
    clamped offsets, the offset gradient times the clamp's right derivative
    (1 on [-k*d, (K-1-k)*d), else 0)."""
    x, offsets, weight, dout, mask = map(_f64, (x, offsets, weight, dout, mask))
    raw = offsets
    if constrained:
        offsets = constrain_offsets(offsets, dilation)
    B, C_in, L_in, C_out, K, G = _shapes(x, offsets, weight, groups)
    L_out = output_length(L_in, K, stride, padding, dilation, lib)
    if L_out < 1 or offsets.shape != (B, G, L_out, K):
        raise ValueError("offsets must be [B, G, L_out, K] with L_out=%d" % L_out)
    if mask is not None and mask.shape != offsets.shape:
        raise ValueError("mask must have the offsets' shape")
    if dout.shape != (B, C_out, L_out):
        raise ValueError("dout must be [B, C_out, L_out]")
    gx = np.empty_like(x)
    goff = np.empty_like(offsets)
    gmask = np.empty_like(offsets) if mask is not None else None
    gw = np.empty_like(weight)
    gb = np.empty(C_out, dtype=np.float64)
    st = _load(lib).oracle_backward(_ptr(x), _ptr(offsets), _ptr(mask), _ptr(weight), _ptr(dout),
                                 B, C_in, L_in, C_out, K, stride, padding, dilation, groups, G,
                                 _ptr(gx), _ptr(goff), _ptr(gmask), _ptr(gw), _ptr(gb))
    if st:
        raise ValueError("oracle_backward: " + _ERR.get(st, str(st)))
    if constrained:
        k = np.arange(K, dtype=np.float64)
        goff = goff * ((raw >= -k * dilation) & (raw < (K - 1 - k) * dilation))
    return {"x": gx, "offsets": goff, "mask": gmask, "weight": gw, "bias": gb}


def packed_heads(x, trunk_weight, trunk_bias, off_weight, off_bias, mask_weight=None, mask_bias=None,
                 stride=1, padding=0, dilation=1, lib=None):
    """Offsets (and mask) the packed layer's generator computes from x, in
    float64: trunk_weight [C_in, 1, K], off_weight / mask_weight
    [G*K, C_in, 1] (biases [C_in], [G*K], or None).  Returns (offsets, mask)
    with shapes [B, G, L_out, K]; mask is None without mask_weight."""
    x, tw, tb, ow, ob, mw, mb = map(_f64, (x, trunk_weight, trunk_bias, off_weight, off_bias, mask_weight,
                                          mask_bias))
    B, C_in, L_in = x.shape
    if tw.ndim != 3 or tw.shape[:2] != (C_in, 1):
        raise ValueError("trunk_weight must be [C_in, 1, K]")
    K = tw.shape[2]
    if ow.ndim != 3 or ow.shape[1:] != (C_in, 1) or ow.shape[0] % K:
        raise ValueError("off_weight must be [G*K, C_in, 1]")
    G = ow.shape[0] // K
    if mw is not None and mw.shape != ow.shape:
        raise ValueError("mask_weight must have off_weight's shape")
    if tb is not None and tb.shape != (C_in,):
        raise ValueError("trunk_bias must be [C_in]")
    for bb in (ob, mb):
        if bb is not None and bb.shape != (G * K,):
            raise ValueError("head biases must be [G*K]")
    L_out = output_length(L_in, K, stride, padding, dilation, lib)
    if L_out < 1:
        raise ValueError("no output positions")
    off = np.empty((B, G, L_out, K), dtype=np.float64)
    mask = np.empty_like(off) if mw is not None else None
    st = _load(lib).oracle_packed_heads(_ptr(x), _ptr(tw), _ptr(tb), _ptr(ow), _ptr(ob), _ptr(mw),
                                        _ptr(mb if mw is not None else None), B, C_in, L_in, K, stride,
                                        padding, dilation, G, _ptr(off), _ptr(mask))
    if st:
        raise ValueError("oracle_packed_heads: " + _ERR.get(st, str(st)))
    return off, mask


def packed_forward(x, trunk_weight, trunk_bias, off_weight, off_bias, weight, bias=None, mask_weight=None,
                   mask_bias=None, stride=1, padding=0, dilation=1, groups=1, lib=None, constrained=False):
    """The packed layer: its generator's offsets (and mask), then the
    deformable forward (constrained=True: in the constrained mode; the
    returned offsets are the generator's, unclamped).  Returns (out,
    offsets, mask)."""
    off, mask = packed_heads(x, trunk_weight, trunk_bias, off_weight, off_bias, mask_weight, mask_bias,
                             stride, padding, dilation, lib)
    out = forward(x, off, weight, bias, mask, stride, padding, dilation, groups, lib, constrained=constrained)
    return out, off, mask


def output_size2d(H, W, kh, kw, stride=(1, 1), padding=(0, 0), dilation=(1, 1), lib=None):
    """(H_out, W_out): the conv closed form per axis."""
    return (output_length(H, kh, stride[0], padding[0], dilation[0], lib),
            output_length(W, kw, stride[1], padding[1], dilation[1], lib))


def forward2d(x, offsets, weight, bias=None, mask=None, stride=(1, 1), padding=(0, 0), dilation=(1, 1), groups=1,
              lib=None):
    """2D modulated deformable convolution in float64.  x [B, C_in, H, W],
    offsets [B, 2*G*kh*kw, H_out, W_out] ((g, i, j, (row, column)) order),
    mask [B, G*kh*kw, H_out, W_out] or None, weight [C_out, C_in/groups, kh,
    kw]; returns out [B, C_out, H_out, W_out]."""
    x, offsets, weight, bias, mask = map(_f64, (x, offsets, weight, bias, mask))
    B, C_in, H, W = x.shape
    C_out, cpg, kh, kw = weight.shape
    if cpg * groups != C_in:
        raise ValueError("weight shape does not match C_in / groups")
    H_out, W_out = output_size2d(H, W, kh, kw, stride, padding, dilation, lib)
    if H_out < 1 or W_out < 1 or offsets.ndim != 4 or offsets.shape[1] % (2 * kh * kw):
        raise ValueError("bad output size or offsets")
    G = offsets.shape[1] // (2 * kh * kw)
    if offsets.shape != (B, 2 * G * kh * kw, H_out, W_out):
        raise ValueError("offsets must be [B, 2*G*kh*kw, H_out, W_out]")
    if mask is not None and mask.shape != (B, G * kh * kw, H_out, W_out):
        raise ValueError("mask must be [B, G*kh*kw, H_out, W_out]")
    out = np.empty((B, C_out, H_out, W_out), dtype=np.float64)
    st = _load(lib).oracle_forward2d(_ptr(x), _ptr(offsets), _ptr(mask), _ptr(weight), _ptr(bias), B, C_in, H, W,
                                     C_out, kh, kw, stride[0], stride[1], padding[0], padding[1], dilation[0],
                                     dilation[1], groups, G, _ptr(out))
    if st:
        raise ValueError("oracle_forward2d: " + _ERR.get(st, str(st)))
    return out
