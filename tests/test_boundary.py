"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every entry point include/dc1d.h declares,
compute the conv1d output length, and reject every malformed call with the
documented status before touching a device.  Fake non-NULL data pointers
are used: host validation never dereferences them.
"""
import ctypes
import os
import re

import pytest

import oracle
from deformable_convolution_amd import dc1d

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dc1d.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dc1d.library_path()):
        from deformable_convolution_amd.csrc import build
        build.build()
    return dc1d.load_library()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dc1d_\w+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert {"dc1d_forward", "dc1d_output_length", "dc1d_workspace_bytes", "dc1d_debug_positions",
            "dc1d_status_string", "dc1d_plan"} <= set(names)
    for n in names:
        assert hasattr(lib, n), "libdc1d.so does not export %s" % n


def test_output_length_matches_oracle(lib):
    for L_in in range(0, 30):
        for K in range(1, 5):
            for s in range(1, 4):
                for p in range(0, 3):
                    for d in range(1, 3):
                        assert dc1d.output_length(L_in, K, s, p, d) == oracle.output_length(L_in, K, s, p, d)
    assert dc1d.output_length(128, 16, 1, 0, 3) == 83
    assert dc1d.output_length(-1, 3, 1, 0, 1) == -1
    assert dc1d.output_length(10, 0, 1, 0, 1) == -1
    assert dc1d.output_length(10, 3, 0, 0, 1) == -1
    assert dc1d.output_length(10, 3, 1, -1, 1) == -1
    assert dc1d.output_length(10, 3, 1, 0, 0) == -1


def test_status_strings(lib):
    for st in range(9):
        assert dc1d.status_string(st)
    assert dc1d.status_string(0) == "ok"
    assert dc1d.status_string(99) == "unknown status"


def test_resolve_padding():
    assert dc1d.resolve_padding("valid", 16, 1, 3) == 0
    assert dc1d.resolve_padding("same", 3, 1, 4) == 4
    assert dc1d.resolve_padding(2, 3) == 2
    with pytest.raises(ValueError):
        dc1d.resolve_padding("same", 4, 1, 1)  # asymmetric
    with pytest.raises(ValueError):
        dc1d.resolve_padding("same", 3, 2, 1)
    with pytest.raises(ValueError):
        dc1d.resolve_padding("full", 3)


# ---- error codes ------------------------------------------------------------

FAKE = 0x10000000  # a non-NULL address that host validation never dereferences


def T(shape, dtype=0, addr=FAKE):
    d = dc1d._Tensor()
    d.data = addr
    d.dtype = dtype
    d.ndim = len(shape)
    for i, s in enumerate(shape):
        d.shape[i] = s
    return d


def call(lib, x, off, mask, w, bias, out, s=1, p=0, d=1, groups=1, G=None, ws=None, ws_n=0):
    if G is None:
        G = off.shape[1]
    r = lambda t: None if t is None else ctypes.byref(t)
    return lib.dc1d_forward(r(x), r(off), r(mask), r(w), r(bias), r(out), s, p, d, groups, G, ws, ws_n, None)


def good(B=2, C=8, L=20, K=3, G=2, C_out=6, groups=1, addr0=FAKE):
    L_out = L - K + 1
    step = 1 << 24
    x = T([B, C, L], addr=addr0)
    off = T([B, G, L_out, K], addr=addr0 + step)
    mask = T([B, G, L_out, K], addr=addr0 + 2 * step)
    w = T([C_out, C // groups, K], addr=addr0 + 3 * step)
    bias = T([C_out], addr=addr0 + 4 * step)
    out = T([B, C_out, L_out], addr=addr0 + 5 * step)
    return x, off, mask, w, bias, out


def _device_visible():
    # counting devices does not initialise the runtime
    import torch
    return torch.cuda.device_count() > 0


def test_valid_call_reaches_device_check(lib):
    # everything host-checkable is fine, so the only failure left is the
    # missing gfx950 device.  The descriptors hold fake addresses: where a
    # device is visible this call would pass the device check and launch on
    # them, so it is made only on hosts without one.
    if _device_visible():
        pytest.skip("a device is visible: a valid call would launch on the fake addresses")
    st = call(lib, *good())
    assert st == dc1d.ERR_DEVICE


def test_null_pointers(lib):
    x, off, mask, w, bias, out = good()
    assert call(lib, None, off, mask, w, bias, out, G=2) == dc1d.ERR_NULL_PTR
    assert call(lib, x, None, mask, w, bias, out, G=2) == dc1d.ERR_NULL_PTR
    assert call(lib, x, off, mask, None, bias, out) == dc1d.ERR_NULL_PTR
    assert call(lib, x, off, mask, w, bias, None) == dc1d.ERR_NULL_PTR
    x.data = None
    assert call(lib, x, off, mask, w, bias, out) == dc1d.ERR_NULL_PTR


def test_bad_args(lib):
    x, off, mask, w, bias, out = good()
    assert call(lib, x, off, mask, w, bias, out, s=0) == dc1d.ERR_BAD_ARG
    assert call(lib, x, off, mask, w, bias, out, p=-1) == dc1d.ERR_BAD_ARG
    assert call(lib, x, off, mask, w, bias, out, d=0) == dc1d.ERR_BAD_ARG
    assert call(lib, x, off, mask, w, bias, out, groups=0) == dc1d.ERR_BAD_ARG
    assert call(lib, x, off, mask, w, bias, out, G=0) == dc1d.ERR_BAD_ARG
    # offset_groups disagreeing with offsets.shape[1] (the double entry)
    assert call(lib, x, off, mask, w, bias, out, G=4) == dc1d.ERR_BAD_ARG
    # offset groups not dividing C_in
    x3, off3, mask3, w3, b3, out3 = good(G=3)
    assert call(lib, x3, off3, mask3, w3, b3, out3) == dc1d.ERR_BAD_ARG
    # groups not dividing C_in / C_out
    xg, offg, maskg, wg, bg, outg = good(C=8, C_out=6, groups=4)
    assert call(lib, xg, offg, maskg, wg, bg, outg, groups=4) == dc1d.ERR_BAD_ARG


def test_bad_shapes(lib):
    x, off, mask, w, bias, out = good()
    # offsets length disagreeing with the closed form
    off_bad = T([2, 2, 17, 3], addr=off.data)
    assert call(lib, x, off_bad, mask, w, bias, out) == dc1d.ERR_BAD_SHAPE
    assert call(lib, x, off, T([2, 2, 18, 2], addr=mask.data), w, bias, out) == dc1d.ERR_BAD_SHAPE
    assert call(lib, x, off, mask, w, T([5], addr=bias.data), out) == dc1d.ERR_BAD_SHAPE
    assert call(lib, x, off, mask, w, bias, T([2, 6, 17], addr=out.data)) == dc1d.ERR_BAD_SHAPE
    assert call(lib, x, off, mask, T([6, 4, 3], addr=w.data), bias, out) == dc1d.ERR_BAD_SHAPE
    assert call(lib, T([2, 8]), off, mask, w, bias, out) == dc1d.ERR_BAD_SHAPE
    # L_out <= 0: kernel longer than the padded input
    xs = T([2, 8, 2])
    assert call(lib, xs, T([2, 2, 1, 3]), None, w, bias, T([2, 6, 1])) == dc1d.ERR_BAD_SHAPE
    # beyond the position-range limit
    xb = T([1, 8, (1 << 29) + 1])
    Lb = (1 << 29) - 1
    assert call(lib, xb, T([1, 2, Lb, 3]), None, w, None, T([1, 6, Lb])) == dc1d.ERR_BAD_SHAPE


def test_bad_dtypes(lib):
    x, off, mask, w, bias, out = good()
    assert call(lib, T([2, 8, 20], dtype=7), off, mask, w, bias, out) == dc1d.ERR_BAD_DTYPE
    assert call(lib, x, T([2, 2, 18, 3], dtype=1, addr=off.data), mask, w, bias, out) == dc1d.ERR_BAD_DTYPE
    assert call(lib, x, off, mask, w, bias, T([2, 6, 18], dtype=1, addr=out.data)) == dc1d.ERR_BAD_DTYPE


def test_alias(lib):
    x, off, mask, w, bias, out = good()
    out_on_x = T([2, 6, 18], addr=x.data + 64)
    assert call(lib, x, off, mask, w, bias, out_on_x) == dc1d.ERR_ALIAS
    out_on_bias = T([2, 6, 18], addr=bias.data - 8)
    assert call(lib, x, off, mask, w, bias, out_on_bias) == dc1d.ERR_ALIAS


def test_positions_entry_validation(lib):
    off = T([1, 1, 18, 3])
    i0 = ctypes.c_void_p(FAKE)
    assert lib.dc1d_debug_positions(None, 20, 1, 0, 1, i0, i0, i0, None) == dc1d.ERR_NULL_PTR
    assert lib.dc1d_debug_positions(ctypes.byref(off), 20, 0, 0, 1, i0, i0, i0, None) == dc1d.ERR_BAD_ARG
    assert lib.dc1d_debug_positions(ctypes.byref(off), 21, 1, 0, 1, i0, i0, i0, None) == dc1d.ERR_BAD_SHAPE
    assert lib.dc1d_debug_positions(ctypes.byref(off), 20, 1, 0, 1, None, i0, i0, None) == dc1d.ERR_NULL_PTR


# ---- backward entry ------------------------------------------------------------

def bcall(lib, x, off, mask, w, gout, gx=None, goff=None, gmask=None, gw=None, gb=None, G=None, ws=None, ws_n=0):
    if G is None:
        G = off.shape[1]
    r = lambda t: None if t is None else ctypes.byref(t)
    return lib.dc1d_backward(r(x), r(off), r(mask), r(w), r(gout), r(gx), r(goff), r(gmask), r(gw), r(gb),
                             1, 0, 1, 1, G, ws, ws_n, None)


def grads_like(x, off, mask, w, base=FAKE + (8 << 24)):
    step = 1 << 24
    return (T(list(x.shape[:3]), addr=base), T(list(off.shape[:4]), addr=base + step),
            T(list(mask.shape[:4]), addr=base + 2 * step), T(list(w.shape[:3]), addr=base + 3 * step),
            T([w.shape[0]], addr=base + 4 * step))


def test_backward_validation(lib):
    x, off, mask, w, bias, out = good()
    gout = out  # grad_out has the output's shape
    gx, goff, gmask, gw, gb = grads_like(x, off, mask, w)
    # everything host-checkable is fine (made only without a device: with one
    # the call would launch on the fake addresses)
    if not _device_visible():
        assert bcall(lib, x, off, mask, w, gout, gx, goff, gmask, gw, gb) == dc1d.ERR_DEVICE
    assert bcall(lib, x, off, mask, w, None, gx) == dc1d.ERR_NULL_PTR
    # every gradient in the inputs' dtype (bf16 inputs with an fp32 gradient, and the reverse)
    xb = T([2, 8, 20], dtype=1, addr=x.data)
    ob = T([2, 2, 18, 3], dtype=1, addr=off.data)
    wb = T([6, 8, 3], dtype=1, addr=w.data)
    gb16 = T([2, 6, 18], dtype=1, addr=gout.data)
    assert bcall(lib, xb, ob, None, wb, gb16, gx=gx) == dc1d.ERR_BAD_DTYPE
    assert bcall(lib, x, off, mask, w, gout, gx=T([2, 8, 20], dtype=1, addr=gx.data)) == dc1d.ERR_BAD_DTYPE
    # grad_out in the inputs' dtype
    assert bcall(lib, x, off, mask, w, gb16, gx=gx) == dc1d.ERR_BAD_DTYPE
    # a mask gradient needs a mask
    assert bcall(lib, x, off, None, w, gout, gmask=gmask) == dc1d.ERR_BAD_ARG
    # gradient shapes follow their inputs
    assert bcall(lib, x, off, mask, w, gout, gx=T([2, 8, 19], addr=gx.data)) == dc1d.ERR_BAD_SHAPE
    assert bcall(lib, x, off, mask, w, gout, gb=T([5], addr=gb.data)) == dc1d.ERR_BAD_SHAPE
    assert bcall(lib, x, off, mask, w, T([2, 6, 17], addr=gout.data)) == dc1d.ERR_BAD_SHAPE
    # no gradient on an input or on another gradient
    assert bcall(lib, x, off, mask, w, gout, gx=T([2, 8, 20], addr=x.data)) == dc1d.ERR_ALIAS
    assert bcall(lib, x, off, mask, w, gout, gx=gx, gw=T([6, 8, 3], addr=gx.data + 16)) == dc1d.ERR_ALIAS


# ---- empty input sequences -----------------------------------------------------

def test_empty_sequence_rejected(lib):
    # L_in == 0 with enough padding gives L_out >= 1 by the closed form, but
    # there is nothing to sample: rejected before any device work
    L_out = dc1d.output_length(0, 3, 1, 2, 1)
    assert L_out == 2
    w = T([6, 8, 3], addr=FAKE + (3 << 24))
    st = call(lib, T([2, 8, 0], addr=None), T([2, 2, L_out, 3], addr=FAKE + (1 << 24)), None, w, None,
              T([2, 6, L_out], addr=FAKE + (5 << 24)), p=2)
    assert st == dc1d.ERR_BAD_SHAPE
    n = ctypes.c_size_t(0)
    r = ctypes.byref
    assert lib.dc1d_workspace_bytes(r(T([2, 8, 0], addr=None)), r(T([2, 2, L_out, 3])), None, r(w), None,
                                    1, 2, 1, 1, 2, r(n)) == dc1d.ERR_BAD_SHAPE
    # the backward validates the same way
    gout = T([2, 6, L_out], addr=FAKE + (6 << 24))
    assert lib.dc1d_backward(r(T([2, 8, 0], addr=None)), r(T([2, 2, L_out, 3], addr=FAKE + (1 << 24))), None,
                             r(w), r(gout), None, None, None, None, None, 1, 2, 1, 1, 2, None, 0,
                             None) == dc1d.ERR_BAD_SHAPE
    # and the packed layer (its forward's validation)
    tw, ow = T([8, 1, 3], addr=FAKE + (7 << 24)), T([6, 8, 1], addr=FAKE + (8 << 24))
    assert lib.dc1d_packed_workspace_bytes(r(T([2, 8, 0], addr=None)), r(tw), r(ow), None, r(w), 1, 2, 1, 1,
                                           r(n)) == dc1d.ERR_BAD_SHAPE


def test_empty_image_rejected(lib):
    r = ctypes.byref
    w = T([6, 4, 3, 3], addr=FAKE + (3 << 24))
    n = ctypes.c_size_t(0)
    for H, W in ((0, 5), (5, 0), (0, 0)):
        Ho = dc1d.output_length(H, 3, 1, 2, 1)
        Wo = dc1d.output_length(W, 3, 1, 2, 1)
        x = T([1, 4, H, W], addr=None)
        off = T([1, 18, Ho, Wo], addr=FAKE + (1 << 24))
        out = T([1, 6, Ho, Wo], addr=FAKE + (5 << 24))
        assert lib.dc2d_forward(r(x), r(off), None, r(w), None, r(out), 1, 1, 2, 2, 1, 1, 1, 1, None, 0,
                                None) == dc1d.ERR_BAD_SHAPE
        assert lib.dc2d_workspace_bytes(r(x), r(off), None, r(w), None, 1, 1, 2, 2, 1, 1, 1, 1,
                                        r(n)) == dc1d.ERR_BAD_SHAPE


def test_kernel_events_arguments(lib):
    # both events or neither (no device needed: only the per-thread setting)
    assert lib.dc1d_set_kernel_events(None, ctypes.c_void_p(FAKE)) == dc1d.ERR_NULL_PTR
    assert lib.dc1d_set_kernel_events(ctypes.c_void_p(FAKE), None) == dc1d.ERR_NULL_PTR
    assert lib.dc1d_set_kernel_events(None, None) == dc1d.OK
