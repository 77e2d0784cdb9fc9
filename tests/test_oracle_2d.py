"""Pins for the oracle's 2D modulated deformable convolution (CPU only).

``oracle.forward2d`` (the two stages of the deformable convolution article,
section Deformable Convolution, in 2D with bilinear sampling; offsets in the
torchvision issue's layout) is pinned against things other than itself:

* the torchvision issue's printed demo, value for value
  (``tests/golden/torchvision_issue_demo.json``);
* zero offsets: CPU float64 ``torch.nn.functional.conv2d`` (strides,
  padding, dilation, groups, several offset groups);
* a constant integer offset per group: ``conv2d`` of the shifted,
  zero-filled input;
* one-row (one-column) images with a one-row (one-column) kernel and no
  offset across that axis: the 1D oracle (pinned on its own) along the other
  axis, which fixes which offset channel is the row and which the column;
* a bilinear field a + b*r + c*s + e*r*s is reproduced exactly at interior
  fractional positions (bilinear interpolation is exact on it);
* the product-of-hats brute force on tiny random inputs, edges included;
* masks: all ones equal none bit for bit, zero gives the bias.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "torchvision_issue_demo.json")


def close(a, b, rel=1e-12):
    scale = max(1.0, float(np.abs(b).max()))
    assert a.shape == b.shape, (a.shape, b.shape)
    assert np.abs(a - b).max() <= rel * scale, (np.abs(a - b).max(), scale)


def test_torchvision_issue_demo_2d():
    g = json.load(open(GOLDEN))
    x = np.arange(27.0).reshape(1, 3, 3, 3)
    pairs = np.array([[0, -1], [0, 1], [-1, 0]], dtype=np.float64)  # (row, column) per offset group
    off = np.broadcast_to(pairs.reshape(1, 6, 1, 1), (1, 6, 3, 3)).copy()
    w = np.array([[1, 0, 0], [0, 1, 0], [1, 1, 0], [0, 0, 1], [0, 1, 0]], dtype=np.float64).reshape(5, 3, 1, 1)
    got = oracle.forward2d(x, off, w)
    assert np.array_equal(got[0], np.array(g["printed_output"], dtype=np.float64))


# (B, C_in, C_out, H, W, kh, kw, stride, padding, dilation, groups, G)
SHAPES = [
    (1, 2, 3, 7, 6, 3, 3, (1, 1), (1, 1), (1, 1), 1, 1),
    (2, 4, 6, 9, 8, 3, 2, (2, 1), (1, 0), (1, 2), 2, 2),
    (1, 6, 3, 8, 9, 2, 3, (1, 2), (0, 2), (2, 1), 3, 3),
    (2, 3, 3, 6, 7, 1, 3, (1, 1), (0, 1), (1, 1), 3, 1),
]


def make(shape, seed, off=None, mask=False):
    B, C_in, C_out, H, W, kh, kw, s, p, d, groups, G = shape
    r = np.random.default_rng(seed)
    Ho, Wo = oracle.output_size2d(H, W, kh, kw, s, p, d)
    c = {"x": r.standard_normal((B, C_in, H, W)),
         "weight": r.standard_normal((C_out, C_in // groups, kh, kw)),
         "bias": r.standard_normal(C_out),
         "kw": dict(stride=s, padding=p, dilation=d, groups=groups), "G": G, "Ho": Ho, "Wo": Wo}
    n_off = (B, 2 * G * kh * kw, Ho, Wo)
    c["offsets"] = r.uniform(-2.5, 2.5, n_off) if off is None else off(r, n_off)
    c["mask"] = r.uniform(0.2, 1.4, (B, G * kh * kw, Ho, Wo)) if mask else None
    return c


def run(c, **over):
    a = dict(c, **over)
    return oracle.forward2d(a["x"], a["offsets"], a["weight"], a["bias"], a["mask"], **a["kw"])


def conv2d(x, w, b, kw):
    return F.conv2d(torch.tensor(x), torch.tensor(w), None if b is None else torch.tensor(b), **kw).numpy()


@pytest.mark.parametrize("shape", SHAPES)
def test_zero_offsets_equal_conv2d(shape):
    c = make(shape, 41, off=lambda r, n: np.zeros(n))
    close(run(c), conv2d(c["x"], c["weight"], c["bias"], c["kw"]))


@pytest.mark.parametrize("shape", SHAPES[:3])
def test_integer_group_shift_is_shifted_conv2d(shape):
    B, C_in, C_out, H, W, kh, kw, s, p, d, groups, G = shape
    r = np.random.default_rng(42)
    shifts = r.integers(-2, 3, (G, 2))

    def off(rr, n):
        o = np.zeros(n)
        for g in range(G):
            for t in range(kh * kw):
                o[:, 2 * (g * kh * kw + t)] = shifts[g, 0]
                o[:, 2 * (g * kh * kw + t) + 1] = shifts[g, 1]
        return o

    c = make(shape, 43, off=off)
    # the zero-extended input seen from the shifted grid: sample (a, b) of a
    # tap of channel ci reads x~(a + dy, b + dx); pad x by m zeros and crop it
    # so that conv2d without padding reads exactly those values
    m = max(p) + 3
    xe = np.pad(c["x"], ((0, 0), (0, 0), (m, 2 * m), (m, 2 * m)))
    xs = np.zeros((B, C_in, H + m + p[0], W + m + p[1]))
    cpo = C_in // G
    for ci in range(C_in):
        dy, dx = shifts[ci // cpo]
        r0, c0 = m - p[0] + dy, m - p[1] + dx
        xs[:, ci] = xe[:, ci, r0:r0 + xs.shape[2], c0:c0 + xs.shape[3]]
    kw = dict(c["kw"], padding=0)
    ref = conv2d(xs, c["weight"], c["bias"], kw)[:, :, :c["Ho"], :c["Wo"]]
    close(run(c), ref)


@pytest.mark.parametrize("axis", ["row", "column"])
def test_one_line_reduces_to_the_1d_oracle(axis):
    r = np.random.default_rng(44)
    B, C_in, C_out, L, K, s, p, d, G = 2, 4, 5, 13, 3, 2, 2, 2, 2
    x1 = r.standard_normal((B, C_in, L))
    w1 = r.standard_normal((C_out, C_in, K))
    L_out = oracle.output_length(L, K, s, p, d)
    o1 = r.uniform(-3, 3, (B, G, L_out, K))
    ref = oracle.forward(x1, o1, w1, None, None, s, p, d)
    z = np.zeros((B, G, L_out, K))
    if axis == "column":  # a one-row image, kernel 1 x K, offsets only along the columns
        x2, w2 = x1[:, :, None, :], w1[:, :, None, :]
        pair = np.stack([z, o1], axis=-1)                                  # [B, G, L_out, K, (row, col)]
        off = pair.transpose(0, 1, 3, 4, 2).reshape(B, 2 * G * K, 1, L_out)
        got = oracle.forward2d(x2, off, w2, stride=(1, s), padding=(0, p), dilation=(1, d))[:, :, 0, :]
    else:  # a one-column image, kernel K x 1, offsets only along the rows
        x2, w2 = x1[:, :, :, None], w1[:, :, :, None]
        pair = np.stack([o1, z], axis=-1)
        off = pair.transpose(0, 1, 3, 4, 2).reshape(B, 2 * G * K, L_out, 1)
        got = oracle.forward2d(x2, off, w2, stride=(s, 1), padding=(p, 0), dilation=(d, 1))[:, :, :, 0]
    close(got, ref)


def test_bilinear_field_is_reproduced():
    B, C, H, W, kh, kw = 1, 2, 9, 10, 3, 3
    a, b, c_, e = 0.3, -0.7, 1.1, 0.25
    rr, ss = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    x = np.broadcast_to(a + b * rr + c_ * ss + e * rr * ss, (B, C, H, W)).copy()
    r = np.random.default_rng(45)
    w = r.standard_normal((3, C, kh, kw))
    Ho, Wo = oracle.output_size2d(H, W, kh, kw, (1, 1), (0, 0), (1, 1))
    off = r.uniform(-0.45, 0.45, (B, 2 * kh * kw, Ho, Wo))
    for i, j in itertools.product(range(kh), range(kw)):  # keep every position inside the image
        by = np.arange(Ho)[:, None] + i + np.zeros((1, Wo))
        bx = np.arange(Wo)[None, :] + j + np.zeros((Ho, 1))
        off[0, 2 * (i * kw + j)] = np.clip(off[0, 2 * (i * kw + j)], -by, H - 1 - by)
        off[0, 2 * (i * kw + j) + 1] = np.clip(off[0, 2 * (i * kw + j) + 1], -bx, W - 1 - bx)
    got = oracle.forward2d(x, off, w)
    ref = np.zeros_like(got)
    for co, i, j in itertools.product(range(3), range(kh), range(kw)):
        py = np.arange(Ho)[:, None] + i + off[0, 2 * (i * kw + j)]
        px = np.arange(Wo)[None, :] + j + off[0, 2 * (i * kw + j) + 1]
        ref[0, co] += w[co].sum(axis=0)[i, j] * (a + b * py + c_ * px + e * py * px)
    close(got, ref, 1e-11)


def hat2d(x, off, w, bias, mask, s, p, d, groups):
    B, C_in, H, W = x.shape
    C_out, cpg, kh, kw = w.shape
    Ho, Wo = off.shape[2], off.shape[3]
    G = off.shape[1] // (2 * kh * kw)
    cpo, opg = C_in // G, C_out // groups
    rows, cols = np.arange(H)[:, None], np.arange(W)[None, :]
    out = np.zeros((B, C_out, Ho, Wo))
    for bb, co, oh, ow in itertools.product(range(B), range(C_out), range(Ho), range(Wo)):
        acc = bias[co]
        for cl in range(cpg):
            ci = (co // opg) * cpg + cl
            g = ci // cpo
            for i, j in itertools.product(range(kh), range(kw)):
                t = (g * kh + i) * kw + j
                py = oh * s[0] - p[0] + i * d[0] + off[bb, 2 * t, oh, ow]
                px = ow * s[1] - p[1] + j * d[1] + off[bb, 2 * t + 1, oh, ow]
                hat = np.maximum(0, 1 - np.abs(py - rows)) * np.maximum(0, 1 - np.abs(px - cols))
                v = float((hat * x[bb, ci]).sum())
                if mask is not None:
                    v *= mask[bb, t, oh, ow]
                acc += w[co, cl, i, j] * v
        out[bb, co, oh, ow] = acc
    return out


@pytest.mark.parametrize("shape", SHAPES)
def test_equals_product_of_hats_brute_force(shape):
    c = make(shape, 46, mask=True)
    kw = c["kw"]
    close(run(c), hat2d(c["x"], c["offsets"], c["weight"], c["bias"], c["mask"], kw["stride"], kw["padding"],
                        kw["dilation"], kw["groups"]))


def test_mask_invariants():
    c = make(SHAPES[1], 47, mask=True)
    ones = run(c, mask=np.ones_like(c["mask"]))
    assert np.array_equal(ones, run(c, mask=None))
    zero = run(c, mask=np.zeros_like(c["mask"]))
    close(zero, np.broadcast_to(c["bias"][None, :, None, None], zero.shape))
