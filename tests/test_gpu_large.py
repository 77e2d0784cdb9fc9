"""Tensors past 2^31 elements: the kernels' 64-bit addressing.

Inputs are drawn on the GPU (seeded); the oracle checks sampled outputs,
each on a small sub-problem cut from the full tensors: the input window
every tap of that output can reach (its grid span plus the largest |offset|
and two positions each side, clipped to [0, L_in)), the output's offsets
moved by the window's start (an integer, added in float64, so the split of
every position is unchanged), one output channel, stride 1, no padding.
Positions outside the clipped window are never reached, or lie outside
[0, L_in) in both problems, so the sub-problem's output is the full one's.
Tolerance as in the parity tests: max|err| <= 1e-5 * sqrt(C_in/groups * K).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from deformable_convolution_amd import dc1d

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def reference_at(x, off, w, bias, pts, stride, padding, dilation, groups):
    """Oracle outputs at pts ([n, 3] of (b, co, l)) from device tensors."""
    B, C_in, L_in = x.shape
    C_out, cpg, K = w.shape
    G = off.shape[1]
    cpo, opg = C_in // G, C_out // groups
    wc, bc = w.double().cpu().numpy(), bias.double().cpu().numpy()
    out = []
    for b, co, l in pts:
        grp = co // opg
        c0 = grp * cpg
        g0, g1 = c0 // cpo, (c0 + cpg - 1) // cpo + 1  # the offset groups of the conv group
        o = off[b, g0:g1, l, :].double().cpu().numpy()  # [G', K]
        m = int(math.ceil(float(np.abs(o).max()))) + 2
        base = l * stride - padding
        w0 = max(base - m, 0)
        w1 = min(base + (K - 1) * dilation + m + 1, L_in)
        xs = x[b:b + 1, c0:c0 + cpg, w0:w1].double().cpu().numpy()
        lo_mini = (w1 - w0) - (K - 1) * dilation  # the sub-problem's L_out (stride 1, no padding)
        om = np.zeros((1, g1 - g0, lo_mini, K))
        om[0, :, 0, :] = o + float(base - w0)
        r = oracle.forward_points(xs, om, wc[co:co + 1], np.array([[0, 0, 0]]), bc[co:co + 1], None,
                                  stride=1, padding=0, dilation=dilation, groups=1)
        out.append(r[0])
    return np.array(out)


def points(B, C_out, L_out, n, seed):
    rng = np.random.default_rng(seed)
    pts = np.stack([rng.integers(0, B, n), rng.integers(0, C_out, n), rng.integers(0, L_out, n)], 1)
    ends = np.array([[B - 1, C_out - 1, L_out - 1], [B - 1, C_out - 1, L_out - 2], [B - 1, C_out - 1, L_out - 40],
                     [0, 0, 0], [B - 1, C_out - 1, 0]])
    return np.concatenate([pts, ends])


def run(B, C_in, C_out, L_in, K, stride, padding, dilation, groups, G, kernel_prefix, seed):
    print("large", B, C_in, C_out, L_in, K, stride, padding, dilation, groups, G, flush=True)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    L_out = oracle.output_length(L_in, K, stride, padding, dilation)
    x = torch.randn((B, C_in, L_in), device=DEV, generator=gen)
    off = torch.rand((B, G, L_out, K), device=DEV, generator=gen) * 8.0 - 4.0
    w = torch.randn((C_out, C_in // groups, K), device=DEV, generator=gen) / math.sqrt(C_in // groups * K)
    bias = torch.randn((C_out,), device=DEV, generator=gen) * 0.1
    assert x.numel() > 2 ** 31 or off.numel() > 2 ** 31
    kw = dict(stride=stride, padding=padding, dilation=dilation, groups=groups)
    assert dc1d.plan(x, off, w, bias, None, **kw)["kernel"].startswith(kernel_prefix)
    y = dc1d.forward(x, off, w, bias, None, **kw)
    torch.cuda.synchronize()
    pts = points(B, C_out, L_out, 256, seed)
    got = y[pts[:, 0], pts[:, 1], pts[:, 2]].double().cpu().numpy()
    ref = reference_at(x, off, w, bias, pts, stride, padding, dilation, groups)
    tol = 1e-5 * math.sqrt(C_in // groups * K)
    err = float(np.abs(got - ref).max())
    del x, off, w, bias, y
    torch.cuda.empty_cache()
    assert err <= tol, "max|err| %.3g > %.3g" % (err, tol)


def test_dense_input_past_2_31_elements():
    # x: 512 x 4194312 = 2^31 + 4096 elements; the MFMA kernel's windows
    # reach channel rows beyond 2^31
    run(1, 512, 32, (1 << 22) + 8, 3, 1, 1, 1, 1, 1, "mfma_", seed=21)


def test_depthwise_tensors_past_2_31_elements():
    # x, offsets and out each 8 x (2^28 + 8) = 2^31 + 64 elements
    run(1, 8, 8, (1 << 28) + 8, 1, 1, 0, 1, 8, 8, "depthwise", seed=22)
