"""Brute-force 1D deformable convolution through the "hat" kernel.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Linear interpolation of a zero-extended sequence at a real position ``pos``
equals a sum over every integer index weighted by a triangle ("hat") of
half-width one centred on ``pos``:

    v(pos) = sum_i x[i] * max(0, 1 - |pos - i|),   i = 0 .. L_in - 1.

Only the two integer neighbours of ``pos`` get a non-zero weight, and they
get exactly 1 - f and f, so this is the interpolation that the dc1d page
describes ("a fractional offset interpolates linearly", section Demo
notebook) with zeros outside the sequence (the torchvision issue page's
printed demo).  It never floors a position, so it checks the C oracle's
integer/fraction split and its edge handling independently.  Cost is
O(B * C_in * L_out * K * L_in): tiny inputs only.

The position itself, ``l*stride - padding + k*dilation + offset``, is the
conv1d grid position of the conv1d operator page (section Description)
moved by the offset, as in the deformable formula of the dilated /
deformable convolution article (section Deformable Convolution).
"""
from __future__ import annotations

import numpy as np


def _np(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def output_length(L_in, K, stride, padding, dilation):
    """Count the windows l >= 0 whose last tap l*s - p + d(K-1) still lies in
    the padded sequence, i.e. <= L_in - 1 + p (brute force, no closed form)."""
    n = 0
    while n * stride - padding + dilation * (K - 1) <= L_in - 1 + padding:
        n += 1
    return n


def forward(x, offsets, weight, bias=None, mask=None, stride=1, padding=0, dilation=1, groups=1):
    x, offsets, weight, bias, mask = map(_np, (x, offsets, weight, bias, mask))
    B, C_in, L_in = x.shape
    C_out, cpg, K = weight.shape
    G = offsets.shape[1]
    L_out = offsets.shape[2]
    opg = C_out // groups
    cpo = C_in // G
    idx = np.arange(L_in, dtype=np.float64)
    out = np.zeros((B, C_out, L_out), dtype=np.float64)
    for b in range(B):
        for co in range(C_out):
            grp = co // opg
            for l in range(L_out):
                acc = 0.0
                for cl in range(cpg):
                    ci = grp * cpg + cl
                    g = ci // cpo
                    for k in range(K):
                        pos = l * stride - padding + k * dilation + offsets[b, g, l, k]
                        hat = np.maximum(0.0, 1.0 - np.abs(pos - idx))
                        v = float(np.dot(hat, x[b, ci]))
                        if mask is not None:
                            v *= mask[b, g, l, k]
                        acc += weight[co, cl, k] * v
                out[b, co, l] = acc + (0.0 if bias is None else bias[co])
    return out
