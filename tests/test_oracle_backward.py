"""Pins for the oracle's backward (CPU only).

The oracle's backward (``oracle.backward``) is the term-by-term derivative
of its forward.  It is pinned against things other than itself:

* finite differences of the (already pinned) forward oracle, for every
  gradient; the forward is linear in x, the weight, the bias and the mask,
  so a central difference is exact up to rounding for any step, and it is
  piecewise linear in each offset, so a central difference whose step does
  not cross an integer is exact too (the dc1d page checks its offset
  gradient against a finite difference, section Demo notebook);
* at zero offsets, CPU autograd of ``torch.nn.functional.conv1d`` in
  float64 (the conv1d operator page's definition, section Description);
* at non-integer offsets, CPU autograd of an independent formulation that
  never splits a position: the hat form
  ``v(pos) = sum_i x[i] * max(0, 1 - |pos - i|)``;
* at integer offsets, the one-sided (right) difference, the derivative the
  interpolation formula gives with the left neighbour held fixed.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle

# (B, C_in, C_out, L_in, K, stride, padding, dilation, groups, G, mask)
SHAPES = [
    (1, 2, 3, 9, 3, 1, 1, 1, 1, 1, False),
    (2, 4, 6, 11, 2, 2, 2, 2, 2, 2, True),
    (1, 6, 3, 8, 3, 1, 0, 2, 3, 6, False),
    (2, 3, 3, 10, 4, 1, 3, 1, 3, 3, True),
    (1, 4, 2, 7, 1, 2, 1, 1, 1, 4, True),
]


def make_case(shape, seed, frac=(0.15, 0.85), span=4, integer=False):
    B, C_in, C_out, L_in, K, s, p, d, groups, G, mask = shape
    rng = np.random.default_rng(seed)
    L_out = oracle.output_length(L_in, K, s, p, d)
    n = rng.integers(-span, span + 1, (B, G, L_out, K)).astype(np.float64)
    off = n if integer else n + rng.uniform(frac[0], frac[1], n.shape)
    return {
        "x": rng.standard_normal((B, C_in, L_in)),
        "offsets": off,
        "weight": rng.standard_normal((C_out, C_in // groups, K)),
        "bias": rng.standard_normal(C_out),
        "mask": rng.uniform(0.2, 1.5, off.shape) if mask else None,
        "dout": rng.standard_normal((B, C_out, L_out)),
        "kw": dict(stride=s, padding=p, dilation=d, groups=groups),
    }


def objective(c, **over):
    a = {k: c[k] for k in ("x", "offsets", "weight", "bias", "mask")}
    a.update(over)
    out = oracle.forward(a["x"], a["offsets"], a["weight"], a["bias"], a["mask"], **c["kw"])
    return float((c["dout"] * out).sum())


def central(c, name, h):
    base = c[name]
    g = np.zeros_like(base)
    for idx in itertools.product(*[range(n) for n in base.shape]):
        up, dn = base.copy(), base.copy()
        up[idx] += h
        dn[idx] -= h
        g[idx] = (objective(c, **{name: up}) - objective(c, **{name: dn})) / (2 * h)
    return g


def grads(c):
    return oracle.backward(c["x"], c["offsets"], c["weight"], c["dout"], c["mask"], **c["kw"])


def close(a, b, rel=1e-9):
    scale = max(1.0, float(np.abs(b).max()))
    assert np.abs(a - b).max() <= rel * scale, (np.abs(a - b).max(), scale)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%d_C%d_%d_L%d_K%d_s%d_p%d_d%d_g%d_G%d_m%d" % s)
def test_backward_equals_finite_differences(shape):
    c = make_case(shape, seed=11)
    g = grads(c)
    close(g["x"], central(c, "x", 0.5))
    close(g["weight"], central(c, "weight", 0.5))
    close(g["bias"], central(c, "bias", 0.5))
    close(g["offsets"], central(c, "offsets", 0.05))  # fractions stay inside [0.1, 0.9]
    if c["mask"] is not None:
        close(g["mask"], central(c, "mask", 0.5))


def test_integer_offsets_give_the_right_derivative():
    c = make_case(SHAPES[1], seed=12, integer=True)
    g = grads(c)
    h = 0.25
    base = c["offsets"]
    fd = np.zeros_like(base)
    f0 = objective(c)
    for idx in itertools.product(*[range(n) for n in base.shape]):
        up = base.copy()
        up[idx] += h
        fd[idx] = (objective(c, offsets=up) - f0) / h
    close(g["offsets"], fd)


@pytest.mark.parametrize("shape", SHAPES[:4])
def test_zero_offsets_match_conv1d_autograd(shape):
    c = make_case(shape, seed=13)
    c["offsets"] = np.zeros_like(c["offsets"])
    c["mask"] = None
    g = grads(c)
    x = torch.tensor(c["x"], requires_grad=True)
    w = torch.tensor(c["weight"], requires_grad=True)
    b = torch.tensor(c["bias"], requires_grad=True)
    kw = c["kw"]
    out = torch.nn.functional.conv1d(x, w, b, stride=kw["stride"], padding=kw["padding"],
                                     dilation=kw["dilation"], groups=kw["groups"])
    (torch.tensor(c["dout"]) * out).sum().backward()
    close(g["x"], x.grad.numpy(), 1e-12)
    close(g["weight"], w.grad.numpy(), 1e-12)
    close(g["bias"], b.grad.numpy(), 1e-12)


def hat_forward_torch(x, off, w, mask, s, p, d, groups):
    """The hat form in torch ops (autograd-able): every sample is a weighted
    sum over all input positions, weights max(0, 1 - |pos - i|)."""
    B, C_in, L_in = x.shape
    C_out, cpg, K = w.shape
    G, L_out = off.shape[1], off.shape[2]
    cpo = C_in // G
    g_of_ci = torch.arange(C_in) // cpo
    grid = (torch.arange(L_out)[:, None] * s - p + torch.arange(K)[None, :] * d).double()  # [L_out, K]
    pos = grid[None, None] + off[:, g_of_ci]                                               # [B, C_in, L_out, K]
    i = torch.arange(L_in).double()
    hat = torch.clamp(1 - (pos[..., None] - i).abs(), min=0)                               # [..., L_in]
    S = (hat * x[:, :, None, None, :]).sum(-1)                                             # [B, C_in, L_out, K]
    if mask is not None:
        S = S * mask[:, g_of_ci]
    opg = C_out // groups
    outs = []
    for co in range(C_out):
        grp = co // opg
        outs.append(torch.einsum("bclk,ck->bl", S[:, grp * cpg:(grp + 1) * cpg], w[co]))
    return torch.stack(outs, 1)


@pytest.mark.parametrize("shape", SHAPES)
def test_backward_matches_hat_form_autograd(shape):
    c = make_case(shape, seed=14)
    g = grads(c)
    x = torch.tensor(c["x"], requires_grad=True)
    off = torch.tensor(c["offsets"], requires_grad=True)
    w = torch.tensor(c["weight"], requires_grad=True)
    m = torch.tensor(c["mask"], requires_grad=True) if c["mask"] is not None else None
    kw = c["kw"]
    out = hat_forward_torch(x, off, w, m, kw["stride"], kw["padding"], kw["dilation"], kw["groups"])
    (torch.tensor(c["dout"]) * out).sum().backward()
    close(g["x"], x.grad.numpy(), 1e-12)
    close(g["offsets"], off.grad.numpy(), 1e-12)
    close(g["weight"], w.grad.numpy(), 1e-12)
    if m is not None:
        close(g["mask"], m.grad.numpy(), 1e-12)


def test_zero_mask_stops_every_gradient_but_the_mask_and_bias():
    c = make_case(SHAPES[1], seed=15)
    c["mask"] = np.zeros_like(c["mask"])
    g = grads(c)
    assert not g["x"].any() and not g["offsets"].any() and not g["weight"].any()
    assert np.abs(g["mask"]).max() > 0
    close(g["bias"], c["dout"].sum(axis=(0, 2)))


def test_ones_mask_equals_no_mask():
    c = make_case(SHAPES[1], seed=16)
    c["mask"] = np.ones_like(c["mask"])
    g1 = grads(c)
    c["mask"] = None
    g0 = grads(c)
    for k in ("x", "offsets", "weight", "bias"):
        assert np.array_equal(g1[k], g0[k])
