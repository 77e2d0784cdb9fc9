"""Pins for the oracle's constrained mode (CPU only).

The dc1d page (section Usage / DeformConv1d) keeps each tap inside its
receptive field by default, without giving the rule.  The reading taken
(oracle.constrain_offsets): the receptive field of output l is the
undeformed kernel's window [l*s - p, l*s - p + (K-1)*d], and every tap's
sampling position is clamped into it.  Being a reading, it is pinned by
what it implies rather than by printed values:

* K = 1: the window is one point, so the output ignores the offsets and is
  the kernel-1 conv1d (CPU float64 ``conv1d``);
* offsets that already keep every tap inside the window change nothing;
* offsets far beyond the window put every tap at its edge: the output is
  a conv1d whose whole weight sits on the last (or first) tap;
* the hat-form brute force with the position (not the offset) clamped to
  the window, an independent formulation;
* the backward equals central finite differences of the constrained
  forward, with zero offset gradient where a tap is held at an edge.
Planted mistakes in the clamp (bounds mirrored, the per-tap cell
[base - d, base + d] instead of the window, a missing derivative factor)
each fail one of them.
"""
import itertools

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

# (B, C_in, C_out, L_in, K, stride, padding, dilation, groups, G)
SHAPES = [
    (1, 2, 3, 12, 3, 1, 1, 1, 1, 1),
    (2, 4, 4, 15, 4, 2, 3, 2, 2, 2),
    (1, 3, 6, 14, 2, 1, 0, 3, 3, 3),
    (2, 2, 2, 11, 5, 1, 4, 1, 1, 2),
]


def case(shape, seed, off):
    B, C_in, C_out, L_in, K, s, p, d, groups, G = shape
    r = np.random.default_rng(seed)
    L_out = oracle.output_length(L_in, K, s, p, d)
    return {
        "x": r.standard_normal((B, C_in, L_in)),
        "offsets": off(r, (B, G, L_out, K), K, d),
        "weight": r.standard_normal((C_out, C_in // groups, K)),
        "bias": r.standard_normal(C_out),
        "kw": dict(stride=s, padding=p, dilation=d, groups=groups),
    }


def fwd(c, constrained=True, **over):
    a = dict(c, **over)
    return oracle.forward(a["x"], a["offsets"], a["weight"], a["bias"], None, constrained=constrained, **a["kw"])


def close(a, b, rel=1e-12):
    scale = max(1.0, float(np.abs(b).max()))
    assert a.shape == b.shape
    assert np.abs(a - b).max() <= rel * scale, (np.abs(a - b).max(), scale)


def wide(r, shape, K, d):
    return r.uniform(-3.0 * K * d, 3.0 * K * d, shape)


def inside(r, shape, K, d):
    k = np.arange(K)
    return r.uniform(0, 1, shape) * ((K - 1) * d) - k * d  # in [-k*d, (K-1-k)*d]


def conv1d(x, w, b, kw):
    return F.conv1d(torch.tensor(x), torch.tensor(w), torch.tensor(b), **kw).numpy()


@pytest.mark.parametrize("shape", SHAPES)
def test_k1_ignores_offsets(shape):
    B, C_in, C_out, L_in, K, s, p, d, groups, G = shape
    shape = (B, C_in, C_out, L_in, 1, s, p, d, groups, G)
    c = case(shape, 31, wide)
    close(fwd(c), conv1d(c["x"], c["weight"], c["bias"], c["kw"]))


@pytest.mark.parametrize("shape", SHAPES)
def test_offsets_inside_the_window_change_nothing(shape):
    c = case(shape, 32, inside)
    assert np.array_equal(fwd(c), fwd(c, constrained=False))


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("sign", [1, -1])
def test_far_offsets_pin_every_tap_to_an_edge(shape, sign):
    c = case(shape, 33, lambda r, sh, K, d: sign * r.uniform(1e3, 1e4, sh))
    w = c["weight"]
    w_edge = np.zeros_like(w)
    w_edge[:, :, -1 if sign > 0 else 0] = w.sum(axis=2)
    close(fwd(c), conv1d(c["x"], w_edge, c["bias"], c["kw"]))


def hat_clamped(x, offsets, w, b, s, p, d, groups):
    """Brute force: position clamped (in position space) to the window, then
    the hat-weighted sum over every input index."""
    B, C_in, L_in = x.shape
    C_out, cpg, K = w.shape
    G, L_out = offsets.shape[1], offsets.shape[2]
    cpo, opg = C_in // G, C_out // groups
    idx = np.arange(L_in)
    out = np.zeros((B, C_out, L_out))
    for bb, co, l in itertools.product(range(B), range(C_out), range(L_out)):
        grp = co // opg
        acc = b[co]
        lo, hi = l * s - p, l * s - p + (K - 1) * d
        for cl in range(cpg):
            ci = grp * cpg + cl
            for k in range(K):
                pos = min(max(l * s - p + k * d + offsets[bb, ci // cpo, l, k], lo), hi)
                acc += w[co, cl, k] * float(np.sum(x[bb, ci] * np.maximum(0.0, 1.0 - np.abs(pos - idx))))
        out[bb, co, l] = acc
    return out


@pytest.mark.parametrize("shape", SHAPES)
def test_equals_position_clamped_hat_form(shape):
    c = case(shape, 34, wide)
    kw = c["kw"]
    close(fwd(c), hat_clamped(c["x"], c["offsets"], c["weight"], c["bias"], kw["stride"], kw["padding"],
                              kw["dilation"], kw["groups"]))


def fd_offsets(shape, seed):
    """Offsets away from both the window edges and the integers: half far
    outside (clamped), half inside with fractions in [0.2, 0.8]."""
    def gen(r, sh, K, d):
        k = np.arange(K)
        lo, hi = -k * d, (K - 1 - k) * d
        n = r.integers(0, max(1, (K - 1) * d), sh)
        inner = lo + n + r.uniform(0.2, 0.8, sh)
        inner = np.where(inner < hi - 0.1, inner, lo + r.uniform(0.2, 0.8, sh))
        far = np.where(r.uniform(size=sh) < 0.5, hi + 2.5, lo - 2.5)
        return np.where(r.uniform(size=sh) < 0.5, inner, far)
    return case(shape, seed, gen)


@pytest.mark.parametrize("shape", SHAPES[:3])
def test_backward_equals_finite_differences(shape):
    c = fd_offsets(shape, 35)
    B, C_out, L_out = c["x"].shape[0], c["weight"].shape[0], c["offsets"].shape[2]
    dout = np.random.default_rng(36).standard_normal((B, C_out, L_out))
    g = oracle.backward(c["x"], c["offsets"], c["weight"], dout, None, constrained=True, **c["kw"])

    def objective(**over):
        return float((dout * fwd(c, **over)).sum())

    for name, h in (("x", 0.5), ("weight", 0.5), ("offsets", 0.05)):
        base = c[name]
        fd = np.zeros_like(base)
        for idx in itertools.product(*[range(n) for n in base.shape]):
            up, dn = base.copy(), base.copy()
            up[idx] += h
            dn[idx] -= h
            fd[idx] = (objective(**{name: up}) - objective(**{name: dn})) / (2 * h)
        close(g[name], fd, 1e-9)
    K, d = c["offsets"].shape[-1], c["kw"]["dilation"]
    k = np.arange(K)
    held = (c["offsets"] < -k * d) | (c["offsets"] >= (K - 1 - k) * d)
    assert held.any() and not g["offsets"][held].any()


# --- the pins must catch plausible mistakes in the clamp -----------------------

def _mirrored(offsets, dilation):
    o = np.asarray(offsets, dtype=np.float64)
    k = np.arange(o.shape[-1])
    return np.clip(o, -(o.shape[-1] - 1 - k) * dilation, k * dilation)


def _own_cell(offsets, dilation):
    o = np.asarray(offsets, dtype=np.float64)
    return np.clip(o, -dilation, dilation)


def _unclamped_upper(offsets, dilation):
    o = np.asarray(offsets, dtype=np.float64)
    k = np.arange(o.shape[-1])
    return np.maximum(o, -k * dilation)


PIN_CALLS = [
    lambda: test_k1_ignores_offsets(SHAPES[1]),
    lambda: test_offsets_inside_the_window_change_nothing(SHAPES[1]),
    lambda: test_far_offsets_pin_every_tap_to_an_edge(SHAPES[1], 1),
    lambda: test_far_offsets_pin_every_tap_to_an_edge(SHAPES[1], -1),
    lambda: test_equals_position_clamped_hat_form(SHAPES[2]),
]


@pytest.mark.parametrize("mutant", [_mirrored, _own_cell, _unclamped_upper], ids=lambda f: f.__name__)
def test_pins_catch_clamp_mutants(mutant, monkeypatch):
    monkeypatch.setattr(oracle, "constrain_offsets", mutant)
    caught = 0
    for call in PIN_CALLS:
        try:
            call()
        except AssertionError:
            caught += 1
    assert caught, "no pin caught %s" % mutant.__name__


def test_pins_catch_a_missing_clamp_derivative(monkeypatch):
    real = oracle.backward

    def no_factor(*a, **kw):
        kw["constrained"] = False
        args = list(a)
        args[1] = oracle.constrain_offsets(args[1], kw.get("dilation", 1))
        return real(*args, **kw)

    monkeypatch.setattr(oracle, "backward", no_factor)
    with pytest.raises(AssertionError):
        test_backward_equals_finite_differences(SHAPES[0])
