"""Pins for the oracle's packed-layer generator (CPU only).

The packed layer computes its own offsets (and, modulated, its mask) from
the input with a depthwise trunk and pointwise heads (dc1d page, section
PackedDeformConv1d and the Modulation (DCNv2) paragraph; the block's layers
are a reading, stated in ``oracle/dc1d_oracle.c``).  The C oracle's
generator is pinned against things other than itself:

* CPU float64 ``torch.nn.functional.conv1d`` (the conv1d operator page's
  definition, section Description): a depthwise conv (groups = C_in) with
  the layer's stride, padding and dilation, then kernel-1 convs for the
  heads, reshaped [B, G, K, L_out] -> [B, G, L_out, K], and
  ``torch.sigmoid`` for the mask;
* the page's statement that a zero-initialised mask projection starts
  every tap at exactly 0.5 and so halves the output relative to the
  unmodulated layer;
* a zero offset head reduces the layer to a plain conv1d;
* a bias-only offset head puts the bias of head channel g*K + k at
  offsets[:, g, :, k].
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

# (B, C_in, C_out, L_in, K, stride, padding, dilation, groups, G, modulated)
SHAPES = [
    (2, 4, 4, 12, 3, 1, 4, 4, 4, 4, True),      # the page's layer form: depthwise, "same", d4
    (1, 6, 3, 15, 2, 2, 1, 1, 1, 3, False),
    (2, 6, 6, 11, 3, 1, 1, 2, 3, 2, True),
    (1, 4, 8, 9, 1, 3, 0, 1, 2, 1, True),
    (3, 2, 2, 16, 5, 2, 3, 3, 2, 2, False),
]


def make_case(shape, seed, scale=0.5):
    B, C_in, C_out, L_in, K, s, p, d, groups, G, modulated = shape
    r = np.random.default_rng(seed)
    c = {
        "x": r.standard_normal((B, C_in, L_in)),
        "tw": r.standard_normal((C_in, 1, K)),
        "tb": r.standard_normal(C_in),
        "ow": r.standard_normal((G * K, C_in, 1)) * scale,
        "ob": r.standard_normal(G * K),
        "mw": r.standard_normal((G * K, C_in, 1)) if modulated else None,
        "mb": r.standard_normal(G * K) if modulated else None,
        "w": r.standard_normal((C_out, C_in // groups, K)),
        "b": r.standard_normal(C_out),
        "kw": dict(stride=s, padding=p, dilation=d),
        "groups": groups, "G": G, "K": K,
    }
    return c


def heads(c):
    return oracle.packed_heads(c["x"], c["tw"], c["tb"], c["ow"], c["ob"], c["mw"], c["mb"], **c["kw"])


def run(c):
    return oracle.packed_forward(c["x"], c["tw"], c["tb"], c["ow"], c["ob"], c["w"], c["b"], c["mw"], c["mb"],
                                 groups=c["groups"], **c["kw"])


def torch_heads(c):
    t = lambda a: None if a is None else torch.tensor(a, dtype=torch.float64)
    x = t(c["x"])
    trunk = F.conv1d(x, t(c["tw"]), t(c["tb"]), groups=x.shape[1], **c["kw"])
    B, L_out = x.shape[0], trunk.shape[2]

    def head(w, b):
        z = F.conv1d(trunk, t(w), t(b))                        # [B, G*K, L_out]
        return z.reshape(B, c["G"], c["K"], L_out).permute(0, 1, 3, 2)

    off = head(c["ow"], c["ob"]).numpy()
    mask = torch.sigmoid(head(c["mw"], c["mb"])).numpy() if c["mw"] is not None else None
    return off, mask


def close(a, b, rel=1e-12):
    scale = max(1.0, float(np.abs(b).max()))
    assert a.shape == b.shape
    assert np.abs(a - b).max() <= rel * scale, (np.abs(a - b).max(), scale)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%d_C%d_%d_L%d_K%d_s%d_p%d_d%d_g%d_G%d_m%d" % s)
def test_generator_equals_conv1d_composition(shape):
    c = make_case(shape, seed=21)
    off, mask = heads(c)
    toff, tmask = torch_heads(c)
    close(off, toff)
    if c["mw"] is None:
        assert mask is None
    else:
        close(mask, tmask)


def test_zero_mask_projection_halves_the_output():
    c = make_case(SHAPES[0], seed=22)
    c["mw"] = np.zeros_like(c["mw"])
    c["mb"] = np.zeros_like(c["mb"])
    out, off, mask = run(c)
    assert np.all(mask == 0.5)
    c0 = dict(c, mw=None, mb=None)
    out0, off0, mask0 = run(c0)
    assert mask0 is None and np.array_equal(off, off0)
    b = c["b"][None, :, None]
    close(out - b, 0.5 * (out0 - b))


@pytest.mark.parametrize("shape", SHAPES[:4])
def test_zero_offset_head_is_plain_conv1d(shape):
    c = make_case(shape, seed=23)
    c["ow"] = np.zeros_like(c["ow"])
    c["ob"] = np.zeros_like(c["ob"])
    c["mw"], c["mb"] = None, None
    out, off, _ = run(c)
    assert not off.any()
    ref = F.conv1d(torch.tensor(c["x"]), torch.tensor(c["w"]), torch.tensor(c["b"]), groups=c["groups"],
                   **c["kw"]).numpy()
    close(out, ref)


def test_bias_only_offset_head_places_each_channel():
    c = make_case(SHAPES[2], seed=24)
    c["ow"] = np.zeros_like(c["ow"])
    G, K = c["G"], c["K"]
    c["ob"] = np.arange(G * K, dtype=np.float64) + 0.25
    off, _ = heads(c)
    for g in range(G):
        for k in range(K):
            assert np.all(off[:, g, :, k] == g * K + k + 0.25)


@pytest.mark.parametrize("shape", SHAPES)
def test_constrained_packed_is_constrained_forward_of_the_generated_offsets(shape):
    """The constrained packed layer: the unconstrained generator's offsets,
    fed to the constrained forward (pinned on its own); with the offsets
    scaled up most taps leave their receptive field, so the two modes
    differ."""
    c = make_case(shape, seed=27, scale=4.0)
    out, off, mask = oracle.packed_forward(c["x"], c["tw"], c["tb"], c["ow"], c["ob"], c["w"], c["b"], c["mw"],
                                           c["mb"], groups=c["groups"], constrained=True, **c["kw"])
    off0, mask0 = heads(c)
    assert np.array_equal(off, off0)
    ref = oracle.forward(c["x"], off0, c["w"], c["b"], mask0, groups=c["groups"], constrained=True, **c["kw"])
    assert np.array_equal(out, ref)
    free, _, _ = run(c)
    assert np.abs(out - free).max() > 1e-6


def test_constrained_packed_with_zero_offset_head_is_plain_conv1d():
    c = make_case(SHAPES[2], seed=28)
    c["ow"] = np.zeros_like(c["ow"])
    c["ob"] = np.zeros_like(c["ob"])
    c["mw"], c["mb"] = None, None
    out, _, _ = oracle.packed_forward(c["x"], c["tw"], c["tb"], c["ow"], c["ob"], c["w"], c["b"], None, None,
                                      groups=c["groups"], constrained=True, **c["kw"])
    ref = F.conv1d(torch.tensor(c["x"]), torch.tensor(c["w"]), torch.tensor(c["b"]), groups=c["groups"],
                   **c["kw"]).numpy()
    close(out, ref)


def test_sigmoid_values():
    c = make_case(SHAPES[0], seed=25)
    c["mw"] = np.zeros_like(c["mw"])
    c["mb"] = np.array([-40.0, -1.0, 0.0, 1.0, 40.0, 2.0] * (c["mw"].shape[0] // 6 + 1))[: c["mw"].shape[0]]
    _, mask = heads(c)
    z = c["mb"]
    expect = np.where(z >= 0, 1.0 / (1.0 + np.exp(-np.abs(z))), np.exp(-np.abs(z)) / (1.0 + np.exp(-np.abs(z))))
    K = c["K"]
    for gk, e in enumerate(expect):
        close(mask[:, gk // K, :, gk % K], np.full(mask[:, 0, :, 0].shape, e), 1e-15)


def test_shape_errors():
    c = make_case(SHAPES[0], seed=26)
    with pytest.raises(ValueError):
        oracle.packed_heads(c["x"], c["tw"][:, :, :2], None, c["ow"], None, **c["kw"])
    with pytest.raises(ValueError):
        oracle.packed_heads(c["x"], c["tw"], None, c["ow"][:-1], None, **c["kw"])
    with pytest.raises(ValueError):
        oracle.packed_heads(c["x"], c["tw"], None, c["ow"], None, c["ow"][:, :-1], **c["kw"])
