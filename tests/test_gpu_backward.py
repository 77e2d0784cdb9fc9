"""GPU parity of the backward: libdc1d's dc1d_backward through the C ABI
against the oracle's backward (itself pinned in test_oracle_backward.py).

Tolerance, per gradient, elementwise:
  * fp32: |gpu - oracle| <= 1e-5 * sqrt(n) * rms(oracle) + 1e-6
    with n the number of products summed into one element (fp32
    accumulation; the oracle is double): grad_x: (C_out/groups) * K * 2;
    grad_offsets and grad_mask: (C_in/G) * (C_out/groups); grad_weight and
    grad_bias: B * L_out.
  * bf16 (bf16 storage, fp32 arithmetic, each gradient rounded once):
    |gpu - oracle| <= 2e-2 * max(|oracle|, rms(oracle)), the forward's bf16
    bound.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from deformable_convolution_amd import dc1d, inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def terms(w):
    opg = w.C_out // w.groups
    cpo = w.C_in // w.G
    return {"x": opg * w.K * 2, "offsets": cpo * opg, "mask": cpo * opg, "weight": max(1, w.B * w.L_out),
            "bias": max(1, w.B * w.L_out)}


def run_backward(w, seed=0):
    print("backward case", w, "seed", seed, flush=True)
    t = inputs.make_inputs(w, seed=seed)
    gen = torch.Generator().manual_seed(seed + 1000)
    dout = torch.randn((w.B, w.C_out, w.L_out), generator=gen, dtype=torch.float32)
    if w.dtype == "bf16":
        dout = dout.to(torch.bfloat16)
    g = {k: (v.to(DEV) if v is not None else None) for k, v in t.items()}
    got = dc1d.backward(g["x"], g["offsets"], g["weight"], dout.to(DEV), g["mask"], stride=w.stride,
                        padding=w.padding, dilation=w.dilation, groups=w.groups)
    torch.cuda.synchronize()
    ref = oracle.backward(t["x"], t["offsets"], t["weight"], dout, t["mask"], stride=w.stride, padding=w.padding,
                          dilation=w.dilation, groups=w.groups)
    n = terms(w)
    for k, r in ref.items():
        if r is None:
            assert k not in got
            continue
        a = got[k].double().cpu().numpy()
        assert a.shape == r.shape, k
        assert np.isfinite(a).all(), k
        if r.size == 0:
            continue
        rms = math.sqrt(float(np.mean(r ** 2)))
        if w.dtype == "f32":
            tol = 1e-5 * math.sqrt(n[k]) * rms + 1e-6
            err = float(np.abs(a - r).max())
            assert err <= tol, "%s grad_%s: max|err| %.3g > %.3g" % (w.name, k, err, tol)
        else:
            assert got[k].dtype == torch.bfloat16, k
            bad = np.abs(a - r) > 2e-2 * np.maximum(np.abs(r), rms)
            assert not bad.any(), "%s grad_%s: %d elements beyond the bf16 bound" % (w.name, k, int(bad.sum()))
    return got, ref


def fp32_shapes():
    cases = []
    # (B, C_in, C_out, L_in, K, s, p, d, groups, G, mask, off_scale)
    spec = [
        (1, 4, 4, 32, 3, 1, 0, 1, 1, 1, False, 2.0),
        (2, 64, 128, 40, 3, 1, 1, 1, 1, 1, False, 2.0),
        (3, 33, 70, 57, 5, 2, 3, 2, 1, 3, True, 6.0),
        (2, 96, 200, 129, 4, 1, 0, 3, 1, 4, False, 3.0),
        (1, 40, 36, 300, 7, 3, 5, 1, 1, 8, True, 30.0),
        (5, 16, 48, 11, 1, 1, 0, 1, 1, 2, False, 1.5),
        (2, 12, 18, 50, 3, 1, 1, 2, 3, 4, True, 4.0),
        (2, 24, 24, 100, 5, 1, 2, 2, 24, 24, True, 4.0),
        (2, 8, 24, 90, 3, 2, 1, 1, 8, 2, False, 3.0),
        (1, 6, 6, 500, 3, 1, 1, 1, 6, 6, False, 200.0),
        (2, 16, 16, 300, 3, 2, 1, 1, 16, 16, True, 3.0),     # depthwise, strided (gathered grad_x)
        (1, 8, 8, 700, 9, 1, 4, 24, 8, 8, True, 5.0),       # depthwise, wide dilation (scattered grad_x)
        (1, 4, 4, 1500, 5, 1, 2, 2, 4, 4, False, 20.0),     # depthwise, some samples moved > 16 (fix pass)
        (2, 16, 16, 1100, 7, 1, 9, 3, 16, 16, True, 6.0),   # depthwise, wide padding, three gather tiles
        (2, 12, 12, 905, 4, 3, 5, 2, 12, 4, False, 7.0),    # depthwise, stride 3, offsets shared by 3 channels
    ]
    for i, (B, C_in, C_out, L_in, K, s, p, d, groups, G, mask, sc) in enumerate(spec):
        L_out = oracle.output_length(L_in, K, s, p, d)
        cases.append(inputs.custom("bwd%d" % i, B=B, C_in=C_in, C_out=C_out, L_in=L_in, K=K, stride=s, padding=p,
                                   dilation=d, groups=groups, G=G, L_out=L_out, off_dist=("uniform", -sc, sc),
                                   mask_dist=("sigmoid_normal", 0.0, 1.0) if mask else None))
    return cases


@pytest.mark.parametrize("w", fp32_shapes(), ids=lambda w: w.name)
def test_backward_ragged_shapes(w):
    run_backward(w, seed=4)


@pytest.mark.parametrize("name", ["tiny", "dc1d_layer", "depthwise"])
def test_backward_workloads_reduced_batch(name):
    w = inputs.WORKLOADS[name]
    if name != "tiny":
        w = w.with_batch(1)
    if name == "depthwise":
        w = inputs.custom("depthwise[C=128]", B=1, C_in=128, C_out=128, L_in=4096, K=5, padding=2, dilation=2,
                          groups=128, G=128, L_out=4092, x_dist=("normal", 0.0, 1.0),
                          off_dist=("uniform", -4.0, 4.0), w_var=1 / 5)
    run_backward(w)


def test_backward_mask_of_ones_equals_no_mask_except_grad_x_rounding():
    w = inputs.custom("ones", B=2, C_in=16, C_out=32, L_in=64, K=3, padding=1, G=2, L_out=64,
                      mask_dist=("sigmoid_normal", 0.0, 1.0))
    t = {k: (v.to(DEV) if v is not None else None) for k, v in inputs.make_inputs(w, seed=7).items()}
    dout = torch.randn((w.B, w.C_out, w.L_out), device=DEV)
    ones = torch.ones_like(t["mask"])
    a = dc1d.backward(t["x"], t["offsets"], t["weight"], dout, ones, padding=1)
    b = dc1d.backward(t["x"], t["offsets"], t["weight"], dout, None, padding=1)
    torch.cuda.synchronize()
    for k in ("offsets", "weight", "bias"):
        assert torch.equal(a[k], b[k]), k
    assert torch.allclose(a["x"], b["x"], rtol=1e-5, atol=1e-6)


def test_backward_subset_of_gradients_and_empty_batch():
    w = inputs.custom("subset", B=1, C_in=8, C_out=8, L_in=30, K=3, L_out=28)
    t = {k: (v.to(DEV) if v is not None else None) for k, v in inputs.make_inputs(w, seed=8).items()}
    dout = torch.randn((1, 8, 28), device=DEV)
    only_b = dc1d.backward(t["x"], t["offsets"], t["weight"], dout, need=("bias",))
    torch.cuda.synchronize()
    assert set(only_b) == {"bias"}
    assert torch.allclose(only_b["bias"], dout.sum(dim=(0, 2)), rtol=1e-5, atol=1e-5)
    w0 = w.with_batch(0)
    t0 = {k: (v.to(DEV) if v is not None else None) for k, v in inputs.make_inputs(w0, seed=8).items()}
    g0 = dc1d.backward(t0["x"], t0["offsets"], t0["weight"], torch.zeros((0, 8, 28), device=DEV))
    torch.cuda.synchronize()
    assert torch.count_nonzero(g0["weight"]) == 0 and torch.count_nonzero(g0["bias"]) == 0


def bf16_shapes():
    cases = []
    # (B, C_in, C_out, L_in, K, s, p, d, groups, G, mask, off_scale)
    spec = [
        (2, 64, 96, 77, 3, 1, 1, 1, 1, 2, True, 3.0),        # dense, masked
        (1, 40, 36, 300, 7, 3, 5, 1, 1, 8, False, 30.0),     # dense, strided, wide offsets
        (2, 12, 18, 50, 3, 1, 1, 2, 3, 4, True, 4.0),        # grouped
        (2, 16, 16, 300, 3, 2, 1, 1, 16, 16, True, 3.0),     # depthwise, strided (gathered grad_x)
        (1, 8, 8, 700, 9, 1, 4, 24, 8, 8, False, 5.0),       # depthwise, wide dilation (scattered grad_x)
        (1, 4, 4, 1500, 5, 1, 2, 2, 4, 4, True, 20.0),       # depthwise, samples moved > 16 (fix pass)
    ]
    for i, (B, C_in, C_out, L_in, K, s, p, d, groups, G, mask, sc) in enumerate(spec):
        L_out = oracle.output_length(L_in, K, s, p, d)
        cases.append(inputs.custom("bwd_bf16_%d" % i, B=B, C_in=C_in, C_out=C_out, L_in=L_in, K=K, stride=s,
                                   padding=p, dilation=d, groups=groups, G=G, L_out=L_out, dtype="bf16",
                                   off_dist=("uniform", -sc, sc),
                                   mask_dist=("sigmoid_normal", 0.0, 1.0) if mask else None))
    return cases


@pytest.mark.parametrize("w", bf16_shapes(), ids=lambda w: w.name)
def test_backward_bf16_ragged_shapes(w):
    run_backward(w, seed=6)


@pytest.mark.parametrize("name", ["long_seq_bf16", "dcnv2_bf16"])
def test_backward_bf16_workloads_reduced_batch(name):
    run_backward(inputs.WORKLOADS[name].with_batch(1), seed=2)


@pytest.mark.parametrize("G", [1, 4])
def test_dense_backward_repeats_bit_for_bit(G):
    """The dense path sums every gradient in a fixed order (the offset and
    mask gradients per channel block into workspace slots added in slot
    order, the GEMMs unsplit or split-reduced in split order, grad_x
    gathered, grad_bias per channel): the same call twice gives the same
    bits.  (Offsets within the gather's reach of 16 positions.)"""
    w = inputs.custom("bwd_repeat", B=4, C_in=512, C_out=512, L_in=128, K=16, dilation=3, G=G, L_out=83)
    t = {k: (v.to(DEV) if v is not None else None) for k, v in inputs.make_inputs(w, seed=11).items()}
    mask = torch.rand(t["offsets"].shape, device=DEV)
    dout = torch.randn((w.B, w.C_out, w.L_out), device=DEV)
    a = dc1d.backward(t["x"], t["offsets"], t["weight"], dout, mask, dilation=3)
    b = dc1d.backward(t["x"], t["offsets"], t["weight"], dout, mask, dilation=3)
    torch.cuda.synchronize()
    for k in ("x", "offsets", "mask", "weight", "bias"):
        assert torch.equal(a[k], b[k]), k


def test_depthwise_backward_repeats_bit_for_bit():
    """The depthwise gather pass sums grad_weight and grad_bias per block
    (waves in order) into workspace slots that a second launch adds in block
    order; grad_x and the offset and mask gradients are gathered: the same
    call twice at the measured depthwise size gives the same bits.  (Offsets
    within the gather pass's reach, so no sample is left to its fix pass.)"""
    w = inputs.WORKLOADS["depthwise"]
    t = {k: (v.to(DEV) if v is not None else None) for k, v in inputs.make_inputs(w, seed=12).items()}
    t["offsets"] = t["offsets"].clamp(-15.0, 15.0)
    mask = torch.rand(t["offsets"].shape, device=DEV)
    dout = torch.randn((w.B, w.C_out, w.L_out), device=DEV)
    kw = dict(stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)
    a = dc1d.backward(t["x"], t["offsets"], t["weight"], dout, mask, **kw)
    b = dc1d.backward(t["x"], t["offsets"], t["weight"], dout, mask, **kw)
    torch.cuda.synchronize()
    for k in ("x", "offsets", "mask", "weight", "bias"):
        assert torch.equal(a[k], b[k]), k
