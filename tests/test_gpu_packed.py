"""GPU parity of the packed layer (fp32): libdc1d's dc1d_packed_forward
through the C ABI against the oracle's generator and forward (pinned in
test_oracle_packed.py and test_oracle_pins.py).

Tolerances, elementwise, derived from the arithmetic:
* offsets (a C_in-term fp32 sum over the trunk's K-term fp32 sums):
  tol_o = 1e-5 * sqrt(C_in) * max(rms(offsets), 1);
* mask = sigmoid(z), z like an offset: tol_m = tol_o / 4 + 2^-20 (the
  sigmoid's slope is at most 1/4; the GPU's exponential, exp2 of z*log2(e),
  is off by about (|z| + 2) * 2^-24 relatively, which the sigmoid scales by
  s(1 - s) <= 1/4, plus the final add and the reciprocal instruction,
  within an ulp);
* out: against the oracle's forward evaluated on the offsets and mask the
  GPU generated (checked above against the oracle's generator), with the
  forward's own bound max|err| <= 1e-5 * sqrt(cpg*K): the generator's
  errors are held to theirs, the forward's to its.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from deformable_convolution_amd import dc1d, inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def rms(a):
    return math.sqrt(float(np.mean(a ** 2))) if a.size else 0.0


def run_packed(w, seed=0, check_out=True, constrained=False):
    print("packed case", w, "seed", seed, "constrained", constrained, flush=True)
    t = inputs.make_packed_inputs(w, seed=seed)
    g = {k: (v.to(DEV) if v is not None else None) for k, v in t.items()}
    kw = dict(stride=w.stride, padding=w.padding, dilation=w.dilation)
    got = dc1d.packed_forward(g["x"], g["trunk_weight"], g["trunk_bias"], g["off_weight"], g["off_bias"], g["weight"],
                              g["bias"], g["mask_weight"], g["mask_bias"], groups=w.groups, with_offsets=True,
                              constrained=constrained, **kw)
    torch.cuda.synchronize()
    out, gen = got
    off, mask = gen if w.modulated else (gen, None)
    r_out, r_off, r_mask = oracle.packed_forward(t["x"], t["trunk_weight"], t["trunk_bias"], t["off_weight"],
                                                 t["off_bias"], t["weight"], t["bias"], t["mask_weight"],
                                                 t["mask_bias"], groups=w.groups, constrained=constrained, **kw)
    a_off = off.double().cpu().numpy()
    assert a_off.shape == r_off.shape
    tol_o = 1e-5 * math.sqrt(w.C_in) * max(rms(r_off), 1.0)
    err_o = float(np.abs(a_off - r_off).max())
    assert err_o <= tol_o, "%s offsets: %.3g > %.3g" % (w.name, err_o, tol_o)
    tol_m = tol_o / 4 + 2.0 ** -20
    if w.modulated:
        a_m = mask.double().cpu().numpy()
        err_m = float(np.abs(a_m - r_mask).max())
        assert err_m <= tol_m, "%s mask: %.3g > %.3g" % (w.name, err_m, tol_m)
    else:
        assert mask is None
    if check_out:
        a_out = out.double().cpu().numpy()
        assert a_out.shape == r_out.shape and np.isfinite(a_out).all()
        g_out = oracle.forward(t["x"], a_off, t["weight"], t["bias"], mask.double().cpu().numpy() if w.modulated else None,
                               groups=w.groups, constrained=constrained, **kw)
        tol = 1e-5 * math.sqrt((w.C_in // w.groups) * w.K)
        err = float(np.abs(a_out - g_out).max())
        assert err <= tol, "%s out: %.3g > %.3g" % (w.name, err, tol)
    return out


def shapes():
    # (B, C_in, C_out, L_in, K, s, p, d, groups, G, modulated)
    spec = [
        (2, 48, 96, 100, 3, 1, 1, 1, 1, 2, True),      # dense main conv: MFMA forward
        (3, 16, 24, 77, 5, 2, 2, 2, 4, 4, False),      # grouped, strided: direct forward
        (2, 8, 8, 33, 1, 1, 0, 1, 8, 8, True),         # K = 1, depthwise
        (1, 1, 1, 5, 2, 1, 0, 1, 1, 1, False),         # smallest
        (1, 512, 32, 64, 3, 1, 1, 1, 1, 8, True),      # long head reduction: split head GEMM
        (2, 24, 48, 300, 7, 3, 5, 1, 24, 6, True),     # depthwise multiplier, G < C_in
        (5, 40, 40, 129, 4, 1, 0, 3, 40, 40, False),   # ragged tiles, even K
        # more head tiles than CUs (the persistent head GEMM walks several per
        # workgroup): ragged columns; two row blocks with a ragged second
        (3, 32, 32, 12001, 3, 1, 1, 1, 32, 16, True),
        (2, 50, 50, 9000, 3, 1, 1, 1, 50, 25, True),
        # depthwise with one offset group per channel: strided and dilated,
        # ragged tiles; unmodulated
        (3, 16, 16, 777, 5, 2, 3, 2, 16, 16, True),
        (2, 32, 32, 1000, 3, 1, 1, 1, 32, 32, False),
        # output lengths a multiple of 32: the persistent head kernel.  Four
        # slabs of 32 groups (the workload's shape, smaller); three slabs
        # padded to four, C_in padded to 64, K = 4; one slab (each wave one
        # column block), K = 2, a partial column tile; two slabs, K = 1;
        # strided, two slabs
        (2, 64, 64, 1024, 3, 1, 1, 1, 64, 64, True),
        (3, 40, 40, 99, 4, 1, 0, 1, 40, 40, True),
        (2, 16, 16, 161, 2, 1, 0, 1, 16, 8, False),
        (1, 24, 24, 64, 1, 1, 0, 1, 24, 24, True),
        (2, 32, 32, 255, 3, 2, 1, 1, 32, 32, True),
    ]
    out = []
    for i, (B, C_in, C_out, L_in, K, s, p, d, groups, G, mod) in enumerate(spec):
        L_out = oracle.output_length(L_in, K, s, p, d)
        out.append(inputs.packed_custom("packed%d" % i, B=B, C_in=C_in, C_out=C_out, L_in=L_in, K=K, stride=s,
                                        padding=p, dilation=d, groups=groups, G=G, L_out=L_out, modulated=mod))
    return out


@pytest.mark.parametrize("name", ["packed_page", "packed_page_modulated"])
def test_packed_page_layer(name):
    run_packed(inputs.PACKED_WORKLOADS[name])


@pytest.mark.parametrize("w", shapes(), ids=lambda w: w.name)
def test_packed_ragged_shapes(w):
    run_packed(w, seed=3)


@pytest.mark.parametrize("i", [0, 1, 2, 5, 6, 9])
def test_packed_constrained_shapes(i):
    """The constrained mode on generated offsets: the clamp to the receptive
    field moves a position by no more than the offset's own error, so the
    tolerances are the unconstrained ones; the offsets come back as
    generated."""
    run_packed(shapes()[i], seed=5, constrained=True)


def test_packed_constrained_page_layer():
    run_packed(inputs.PACKED_WORKLOADS["packed_page_modulated"], seed=6, constrained=True)


def test_packed_full_size_workload():
    """The measured workload at full size, in the launch configuration the
    bench times (every element compared)."""
    run_packed(inputs.PACKED_WORKLOADS["packed"], seed=0)


def test_packed_without_offsets_output_matches_with():
    w = inputs.PACKED_WORKLOADS["packed_page_modulated"]
    t = {k: (v.to(DEV) if v is not None else None) for k, v in inputs.make_packed_inputs(w, seed=5).items()}
    args = (t["x"], t["trunk_weight"], t["trunk_bias"], t["off_weight"], t["off_bias"], t["weight"], t["bias"],
            t["mask_weight"], t["mask_bias"])
    kw = dict(padding=w.padding, dilation=w.dilation, groups=w.groups)
    a = dc1d.packed_forward(*args, **kw)
    b, _ = dc1d.packed_forward(*args, with_offsets=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_packed_zero_mask_projection_halves_output():
    """The page's initial state: a zero-initialised mask projection gates
    every tap at 0.5, halving the output relative to the unmodulated layer
    (bias aside)."""
    w = inputs.PACKED_WORKLOADS["packed_page_modulated"]
    t = {k: (v.to(DEV) if v is not None else None) for k, v in inputs.make_packed_inputs(w, seed=6).items()}
    kw = dict(padding=w.padding, dilation=w.dilation, groups=w.groups)
    zw, zb = torch.zeros_like(t["mask_weight"]), torch.zeros_like(t["mask_bias"])
    ym, (off, mask) = dc1d.packed_forward(t["x"], t["trunk_weight"], t["trunk_bias"], t["off_weight"], t["off_bias"],
                                          t["weight"], t["bias"], zw, zb, with_offsets=True, **kw)
    y0 = dc1d.packed_forward(t["x"], t["trunk_weight"], t["trunk_bias"], t["off_weight"], t["off_bias"],
                             t["weight"], t["bias"], **kw)
    torch.cuda.synchronize()
    assert torch.all(mask == 0.5)
    b = t["bias"][None, :, None]
    assert torch.allclose(ym - b, 0.5 * (y0 - b), rtol=1e-6, atol=1e-6)


def test_packed_argument_errors():
    w = inputs.PACKED_WORKLOADS["packed_page_modulated"]
    t = {k: (v.to(DEV) if v is not None else None) for k, v in inputs.make_packed_inputs(w, seed=7).items()}
    kw = dict(padding=w.padding, dilation=w.dilation, groups=w.groups)
    base = [t["x"], t["trunk_weight"], t["trunk_bias"], t["off_weight"], t["off_bias"], t["weight"], t["bias"],
            t["mask_weight"], t["mask_bias"]]
    bad = list(base)
    bad[0] = t["x"].to(torch.bfloat16)
    with pytest.raises(dc1d.Dc1dValueError):
        dc1d.packed_forward(*bad, **kw)
    bad = list(base)
    bad[7] = None  # a mask bias without a mask weight
    with pytest.raises(dc1d.Dc1dValueError):
        dc1d.packed_forward(*bad, **kw)
    bad = list(base)
    bad[5] = t["weight"][:, :, :2].contiguous()  # the main conv's K differs from the trunk's
    with pytest.raises(dc1d.Dc1dValueError):
        dc1d.packed_forward(*bad, **kw)
    bad = list(base)
    bad[3] = t["off_weight"][:-1].contiguous()  # G*K rows not a multiple of K
    with pytest.raises(dc1d.Dc1dValueError):
        dc1d.packed_forward(*bad, **kw)
    x0 = t["x"][:0].contiguous()
    y = dc1d.packed_forward(x0, *base[1:], **kw)
    torch.cuda.synchronize()
    assert y.shape == (0, w.C_out, w.L_out)


# ---- bf16 storage --------------------------------------------------------------
#
# Every tensor of the call in bf16: the generator runs in fp32 on the widened
# parameters, its offsets (and mask) are rounded once to bf16, and the bf16
# forward reads those.  Checked in two parts, each against the oracle with
# the bf16 bound |gpu - oracle| <= 2e-2 * max(|oracle|, rms(oracle))
# elementwise: the generated offsets and mask against the oracle's
# generator, and the output against the oracle's forward of the GPU's own
# bf16 offsets and mask (so that the forward's check does not depend on how
# an offset's rounding moves a sample).

def _bf16_bound(a, r, what):
    rms_r = rms(r)
    bad = np.abs(a - r) > 2e-2 * np.maximum(np.abs(r), rms_r)
    assert not bad.any(), "%s: %d elements beyond the bf16 bound" % (what, int(bad.sum()))


def run_packed_bf16(w, seed=0):
    print("packed bf16 case", w, "seed", seed, flush=True)
    t32 = inputs.make_packed_inputs(w, seed=seed)
    t = {k: (v.to(torch.bfloat16) if v is not None else None) for k, v in t32.items()}
    g = {k: (v.to(DEV) if v is not None else None) for k, v in t.items()}
    kw = dict(stride=w.stride, padding=w.padding, dilation=w.dilation)
    out, gen = dc1d.packed_forward(g["x"], g["trunk_weight"], g["trunk_bias"], g["off_weight"], g["off_bias"],
                                   g["weight"], g["bias"], g["mask_weight"], g["mask_bias"], groups=w.groups,
                                   with_offsets=True, **kw)
    torch.cuda.synchronize()
    off, mask = gen if w.modulated else (gen, None)
    assert out.dtype == torch.bfloat16 and off.dtype == torch.bfloat16
    r_off, r_mask = oracle.packed_heads(t["x"], t["trunk_weight"], t["trunk_bias"], t["off_weight"], t["off_bias"],
                                        t["mask_weight"], t["mask_bias"], **kw)
    _bf16_bound(off.double().cpu().numpy(), r_off, "%s offsets" % w.name)
    if w.modulated:
        _bf16_bound(mask.double().cpu().numpy(), r_mask, "%s mask" % w.name)
    r_out = oracle.forward(t["x"], off.cpu(), t["weight"], t["bias"], mask.cpu() if w.modulated else None,
                           groups=w.groups, **kw)
    a_out = out.double().cpu().numpy()
    assert np.isfinite(a_out).all()
    _bf16_bound(a_out, r_out, "%s out" % w.name)


@pytest.mark.parametrize("name", ["packed_page", "packed_page_modulated"])
def test_packed_bf16_page_layer(name):
    run_packed_bf16(inputs.PACKED_WORKLOADS[name], seed=11)


@pytest.mark.parametrize("i", [0, 1, 3, 4, 8])
def test_packed_bf16_ragged_shapes(i):
    run_packed_bf16(shapes()[i], seed=12)
