"""GPU parity of the 2D modulated deformable convolution (dc2d_forward
through the C ABI) against the oracle's forward2d (pinned in
test_oracle_2d.py).

Tolerances (the oracle is exact up to double rounding):
  * fp32: max |gpu - oracle| <= 1e-5 * sqrt(C_in/groups * kh * kw) *
    max(rms(oracle), 1)
  * bf16 (bf16 storage, samples rounded once to bf16 for the MFMA, fp32
    accumulation, one rounding of the output):
    |gpu - oracle| <= 2e-2 * max(|oracle|, rms(oracle)) elementwise
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from deformable_convolution_amd import dc1d, inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def run2d(w, seed=0, points=None):
    print("2d case", w, "seed", seed, flush=True)
    t = inputs.make_inputs2d(w, seed=seed)
    g = {k: (v.to(DEV) if v is not None else None) for k, v in t.items()}
    kw = dict(stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)
    got = dc1d.forward2d(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], **kw)
    torch.cuda.synchronize()
    ref = oracle.forward2d(t["x"], t["offsets"], t["weight"], t["bias"], t["mask"], **kw)
    a = got.double().cpu().numpy()
    assert a.shape == ref.shape and np.isfinite(a).all()
    rms = math.sqrt(float(np.mean(ref ** 2))) if ref.size else 0.0
    if w.dtype == "f32":
        tol = 1e-5 * math.sqrt(w.C_in // w.groups * w.kh * w.kw)
        err = float(np.abs(a - ref).max())
        assert err <= tol, "%s: max|err| %.3g > %.3g" % (w.name, err, tol)
    else:
        bad = np.abs(a - ref) > 2e-2 * np.maximum(np.abs(ref), rms)
        assert not bad.any(), "%s: %d elements beyond the bf16 bound" % (w.name, int(bad.sum()))
    return dc1d.plan2d(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], **kw)


def shapes():
    # (B, C_in, C_out, H, W, kh, kw, stride, padding, dilation, groups, G, dtype, modulated)
    spec = [
        (2, 32, 64, 13, 11, 3, 3, (1, 1), (1, 1), (1, 1), 1, 1, "f32", True),     # dense, ragged tiles
        (1, 48, 40, 17, 9, 3, 2, (2, 1), (1, 0), (1, 2), 1, 3, "f32", False),     # strides, dilations, G = 3
        (2, 20, 36, 10, 12, 5, 5, (1, 2), (2, 2), (1, 1), 1, 2, "f32", True),     # 5x5, C_in/G not a run multiple
        (1, 70, 33, 8, 8, 1, 1, (1, 1), (0, 0), (1, 1), 1, 7, "f32", True),       # 1x1 taps (Kred = C_in)
        (2, 12, 18, 9, 10, 3, 3, (1, 1), (1, 1), (1, 1), 3, 2, "f32", True),      # grouped -> direct
        (1, 8, 8, 15, 15, 3, 3, (1, 1), (1, 1), (2, 2), 8, 8, "f32", False),      # depthwise -> direct
        (2, 32, 64, 13, 11, 3, 3, (1, 1), (1, 1), (1, 1), 1, 2, "bf16", True),    # bf16 dense
        (1, 16, 16, 12, 12, 3, 3, (2, 2), (1, 1), (1, 1), 4, 4, "bf16", True),    # bf16 grouped
        # one offset group with 1, 4 or 9 taps
        (2, 32, 64, 13, 11, 3, 3, (1, 1), (1, 1), (1, 1), 1, 1, "bf16", True),    # bf16, ragged tiles
        (1, 40, 48, 9, 7, 2, 2, (1, 1), (0, 0), (1, 1), 1, 1, "f32", False),     # 2x2 taps, no mask
        (1, 24, 32, 6, 10, 1, 1, (1, 1), (0, 0), (1, 1), 1, 1, "bf16", True),     # 1x1 taps
        (2, 33, 40, 14, 10, 3, 3, (2, 1), (1, 2), (1, 2), 1, 1, "f32", True),     # strides, dilations, C_in odd
    ]
    out = []
    for i, (B, C_in, C_out, H, W, kh, kw, s, p, d, groups, G, dt, mod) in enumerate(spec):
        Ho, Wo = oracle.output_size2d(H, W, kh, kw, s, p, d)
        out.append(inputs.custom2d("shape2d_%d" % i, B=B, C_in=C_in, C_out=C_out, H=H, W=W, kh=kh, kw=kw, stride=s,
                                   padding=p, dilation=d, groups=groups, G=G, Ho=Ho, Wo=Wo, dtype=dt, modulated=mod,
                                   off_var=2.0))
    return out


@pytest.mark.parametrize("w", shapes(), ids=lambda w: w.name)
def test_2d_ragged_shapes(w):
    run2d(w, seed=3)


def test_2d_shapes_reach_both_paths():
    names = {w.name: None for w in shapes()}
    seen = set()
    for w in shapes():
        t = inputs.make_inputs2d(w.with_batch(1), seed=0)
        g = {k: (v.to(DEV) if v is not None else None) for k, v in t.items()}
        seen.add(dc1d.plan2d(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], stride=w.stride,
                             padding=w.padding, dilation=w.dilation, groups=w.groups))
    assert names and seen == {"im2col2d_gemm_f32", "im2col2d_gemm_bf16", "direct2d"}


@pytest.mark.parametrize("name", ["dcn2d_article", "dcn2d", "dcn2d_bf16"])
def test_2d_workloads(name):
    w = inputs.WORKLOADS_2D[name]
    if name != "dcn2d_article":
        w = w.with_batch(1)  # the oracle's size; the full batch is sampled below
    run2d(w)


@pytest.mark.parametrize("name", ["dcn2d", "dcn2d_bf16"])
def test_2d_full_size_sampled(name):
    """The measured workloads at full size, in the bench's launch
    configuration, against the oracle on whole images of a few batches
    (every batch of one output equals the oracle on that batch alone)."""
    w = inputs.WORKLOADS_2D[name]
    t = inputs.make_inputs2d(w, seed=0)
    g = {k: (v.to(DEV) if v is not None else None) for k, v in t.items()}
    kw = dict(stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)
    got = dc1d.forward2d(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], **kw)
    torch.cuda.synchronize()
    for b in (0, w.B - 1):
        sl = {k: (v[b:b + 1] if v is not None and k in ("x", "offsets", "mask") else v) for k, v in t.items()}
        ref = oracle.forward2d(sl["x"], sl["offsets"], sl["weight"], sl["bias"], sl["mask"], **kw)
        a = got[b:b + 1].double().cpu().numpy()
        rms = math.sqrt(float(np.mean(ref ** 2)))
        if w.dtype == "f32":
            tol = 1e-5 * math.sqrt(w.C_in * w.kh * w.kw)
            assert float(np.abs(a - ref).max()) <= tol
        else:
            assert not (np.abs(a - ref) > 2e-2 * np.maximum(np.abs(ref), rms)).any()


def test_2d_torchvision_issue_demo():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "torchvision_issue_demo.json")))
    x = torch.arange(27.0, device=DEV).reshape(1, 3, 3, 3)
    off = torch.tensor([0, -1, 0, 1, -1, 0.0], device=DEV).reshape(1, 6, 1, 1).repeat(1, 1, 3, 3).contiguous()
    w = torch.tensor([[1, 0, 0], [0, 1, 0], [1, 1, 0], [0, 0, 1], [0, 1, 0.0]], device=DEV).reshape(5, 3, 1, 1)
    out = dc1d.forward2d(x, off, w)
    torch.cuda.synchronize()
    assert torch.equal(out[0].cpu(), torch.tensor(g["printed_output"], dtype=torch.float32))


def test_2d_mask_ones_and_errors():
    w = shapes()[0]
    t = {k: (v.to(DEV) if v is not None else None) for k, v in inputs.make_inputs2d(w, seed=4).items()}
    kw = dict(stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)
    a = dc1d.forward2d(t["x"], t["offsets"], t["weight"], t["bias"], torch.ones_like(t["mask"]), **kw)
    b = dc1d.forward2d(t["x"], t["offsets"], t["weight"], t["bias"], None, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    with pytest.raises(dc1d.Dc1dValueError):
        dc1d.forward2d(t["x"], t["offsets"][:, :-1].contiguous(), t["weight"], t["bias"], None, **kw)
    with pytest.raises(dc1d.Dc1dValueError):
        dc1d.forward2d(t["x"], t["offsets"], t["weight"].to(torch.bfloat16), t["bias"], None, **kw)
    x0 = t["x"][:0].contiguous()
    y = dc1d.forward2d(x0, t["offsets"][:0].contiguous(), t["weight"], t["bias"], None, **kw)
    torch.cuda.synchronize()
    assert y.shape[0] == 0
