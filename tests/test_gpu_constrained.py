"""GPU parity of the constrained mode (dc1d_forward_constrained and
dc1d_backward_constrained through the C ABI) against the oracle's
constrained mode (pinned in test_oracle_constrained.py).

Same tolerances as the unconstrained parity tests (test_gpu_parity.py and
test_gpu_backward.py); the shapes reuse their ragged cases, whose offsets
are wide enough that many taps are held at their window's edges, and so
reach every forward kernel family.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import test_gpu_backward as gb
import test_gpu_parity as gp
from deformable_convolution_amd import dc1d, inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.mark.parametrize("w", gp._shape_cases(), ids=lambda w: w.name)
def test_constrained_forward_ragged_shapes(w):
    print("constrained case", w, flush=True)
    t = inputs.make_inputs(w, seed=5)
    g = gp.to_dev(t)
    got = gp.gpu_forward(w, g, constrained=True)
    torch.cuda.synchronize()
    ref = oracle.forward(t["x"], t["offsets"], t["weight"], t["bias"], t["mask"], stride=w.stride,
                         padding=w.padding, dilation=w.dilation, groups=w.groups, constrained=True)
    gp.check(w, got, ref, "constrained")
    # the mode matters on these inputs: some tap left its window
    k = np.arange(w.K)
    off = t["offsets"].double().numpy()
    assert ((off < -k * w.dilation) | (off > (w.K - 1 - k) * w.dilation)).any()


@pytest.mark.parametrize("name", ["dc1d_layer", "depthwise"])
def test_constrained_forward_workloads(name):
    w = inputs.WORKLOADS[name].with_batch(1)
    if name == "depthwise":
        w = inputs.custom("depthwise[C=64]", B=1, C_in=64, C_out=64, L_in=4096, K=5, padding=2, dilation=2,
                          groups=64, G=64, L_out=4092, x_dist=("normal", 0.0, 1.0), off_dist=("uniform", -4.0, 4.0),
                          w_var=1 / 5)
    t = inputs.make_inputs(w, seed=6)
    got = gp.gpu_forward(w, gp.to_dev(t), constrained=True)
    torch.cuda.synchronize()
    ref = oracle.forward(t["x"], t["offsets"], t["weight"], t["bias"], t["mask"], stride=w.stride,
                         padding=w.padding, dilation=w.dilation, groups=w.groups, constrained=True)
    gp.check(w, got, ref, "constrained")


def test_constrained_equals_unconstrained_inside_the_window():
    w = inputs.custom("inside", B=2, C_in=32, C_out=64, L_in=80, K=4, padding=3, dilation=2, G=2, L_out=80)
    t = inputs.make_inputs(w, seed=7)
    k = torch.arange(w.K, dtype=torch.float32)
    lo, hi = -k * w.dilation, (w.K - 1 - k) * w.dilation
    t["offsets"] = lo + torch.rand(t["offsets"].shape, generator=torch.Generator().manual_seed(8)) * (hi - lo)
    g = gp.to_dev(t)
    a = gp.gpu_forward(w, g, constrained=True)
    b = gp.gpu_forward(w, g)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("w", gb.fp32_shapes()[:8], ids=lambda w: w.name)
def test_constrained_backward(w):
    print("constrained backward case", w, flush=True)
    t = inputs.make_inputs(w, seed=9)
    gen = torch.Generator().manual_seed(10)
    dout = torch.randn((w.B, w.C_out, w.L_out), generator=gen, dtype=torch.float32)
    g = gp.to_dev(t)
    got = dc1d.backward(g["x"], g["offsets"], g["weight"], dout.to(DEV), g["mask"], stride=w.stride,
                        padding=w.padding, dilation=w.dilation, groups=w.groups, constrained=True)
    torch.cuda.synchronize()
    ref = oracle.backward(t["x"], t["offsets"], t["weight"], dout, t["mask"], stride=w.stride, padding=w.padding,
                          dilation=w.dilation, groups=w.groups, constrained=True)
    n = gb.terms(w)
    for key, r in ref.items():
        if r is None:
            continue
        a = got[key].double().cpu().numpy()
        if r.size == 0:
            continue
        rms = math.sqrt(float(np.mean(r ** 2)))
        tol = 1e-5 * math.sqrt(n[key]) * rms + 1e-6
        err = float(np.abs(a - r).max())
        assert err <= tol, "%s grad_%s: max|err| %.3g > %.3g" % (w.name, key, err, tol)


def test_constrained_rejects_huge_dilation():
    """(K-1)*dilation = 2^24: the tap bounds would not be exact floats."""
    K, d = 17, 1 << 20
    L_in = (K - 1) * d + 1
    assert oracle.output_length(L_in, K, 1, 0, d) == 1
    x = torch.zeros((1, 1, L_in), device=DEV)
    off = torch.zeros((1, 1, 1, K), device=DEV)
    wt = torch.ones((1, 1, K), device=DEV)
    y = dc1d.forward(x, off, wt, dilation=d)  # unconstrained: accepted
    torch.cuda.synchronize()
    assert y.shape == (1, 1, 1)
    with pytest.raises(dc1d.Dc1dValueError):
        dc1d.forward(x, off, wt, dilation=d, constrained=True)
