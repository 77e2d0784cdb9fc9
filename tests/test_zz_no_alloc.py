"""GPU test of the allocation-free entry point, dc1d_forward_noalloc.

It runs the forward's own kernels with the workspace in the library's
per-device scratch array, so its output must equal dc1d_forward's bit for
bit (the same plan, the same kernels).  Each case makes two calls in a row,
the second on a smaller input, so that what the first call left in the
scratch (split partials, rearranged weights) is there when the second runs:
the second must not read it.  The first call of the file is the entry
point's first use in the process (the scratch address is looked up then).
A shape whose workspace exceeds the scratch is rejected before any launch.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from deformable_convolution_amd import dc1d, inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _dev(t):
    return {k: (v.to(DEV) if v is not None else None) for k, v in t.items()}


def _kw(w):
    return dict(stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)


def _pair(w):
    """(no-alloc output, dc1d_forward output) on the seeded inputs of w."""
    print("no-alloc case", w.name, flush=True)
    t = inputs.make_inputs(w, seed=3)
    g = _dev(t)
    out_na = torch.full((w.B, w.C_out, w.L_out), float("nan"), dtype=g["x"].dtype, device=DEV)
    dc1d.forward_noalloc(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], out=out_na, **_kw(w))
    torch.cuda.synchronize()
    out = dc1d.forward(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], **_kw(w))
    torch.cuda.synchronize()
    return t, out_na, out


def _oracle_points(w, t, got, n=256):
    rng = np.random.default_rng(5)
    pts = np.stack([rng.integers(0, w.B, n), rng.integers(0, w.C_out, n), rng.integers(0, w.L_out, n)], 1)
    ref = oracle.forward_points(t["x"], t["offsets"], t["weight"], pts, t["bias"], t["mask"], **_kw(w))
    g = got[pts[:, 0], pts[:, 1], pts[:, 2]].double().cpu().numpy()
    if w.dtype == "f32":
        assert np.abs(g - ref).max() <= 1e-5 * math.sqrt(w.C_in * w.K / w.groups)
    else:
        rms = math.sqrt(float(np.mean(ref ** 2)))
        assert (np.abs(g - ref) <= 2e-2 * np.maximum(np.abs(ref), rms)).all()


@pytest.mark.parametrize("name,big,small", [
    ("dc1d_layer", 16, 3),      # split reduction: fp32 partial tiles in the scratch
    ("dcnv2_bf16", 4, 1),       # rearranged bf16 weights in the scratch, a mask
    ("long_seq_bf16", 2, 1),    # rearranged bf16 weights, four offset groups
])
def test_noalloc_matches_forward_two_calls(name, big, small):
    w0 = inputs.WORKLOADS[name]
    for B in (big, small):
        w = w0.with_batch(B)
        t, out_na, out = _pair(w)
        assert torch.equal(out_na, out), "%s: dc1d_forward_noalloc differs from dc1d_forward" % w.name
        _oracle_points(w, t, out_na)


def test_noalloc_needs_no_workspace_shapes():
    # the depthwise and direct kernels use no workspace at all
    for name in ("tiny", "depthwise"):
        w = inputs.WORKLOADS[name].with_batch(1)
        t, out_na, out = _pair(w)
        assert torch.equal(out_na, out)


def test_noalloc_rejects_beyond_scratch():
    # 4096 -> 4096 channels, K 3, bf16: the rearranged weights alone exceed the scratch
    B, C, L, K = 1, 4096, 64, 3
    x = torch.zeros((B, C, L), dtype=torch.bfloat16, device=DEV)
    off = torch.zeros((B, 1, L - K + 1, K), dtype=torch.bfloat16, device=DEV)
    wt = torch.zeros((C, C, K), dtype=torch.bfloat16, device=DEV)
    out = torch.zeros((B, C, L - K + 1), dtype=torch.bfloat16, device=DEV)
    need = dc1d.workspace_bytes(x, off, wt)
    assert need > dc1d.noalloc_scratch_bytes()
    with pytest.raises(dc1d.Dc1dValueError) as e:
        dc1d.forward_noalloc(x, off, wt, out=out)
    assert e.value.status == dc1d.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert not out.any()  # nothing was written
