"""Repeatability of every forward kernel at the measured sizes: the same
call five times gives the same bits.

Every forward kernel sums in a fixed order with no atomics (the split
reduction adds the splits in split order), so a difference between runs
would mean a race -- a thread reading a shared-memory tile before its
writer's barrier, a buffer staged while another wave still reads it, a
workspace entry two workgroups both write.  The cases are the measured
workloads in the launch configuration the bench times (each kernel's
real grid, tiles, window sizes and split counts), the wide bf16 kernel's
gathering launch (offsets wider than its windows), the packed layer's head
kernel with its fused trunk, and the 2D path.  Parity with the oracle is
checked elsewhere; this only checks that repeated runs agree.
"""
import pytest
import torch

from deformable_convolution_amd import dc1d, inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
REPEATS = 5


def same_every_time(fn):
    first = fn().clone()
    torch.cuda.synchronize()
    for i in range(1, REPEATS):
        again = fn()
        torch.cuda.synchronize()
        assert torch.equal(first, again), "run %d differs from the first" % i
    return first


def forward_case(w, t):
    g = {k: (v.to(DEV) if v is not None else None) for k, v in t.items()}
    kw = dict(stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)
    print("repeat", w.name, dc1d.plan(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], **kw)["kernel"],
          flush=True)
    return lambda: dc1d.forward(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], **kw)


@pytest.mark.parametrize("name", ["dc1d_layer", "long_seq_bf16", "depthwise", "dcnv2_bf16"])
def test_forward_workloads_repeat_bit_for_bit(name):
    w = inputs.WORKLOADS[name]
    same_every_time(forward_case(w, inputs.make_inputs(w, seed=0)))


def test_wide_kernel_gathered_tiles_repeat_bit_for_bit():
    """Offsets of tens of positions: most of the wide kernel's tiles are
    left to its gathering launch."""
    w = inputs.WORKLOADS["long_seq_bf16"]
    t = inputs.make_inputs(w, seed=1)
    gen = torch.Generator().manual_seed(1)
    t["offsets"] = (torch.randn(t["offsets"].shape, generator=gen) * 40.0).to(t["offsets"].dtype)
    same_every_time(forward_case(w, t))


def test_packed_layer_repeats_bit_for_bit():
    w = inputs.PACKED_WORKLOADS["packed"]
    t = inputs.make_packed_inputs(w, seed=0)
    g = {k: (v.to(DEV) if v is not None else None) for k, v in t.items()}
    kw = dict(stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)

    def run():
        out, (off, mask) = dc1d.packed_forward(g["x"], g["trunk_weight"], g["trunk_bias"], g["off_weight"],
                                               g["off_bias"], g["weight"], g["bias"], g["mask_weight"],
                                               g["mask_bias"], with_offsets=True, **kw)
        return torch.cat([out.flatten(), off.flatten(), mask.flatten()])

    same_every_time(run)


@pytest.mark.parametrize("name", ["dcn2d", "dcn2d_bf16"])
def test_2d_workloads_repeat_bit_for_bit(name):
    w = inputs.WORKLOADS_2D[name]
    t = inputs.make_inputs2d(w, seed=0)
    g = {k: (v.to(DEV) if v is not None else None) for k, v in t.items()}
    kw = dict(stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)
    same_every_time(lambda: dc1d.forward2d(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], **kw))
