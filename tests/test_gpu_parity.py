"""GPU parity: libdc1d (through the C ABI) against the CPU oracle.

Tolerances (float outputs; the oracle is exact up to double rounding):
  * fp32: max |gpu - oracle| <= 1e-5 * sqrt(C_in * K / groups)
  * bf16 (bf16 storage, fp32 accumulation, one RNE rounding of the output):
    |gpu - oracle| <= 2e-2 * max(|oracle|, rms(oracle)) elementwise
Sampling positions (left index, validity bits) must match bit for bit; the
fraction within 2^-24 (it is rounded once in fp32 on the GPU).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from deformable_convolution_amd import dc1d, inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def tol_fp32(w):
    return 1e-5 * math.sqrt(w.C_in * w.K / w.groups)


def to_dev(t):
    return {k: (v.to(DEV) if v is not None else None) for k, v in t.items()}


def gpu_forward(w, g, **kw):
    return dc1d.forward(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], stride=w.stride,
                        padding=w.padding, dilation=w.dilation, groups=w.groups, **kw)


def oracle_forward(w, t):
    return oracle.forward(t["x"], t["offsets"], t["weight"], t["bias"], t["mask"], stride=w.stride,
                          padding=w.padding, dilation=w.dilation, groups=w.groups)


def check(w, got, ref, label=""):
    got = got.double().cpu().numpy() if hasattr(got, "cpu") else got
    assert got.shape == ref.shape
    assert np.isfinite(got).all(), label
    if w.dtype == "f32":
        err = np.abs(got - ref).max() if ref.size else 0.0
        assert err <= tol_fp32(w), "%s %s: max|err| %.3g > %.3g" % (w.name, label, err, tol_fp32(w))
    else:
        rms = math.sqrt(float(np.mean(ref ** 2))) if ref.size else 0.0
        bound = 2e-2 * np.maximum(np.abs(ref), rms)
        bad = np.abs(got - ref) > bound
        assert not bad.any(), "%s %s: %d elements beyond the bf16 bound" % (w.name, label, int(bad.sum()))


def run_case(w, seed=0, **kw):
    print("case", w, "seed", seed, flush=True)
    t = inputs.make_inputs(w, seed=seed)
    g = to_dev(t)
    got = gpu_forward(w, g, **kw)
    torch.cuda.synchronize()
    ref = oracle_forward(w, t)
    check(w, got, ref)
    return t, g, got, ref


# ---- the five workloads at oracle-friendly batch --------------------------

REDUCED = [
    ("tiny", None),
    ("dc1d_layer", 2),
    ("long_seq_bf16", 1),
    ("depthwise", 1),
    ("dcnv2_bf16", 1),
]


@pytest.mark.parametrize("name,B", REDUCED)
def test_workloads_reduced_batch(name, B):
    w = inputs.WORKLOADS[name]
    if B is not None:
        w = w.with_batch(B)
    if name == "long_seq_bf16":
        w = inputs.custom("long_seq_bf16[L=4096]", B=1, C_in=256, C_out=256, L_in=4096, K=3, padding=1, G=4,
                          L_out=4096, dtype="bf16", off_dist=("normal", 0.0, 2.0), w_var=1 / 768, bias="zeros")
    if name == "dcnv2_bf16":
        w = inputs.custom("dcnv2_bf16[L=512]", B=1, C_in=1024, C_out=1024, L_in=512, K=3, stride=2, padding=1,
                          G=8, L_out=256, dtype="bf16", off_dist=("normal", 0.0, 1.5),
                          mask_dist=("sigmoid_normal", 0.0, 1.0), w_var=1 / 3072)
    run_case(w)


# ---- ragged shapes through every kernel -----------------------------------

def _shape_cases():
    cases = []
    # (B, C_in, C_out, L_in, K, s, p, d, groups, G, dtype, mask, off_scale)
    spec = [
        (1, 64, 128, 40, 3, 1, 1, 1, 1, 1, "f32", False, 2.0),      # exact tiles in M
        (3, 33, 70, 57, 5, 2, 3, 2, 1, 3, "f32", True, 6.0),        # ragged M, N, Kred
        (2, 96, 200, 129, 4, 1, 0, 3, 1, 4, "f32", False, 3.0),     # ragged, G*K = 16
        (1, 40, 36, 300, 7, 3, 5, 1, 1, 8, "f32", True, 30.0),      # wide offsets
        (5, 16, 48, 11, 1, 1, 0, 1, 1, 2, "f32", False, 1.5),       # K = 1, short rows
        (2, 512, 64, 64, 16, 1, 0, 3, 1, 1, "f32", False, 1.0),     # long reduction (split path)
        (2, 12, 18, 50, 3, 1, 1, 2, 3, 4, "f32", True, 4.0),        # grouped -> direct
        (2, 24, 24, 100, 5, 1, 2, 2, 24, 24, "f32", True, 4.0),     # depthwise
        (2, 8, 24, 90, 3, 2, 1, 1, 8, 2, "f32", False, 3.0),        # depthwise multiplier 3
        (1, 6, 6, 5000, 3, 1, 1, 1, 6, 6, "f32", False, 2000.0),    # depthwise, offsets too wide for a window
        (2, 64, 96, 77, 3, 1, 1, 1, 1, 2, "bf16", True, 3.0),       # bf16 dense
        (2, 32, 32, 300, 5, 1, 2, 2, 32, 32, "bf16", False, 4.0),   # bf16 depthwise
        (1, 64, 80, 400, 6, 1, 0, 8, 1, 1, "f32", False, 5.0),      # channel blocks of 16 (wide window)
        (2, 30, 64, 90, 3, 1, 1, 1, 1, 3, "bf16", True, 2.0),       # bf16, ci-major order (10 ch / group)
        (2, 36, 64, 90, 3, 1, 1, 1, 1, 3, "bf16", True, 2.0),       # bf16 channel blocks of 8 (12 ch / group)
        (1, 48, 40, 700, 5, 1, 2, 1, 1, 6, "bf16", False, 3.0),     # bf16 channel blocks of 16
        (3, 100, 72, 150, 3, 2, 1, 1, 1, 1, "f32", True, 2.5),      # C_in not a multiple of the block
        (1, 64, 64, 600, 3, 1, 1, 1, 1, 1, "f32", False, 2.0),      # f32 K=3, long rows
        # rows staged in 16-byte words (L_in a multiple of the word): tiles over
        # several batches, ragged channel blocks, windows past both ends
        (3, 40, 64, 96, 3, 1, 1, 1, 1, 1, "bf16", True, 5.0),       # bf16 blocks of 16, 40 channels
        (2, 64, 96, 1024, 3, 2, 1, 1, 1, 2, "bf16", True, 8.0),     # bf16 stride 2, two-slot window
        (4, 24, 40, 52, 4, 1, 2, 2, 1, 1, "f32", False, 6.0),       # f32, 50 columns per batch
        # bf16 blocks of 32 channels with position-major windows
        (3, 64, 96, 96, 3, 1, 1, 1, 1, 2, "bf16", True, 5.0),       # tiles over three batches
        (2, 96, 64, 256, 2, 1, 0, 1, 1, 1, "bf16", False, 3.0),     # two chunks per block (K = 2)
        (1, 512, 64, 64, 3, 1, 0, 1, 1, 1, "bf16", True, 2.0),      # split reduction, ranges start mid-block
        (1, 64, 64, 2048, 3, 1, 1, 1, 1, 2, "bf16", False, 200.0),  # offsets too wide: gathered tiles
        (2, 80, 64, 160, 3, 1, 1, 1, 1, 5, "bf16", True, 3.0),      # a partial last block (80 channels)
        (2, 64, 64, 800, 5, 2, 2, 2, 1, 1, "bf16", False, 6.0),     # stride 2, dilation 2: wider window
    ]
    for i, (B, C_in, C_out, L_in, K, s, p, d, groups, G, dt, mask, sc) in enumerate(spec):
        L_out = oracle.output_length(L_in, K, s, p, d)
        cases.append(inputs.custom("shape%d" % i, B=B, C_in=C_in, C_out=C_out, L_in=L_in, K=K, stride=s,
                                   padding=p, dilation=d, groups=groups, G=G, L_out=L_out, dtype=dt,
                                   off_dist=("uniform", -sc, sc),
                                   mask_dist=("sigmoid_normal", 0.0, 1.0) if mask else None))
    return cases


@pytest.mark.parametrize("w", _shape_cases(), ids=lambda w: w.name)
def test_ragged_shapes(w):
    run_case(w, seed=3)


def test_ragged_shapes_reach_every_kernel():
    """The shapes above run every kernel family and staging order."""
    names = set()
    for w in _shape_cases():
        g = to_dev(inputs.make_inputs(w, seed=3))
        pl = dc1d.plan(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], stride=w.stride,
                       padding=w.padding, dilation=w.dilation, groups=w.groups)
        names.add(pl["kernel"])
    # (fp32 blocks of 32 channels need more LDS than a workgroup has next to
    # the fp32 weight and sample tiles, so the planner never picks them)
    want = {"direct", "depthwise", "mfma_f32", "mfma_bf16", "mfma_f32_cb8", "mfma_f32_cb16", "mfma_bf16_cb8",
            "mfma_bf16_cb16", "mfma_bf16_cb32", "mfma_bf16_cb32t"}
    assert want <= names, sorted(want - names)


# ---- the one-wave-per-SIMD bf16 kernel (256 x 256 tiles) -------------------
#
# Planned for bf16 blocks of 32 channels when its tiles alone fill the GPU,
# so these shapes have about 65536 columns and 200 - 256 output channels.

def _wide_cases():
    # (B, C_in, C_out, L_in, K, s, p, d, G, mask, off_scale)
    spec = [
        (4, 160, 256, 16384, 3, 1, 1, 1, 5, False, 3.0),   # K odd, five blocks: a padding block
        (2, 176, 200, 32768, 3, 1, 1, 2, 11, True, 4.0),   # partial last block, ragged rows, L_out % 4 != 0
        (300, 64, 256, 256, 2, 1, 0, 1, 2, True, 2.0),     # K = 2, tiles over two or three batches
        (512, 160, 256, 128, 3, 1, 1, 1, 5, False, 3.0),   # 128 columns per batch, padding block
        (4, 128, 256, 32768, 4, 2, 1, 1, 4, True, 5.0),    # K = 4, stride 2 (wider window)
        (2, 64, 256, 32768, 3, 1, 1, 1, 2, False, 300.0),  # offsets too wide for any window: all gathered
        (520, 32, 256, 136, 2, 1, 0, 1, 1, True, 2.0),     # one block, 135 columns per batch
    ]
    cases = []
    for i, (B, C_in, C_out, L_in, K, s, p, d, G, mask, sc) in enumerate(spec):
        L_out = oracle.output_length(L_in, K, s, p, d)
        cases.append(inputs.custom("wide%d" % i, B=B, C_in=C_in, C_out=C_out, L_in=L_in, K=K, stride=s,
                                   padding=p, dilation=d, G=G, L_out=L_out, dtype="bf16",
                                   off_dist=("uniform", -sc, sc),
                                   mask_dist=("sigmoid_normal", 0.0, 1.0) if mask else None))
    return cases


def _plan_of(w, g):
    return dc1d.plan(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], stride=w.stride, padding=w.padding,
                     dilation=w.dilation, groups=w.groups)


def _wide_device():
    return torch.cuda.get_device_properties(DEV).multi_processor_count <= 256


@pytest.mark.parametrize("w", _wide_cases(), ids=lambda w: w.name)
def test_wide_kernel(w):
    t = inputs.make_inputs(w, seed=9)
    g = to_dev(t)
    pl = _plan_of(w, g)
    print("plan", pl, flush=True)
    if _wide_device():
        assert pl["kernel"] == "mfma_bf16_wide" and pl["splits"] == 1, pl
    got = gpu_forward(w, g)
    torch.cuda.synchronize()
    check(w, got, oracle_forward(w, t))


def test_wide_kernel_some_tiles_gathered():
    """A few offsets far out: the tiles holding them are gathered by the
    second launch, every other tile is windowed; all match the oracle."""
    w = _wide_cases()[0]
    t = inputs.make_inputs(w, seed=10)
    off = t["offsets"].float()
    for (b, g_, l, k, v) in [(0, 0, 1000, 1, 700.0), (1, 2, 5000, 0, -900.0), (3, 1, 16383, 2, 2000.0),
                             (2, 0, 0, 0, -3000.0)]:
        off[b, g_, l, k] = v
    t["offsets"] = off.to(t["offsets"].dtype)
    g = to_dev(t)
    if _wide_device():
        assert _plan_of(w, g)["kernel"] == "mfma_bf16_wide"
    got = gpu_forward(w, g)
    torch.cuda.synchronize()
    check(w, got, oracle_forward(w, t))


def test_wide_kernel_misaligned_x_takes_the_channel_block_kernel():
    """x not 16-byte aligned: the channel-block kernel runs instead (on its
    own grid, with its own workspace layout); both match the oracle."""
    w = _wide_cases()[0]
    t = inputs.make_inputs(w, seed=12)
    g = to_dev(t)
    if _wide_device():
        assert _plan_of(w, g)["kernel"] == "mfma_bf16_wide"
    a = gpu_forward(w, g)
    b = gpu_forward(w, dict(g, x=_misaligned_copy(g["x"])))
    torch.cuda.synchronize()
    ref = oracle_forward(w, t)
    check(w, a, ref, "wide")
    check(w, b, ref, "channel blocks")


def test_weights_read_in_place_or_rearranged():
    """fp32 blocks of 8 channels x 4 taps read the weights in place when they
    are 16-byte aligned and from a rearranged copy otherwise; same results."""
    w = inputs.custom("cb8", B=2, C_in=64, C_out=96, L_in=128, K=16, dilation=3, L_out=83,
                      off_dist=("normal", 0.0, 1.0))
    t = inputs.make_inputs(w, seed=5)
    g = to_dev(t)
    assert dc1d.plan(g["x"], g["offsets"], g["weight"], g["bias"], None, dilation=3)["kernel"] == "mfma_f32_cb8"
    ref = oracle_forward(w, t)
    check(w, gpu_forward(w, g), ref, "aligned weights")
    buf = torch.empty(g["weight"].numel() + 1, dtype=torch.float32, device=DEV)
    wv = buf[1:].view(g["weight"].shape)
    wv.copy_(g["weight"])
    assert wv.data_ptr() % 16 != 0
    check(w, gpu_forward(w, dict(g, weight=wv)), ref, "misaligned weights")


def _misaligned_copy(t):
    """The same values at a device address that is not 16-byte aligned."""
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=DEV)
    v = buf[1:].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 != 0
    return v


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unaligned_input_and_output_take_the_element_paths(dtype):
    """x rows are staged in 16-byte words and the output written in 16-byte
    words only when the pointers allow; a misaligned x (element staging) and
    a misaligned output (element stores) give the same bits."""
    # enough column tiles to fill the GPU without a split reduction (the
    # direct epilogue)
    w = inputs.custom("align_" + dtype, B=4, C_in=64, C_out=96, L_in=8192, K=3, padding=1, G=2, L_out=8192,
                      dtype=dtype, off_dist=("uniform", -5.0, 5.0), mask_dist=("sigmoid_normal", 0.0, 1.0))
    t = inputs.make_inputs(w, seed=8)
    g = to_dev(t)
    kw = dict(stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)
    pl = dc1d.plan(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], **kw)
    assert pl["kernel"].startswith("mfma_") and pl["splits"] == 1, pl
    ref = oracle_forward(w, t)
    a = gpu_forward(w, g)
    xm = _misaligned_copy(g["x"])
    b = gpu_forward(w, dict(g, x=xm))
    om = _misaligned_copy(torch.zeros_like(a))
    dc1d.forward(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], out=om, **kw)
    torch.cuda.synchronize()
    check(w, a, ref, "aligned")
    assert torch.equal(a, b), "misaligned x"
    assert torch.equal(a, om), "misaligned out"


# ---- positions: bit-exact ---------------------------------------------------

def _adversarial_offsets(shape, seed):
    rng = np.random.default_rng(seed)
    vals = np.array([0.0, -0.0, 1.0, -1.0, 2.0 ** -20, -2.0 ** -20, -2.0 ** -24, 1 - 2.0 ** -24,
                     -(1 - 2.0 ** -24), 0.5, -0.5, 3.75, -3.75, 1e6, -1e6, 3e8, -3e8, 1e9, -1e9,
                     16383.999, -16384.25], dtype=np.float32)
    a = rng.choice(vals, size=shape).astype(np.float32)
    a += (rng.standard_normal(shape) * (rng.uniform(size=shape) < 0.3)).astype(np.float32)
    return torch.from_numpy(a)


@pytest.mark.parametrize("name", inputs.WORKLOAD_ORDER)
def test_positions_bit_exact(name):
    w = inputs.WORKLOADS[name]
    B = 1 if name != "tiny" else 1
    G = min(w.G, 8)
    shape = (B, G, w.L_out, w.K)
    for src in ("workload", "adversarial"):
        if src == "workload":
            off = inputs.make_inputs(w.with_batch(1), seed=1)["offsets"][:, :G].contiguous()
        else:
            off = _adversarial_offsets(shape, seed=5).to(inputs.torch_dtype(w.dtype))
        i0, fr, va = dc1d.debug_positions(off.to(DEV), w.L_in, w.stride, w.padding, w.dilation)
        torch.cuda.synchronize()
        ri0, rfr, rva = oracle.positions(off, w.L_in, w.K, w.stride, w.padding, w.dilation)
        big = np.abs(off.double().numpy()) >= 2.0 ** 29   # clamped offsets: only in-range positions are defined
        ok = ~big
        assert np.array_equal(i0.cpu().numpy()[ok], ri0[ok]), (name, src)
        assert np.array_equal(va.cpu().numpy(), rva), (name, src)
        assert np.abs(fr.cpu().double().numpy()[ok] - rfr[ok]).max() <= 2.0 ** -24, (name, src)


# ---- invariants on the GPU ------------------------------------------------------

@pytest.mark.parametrize("name", ["dc1d_layer", "shape1", "depthwise"])
def test_mask_ones_bit_identical(name):
    """dc1d page, Modulation: an all-ones mask is bit-for-bit identical to no mask."""
    if name == "dc1d_layer":
        w = inputs.WORKLOADS[name].with_batch(2)
    elif name == "depthwise":
        w = inputs.WORKLOADS[name].with_batch(1)
    else:
        w = _shape_cases()[1]
    t = to_dev(inputs.make_inputs(w, seed=4))
    none = dc1d.forward(t["x"], t["offsets"], t["weight"], t["bias"], None, stride=w.stride,
                        padding=w.padding, dilation=w.dilation, groups=w.groups)
    ones = dc1d.forward(t["x"], t["offsets"], t["weight"], t["bias"], torch.ones_like(t["offsets"]),
                        stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)
    zero = dc1d.forward(t["x"], t["offsets"], t["weight"], t["bias"], torch.zeros_like(t["offsets"]),
                        stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)
    torch.cuda.synchronize()
    assert torch.equal(none, ones)
    assert torch.equal(zero, t["bias"][None, :, None].expand_as(zero))


def test_zero_and_integer_offsets_match_conv1d():
    """Zero offsets reproduce conv1d; integer offsets shift exactly (dc1d
    page, Demo notebook), on the dense MFMA path."""
    w = inputs.WORKLOADS["dc1d_layer"].with_batch(2)
    t = inputs.make_inputs(w, seed=6)
    for delta in (0.0, 1.0, -3.0):
        t["offsets"] = torch.full_like(t["offsets"], delta)
        g = to_dev(t)
        got = gpu_forward(w, g)
        torch.cuda.synchronize()
        check(w, got, oracle_forward(w, t), "delta=%g" % delta)


def test_split_reduction_deterministic_and_reusable():
    """The split-reduction path gives bit-identical results call after call
    (its per-tile counters return to zero) and matches the oracle."""
    w = inputs.WORKLOADS["dc1d_layer"]
    t = inputs.make_inputs(w.with_batch(2), seed=8)
    g = to_dev(t)
    info = dc1d.plan(g["x"], g["offsets"], g["weight"], g["bias"], None, dilation=w.dilation)
    print("plan", info, flush=True)
    first = gpu_forward(w, g)
    for _ in range(5):
        again = gpu_forward(w, g)
    torch.cuda.synchronize()
    assert torch.equal(first, again)
    check(w.with_batch(2), first, oracle_forward(w, t))


def test_empty_batch():
    w = inputs.WORKLOADS["tiny"].with_batch(0)
    t = to_dev(inputs.make_inputs(w))
    out = gpu_forward(w, t)
    torch.cuda.synchronize()
    assert out.shape == (0, w.C_out, w.L_out)


def test_offsets_far_outside_give_bias():
    w = inputs.WORKLOADS["dc1d_layer"].with_batch(1)
    t = to_dev(inputs.make_inputs(w, seed=2))
    t["offsets"] = torch.full_like(t["offsets"], 1e9)
    out = gpu_forward(w, t)
    torch.cuda.synchronize()
    assert torch.equal(out, t["bias"][None, :, None].expand_as(out))


def test_workspace_too_small_is_rejected():
    w = inputs.WORKLOADS["dc1d_layer"].with_batch(2)
    t = to_dev(inputs.make_inputs(w))
    need = dc1d.workspace_bytes(t["x"], t["offsets"], t["weight"], t["bias"], None, dilation=w.dilation)
    if need == 0:
        pytest.skip("no workspace needed for this shape on this device")
    small = torch.zeros(need - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        gpu_forward(w, t, workspace=small)
    # big enough but not 256-byte aligned
    big = torch.zeros(need + 512, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        gpu_forward(w, t, workspace=big[16:])
    out = gpu_forward(w, t, workspace=big[256:])
    torch.cuda.synchronize()
    check(w, out, oracle_forward(w, inputs.make_inputs(w)))


# ---- full sizes, sampled outputs -------------------------------------------

@pytest.mark.parametrize("name", ["dc1d_layer", "long_seq_bf16", "depthwise", "dcnv2_bf16"])
def test_full_size_sampled(name):
    """Each workload at its full size, in the launch configuration the bench
    times, checked at 4096 sampled outputs the oracle computes one by one."""
    w = inputs.WORKLOADS[name]
    print("full", w, flush=True)
    t = inputs.make_inputs(w, seed=0)
    g = to_dev(t)
    got = gpu_forward(w, g)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    n = 4096
    pts = np.stack([rng.integers(0, w.B, n), rng.integers(0, w.C_out, n), rng.integers(0, w.L_out, n)], 1)
    # always include the corners (ragged tails of every tile dimension)
    corners = np.array([[0, 0, 0], [w.B - 1, w.C_out - 1, w.L_out - 1], [0, w.C_out - 1, 0],
                        [w.B - 1, 0, w.L_out - 1]])
    pts = np.concatenate([pts, corners])
    ref = oracle.forward_points(t["x"], t["offsets"], t["weight"], pts, t["bias"], t["mask"],
                                stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)
    gv = got[pts[:, 0], pts[:, 1], pts[:, 2]].double().cpu().numpy()
    if w.dtype == "f32":
        err = np.abs(gv - ref).max()
        assert err <= tol_fp32(w), "%s: max|err| %.3g" % (name, err)
    else:
        rms = math.sqrt(float(np.mean(ref ** 2)))
        assert (np.abs(gv - ref) <= 2e-2 * np.maximum(np.abs(ref), rms)).all()
    assert torch.isfinite(got).all()


@pytest.mark.parametrize("name", ["dc1d_layer", "dcnv2_bf16", "depthwise"])
def test_kernel_events_bracket_the_dominant_kernel(name):
    """dc1d_set_kernel_events: the events a forward records around its
    dominant kernel lie inside the call and change no result."""
    w = inputs.WORKLOADS[name].with_batch(2)
    g = to_dev(inputs.make_inputs(w, seed=2))
    ref = gpu_forward(w, g)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    dc1d.set_kernel_events(ev[1], ev[2])
    try:
        ev[0].record()
        out = gpu_forward(w, g)
        ev[3].record()
    finally:
        dc1d.set_kernel_events(None, None)
    torch.cuda.synchronize()
    kernel, call = ev[1].elapsed_time(ev[2]), ev[0].elapsed_time(ev[3])
    assert 0.0 < kernel <= call, (kernel, call)
    assert torch.equal(out, ref)
