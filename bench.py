"""Benchmark of the DeformConv1d forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--only]

One step is one forward (the whole hot path: position split, interpolation,
modulation, contraction, bias) over one batch of seeded synthetic inputs
that are already resident in device memory.  The default workload is the
dc1d page's layer shape (B16, C512 -> 512, K16, dilation 3, "valid", L128,
fp32).  Prints ONE JSON line (rank 0, one GPU):

  value      contraction + sampling GFLOP per step / seconds per step
  roofline   the dominant kernel's achieved rate against its roofline peak:
             algorithmic flops (MFMA-bound) or bytes (HBM-bound) of one
             launch over that kernel's mean duration, from HIP events the
             library records on the launch stream right before and after
             its launch (kernel_ms); call_ms is the whole forward call
             (the small kernels it also enqueues included)
  cpu_baseline  the CPU oracle timed on the host cores (reported baseline)

Parity is checked in the same run: every output of the GPU's forward
against the oracle's (the CPU baseline's own last run); a mismatch aborts
the bench.  Unless --only is given, each of the other named workloads is
also timed and checked (every output against the oracle) and written as one
JSON record to stderr, before the headline line.
--profile-run runs only the warmup + timed launches (no oracle, no JSON),
for rocprofv3; --copy-calibration MB runs one device-to-device copy of that
size (the reference kernel for scaling the HBM byte counters).
--backward times the backward (all five gradients, fp32 workloads) the
same way, with the oracle's backward as parity check and CPU baseline.
--summarize-profile DIR --kernel NAME folds the rocprofv3 output of the
commands listed in PROFILE_COMMANDS (kernel trace, FETCH_SIZE / WRITE_SIZE
passes, copy calibration) into profiles/<workload>__<kernel>.md; the bench
reads the HBM traffic per launch from there while the kernel sources are
unchanged.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DeformConv1d fwd GFLOP/s + % MFMA/HBM roofline (B16 C512 K16 d3 L128)"
PEAK = {  # MI355X published peaks
    "hbm_GBps": 8000.0,
    "mfma_f32_TFLOPs": 157.3,
    "mfma_bf16_TFLOPs": 2516.6,
    "valu_f32_TFLOPs": 157.3,
}
CSRC = "deformable_convolution_amd/csrc"
KERNEL_SOURCES = sorted(os.path.join(CSRC, f) for f in os.listdir(os.path.join(ROOT, CSRC))
                        if f.endswith((".hip", ".h")))


def work(w):
    """Algorithmic work of one forward: contraction flops, sampling flops
    (3 per sample: weight, interpolate; 4 with the mask), bytes moved once."""
    contraction = 2 * w.B * w.C_out * w.L_out * (w.C_in // w.groups) * w.K
    sampling = (4 if w.mask_dist else 3) * w.B * w.C_in * w.L_out * w.K
    es = 4 if w.dtype == "f32" else 2
    n_off = w.B * w.G * w.L_out * w.K
    elems = (w.B * w.C_in * w.L_in + n_off * (2 if w.mask_dist else 1) + w.C_out * (w.C_in // w.groups) * w.K
             + (w.C_out if w.bias is not None else 0) + w.B * w.C_out * w.L_out)
    return contraction, sampling, elems * es


# The sources each measured kernel family is built from (a summary's counters
# stay valid while these are unchanged).  Every family includes the shared
# header and the C ABI's launch code.
_COMMON = ["dc1d_internal.h", "api.hip"]
_MFMA = ["mfma_kernel.h", "k_mfma.hip", "k_mfma_f32.hip", "k_mfma_f32_mask.hip", "k_mfma_bf16.hip",
         "k_mfma_bf16_mask.hip"]
_WIDE = ["mfma_wide.h", "k_mfma_wide.hip"]  # the one-wave-per-SIMD bf16 kernel (includes mfma_kernel.h)
_FAMILY_SOURCES = [
    ("mfma_bf16_wide", _MFMA + _WIDE),
    ("mfma_", _MFMA),
    ("depthwise", ["k_direct.hip"]),
    ("direct2d", ["k_dc2d.hip"]),
    ("direct", ["k_direct.hip"]),
    ("backward", ["k_backward.hip"] + _MFMA),
    ("packed", ["k_packed.hip", "k_heads.hip", "k_direct.hip"] + _MFMA),
    ("im2col2d", ["k_dc2d.hip"] + _MFMA),
]


def kernel_sources(kernel=None):
    """The source files behind `kernel` (all of them when it is unknown)."""
    for prefix, files in _FAMILY_SOURCES:
        if kernel is not None and kernel.startswith(prefix):
            return sorted(os.path.join(CSRC, f) for f in set(files + _COMMON))
    return KERNEL_SOURCES


def kernel_hash(kernel=None):
    h = hashlib.sha256()
    for f in kernel_sources(kernel):
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def workload_label(w):
    return "%s B%d Cin%d Cout%d L%d K%d s%d p%d d%d groups%d G%d%s %s" % (
        w.name, w.B, w.C_in, w.C_out, w.L_in, w.K, w.stride, w.padding, w.dilation, w.groups, w.G,
        " mask" if w.mask_dist else "", w.dtype)


def read_traffic(name, kernel, khash):
    """HBM bytes per launch of `kernel` on workload `name` from the committed
    counter summary, or None if absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "%s__%s.md" % (name, kernel))
    if not os.path.exists(path):
        return None
    meta = {}
    for line in open(path):
        if line.startswith("<!-- ") and "=" in line:
            k, v = line[5:].split("-->")[0].strip().split("=", 1)
            meta[k.strip()] = v.strip()
    if meta.get("kernel_sources") != khash or meta.get("kernel") != kernel:
        return None
    try:
        return float(meta["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def timed(step, steps, warmup, dev, graph=False):
    """Run `warmup` untimed steps (then more, untimed, until 0.2 s have
    passed), then time `steps` of them on the launch stream, twice: step by
    step (an event between consecutive steps, for the
    spread of single steps), then the region (one HIP event on the stream
    before the first step and one after the last, synchronised on both
    sides; the figure the bench reports).  With graph=True the step is also captured
    once into a HIP graph (torch.cuda.CUDAGraph) and the step-by-step
    figures are its replays."""
    import torch

    stream = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        step()
    # and until the GPU has been busy for a while (its clocks ramp up under
    # load; a few warm-up steps of a fraction of a millisecond do not)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.2:
        for _ in range(10):
            step()
        torch.cuda.synchronize()

    def region(run):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(steps):
            run()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    def chain(run):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        for i in range(steps):
            ev[i].record(stream)
            run()
        ev[steps].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[steps]), [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]

    _, eager_ms = chain(step)
    region_ms = region(step)
    if not graph:
        return {"region_ms": region_ms, "launch_ms": eager_ms, "eager_ms": eager_ms, "graph": False}
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step()
    stream.wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    region, launch = chain(g.replay)
    return {"region_ms": region, "launch_ms": launch, "eager_ms": eager_ms, "graph": True}


def kernel_times(step, steps, dev):
    """The dominant kernel's duration (ms) in each of `steps` steps, from HIP
    events that the library records on the launch stream right before and
    right after that kernel's launch (dc1d_set_kernel_events): the fused
    sampling + MFMA kernel without the weight rearrangement before it and
    the split reduction after it, or the depthwise / direct kernel."""
    import torch
    from deformable_convolution_amd import dc1d

    stream = torch.cuda.current_stream(dev)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    for e in evs:
        e.record(stream)  # creates the HIP events
    torch.cuda.synchronize()
    try:
        for i in range(steps):
            dc1d.set_kernel_events(evs[2 * i], evs[2 * i + 1])
            step()
    finally:
        dc1d.set_kernel_events(None, None)
    torch.cuda.synchronize()
    return [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(steps)]


def parity_of(w, got, ref):
    """Elementwise comparison of GPU outputs with the oracle's (float64
    arrays of the same elements): fp32 max|err| <= 1e-5 sqrt(C_in K / groups);
    bf16 |err| <= 2e-2 max(|ref|, rms(ref)) elementwise."""
    n = int(ref.size)
    if w.dtype == "f32":
        err = float(np.abs(got - ref).max())
        tol = 1e-5 * math.sqrt(w.C_in * w.K / w.groups)
        return {"elements": n, "max_err": err, "tol": tol, "ok": bool(err <= tol)}
    rms = math.sqrt(float(np.mean(ref ** 2)))
    worst = float((np.abs(got - ref) / (2e-2 * np.maximum(np.abs(ref), rms))).max())
    return {"elements": n, "max_err_over_tol": worst, "tol": "2e-2*max(|ref|, rms(ref)) elementwise",
            "ok": bool(worst <= 1.0)}


def run_gpu(w, steps, warmup, cold_reps=0, constrained=False, t=None):
    """Time the forward on the GPU.  Returns the plan, the timings and the
    output of the first (untimed) call, for the parity check."""
    import torch
    from deformable_convolution_amd import dc1d, inputs

    dev = torch.device("cuda:0")
    if t is None:
        t = inputs.make_inputs(w, seed=0)
    g = {k: (v.to(dev) if v is not None else None) for k, v in t.items()}
    kw = dict(stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)
    plan = dc1d.plan(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], **kw)
    out = torch.empty((w.B, w.C_out, w.L_out), dtype=g["x"].dtype, device=dev)
    nws = dc1d.workspace_bytes(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], **kw)
    ws = torch.zeros(max(nws, 1), dtype=torch.uint8, device=dev) if nws else None

    def step():
        dc1d.forward(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], out=out, workspace=ws,
                     constrained=constrained, **kw)

    step()
    torch.cuda.synchronize()
    first = out.clone()
    # The timed region: one HIP event on the launch stream before each
    # forward and one after the last; forward i lasts ev[i] -> ev[i+1] (its
    # kernels run back to back on that stream), the region ev[0] -> ev[steps].
    tm = timed(step, steps, warmup, dev)
    kern = kernel_times(step, steps, dev)
    stream = torch.cuda.current_stream(dev)
    cold_ms = []
    if cold_reps:
        # cold: a 512 MiB write (twice the last-level cache) before each
        # forward, outside its events
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(cold_reps):
            flush.fill_(1)
            a.record(stream)
            step()
            b.record(stream)
            torch.cuda.synchronize()
            cold_ms.append(a.elapsed_time(b))
        del flush
    return {"plan": plan, "region_ms": tm["region_ms"], "launch_ms": tm["launch_ms"], "kernel_ms": kern,
            "cold_ms": cold_ms, "eager_ms": tm["eager_ms"], "graph": tm["graph"], "out": first}


def roofline_of(w, kern, kernel_ms, call_ms, constrained=False):
    """The roofline object for a forward: algorithmic work of one launch over
    the dominant kernel's mean duration (events around its launch), against
    its peak (MFMA for the fused kernels, HBM otherwise)."""
    contraction, _, nbytes = work(w)
    if kern.startswith("mfma"):
        peak = PEAK["mfma_f32_TFLOPs"] if w.dtype == "f32" else PEAK["mfma_bf16_TFLOPs"]
        achieved = contraction / (kernel_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4)}
    else:
        achieved = nbytes / (kernel_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK["hbm_GBps"], "unit": "GB/s",
                "frac": round(achieved / PEAK["hbm_GBps"], 4)}
    roof["traffic"] = read_traffic(w.name, kern + ("_constrained" if constrained else ""), kernel_hash(kern))
    roof["kernel"] = kern
    roof["kernel_ms"] = round(kernel_ms, 5)  # the dominant kernel alone (events around its launch)
    roof["call_ms"] = round(call_ms, 5)      # the whole forward call (every kernel it enqueues)
    return roof


def oracle_reference(w, t, constrained=False):
    """Every output of the workload from the oracle, and the seconds it took."""
    import oracle

    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    kw = dict(stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)
    t0 = time.perf_counter()
    ref = oracle.forward(t["x"], t["offsets"], t["weight"], t["bias"], t["mask"], constrained=constrained, **kw)
    return ref, time.perf_counter() - t0


def workload_line(w, steps, warmup):
    """One stderr record: a workload's timing, roofline and full-output parity
    against the oracle."""
    from deformable_convolution_amd import inputs

    t = inputs.make_inputs(w, seed=0)
    r = run_gpu(w, steps, warmup, t=t)
    ref, el = oracle_reference(w, t)
    parity = parity_of(w, r["out"].double().cpu().numpy(), ref)
    if not parity["ok"]:
        raise SystemExit("bench parity check failed for %s: %r" % (w.name, parity))
    contraction, sampling, nbytes = work(w)
    ms = r["region_ms"] / steps
    kern = r["plan"]["kernel"]
    return {"workload": workload_label(w), "kernel": kern, "plan": r["plan"], "steps": steps,
            "ms_per_step": round(ms, 5), "GFLOP/s": round((contraction + sampling) / (ms * 1e-3) / 1e9, 1),
            "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1), "parity": parity,
            "roofline": roofline_of(w, kern, float(np.mean(r["kernel_ms"])), float(np.mean(r["launch_ms"]))),
            "oracle_s": round(el, 2)}


def work_backward(w):
    """Algorithmic work of one backward (all five gradients): the two
    contractions (dS = W^T dout and grad_W = dout S^T, each as many flops as
    the forward's), sampling and scattering (7 flops per sample: the sample,
    dS times the two lerp weights and the two offset/mask terms), and the
    bytes of every input read once and every gradient written once."""
    contraction, _, _ = work(w)
    samples = w.B * w.C_in * w.L_out * w.K
    n_off = w.B * w.G * w.L_out * w.K
    elems_in = (w.B * w.C_in * w.L_in + n_off * (2 if w.mask_dist else 1) + w.C_out * (w.C_in // w.groups) * w.K
                + w.B * w.C_out * w.L_out)
    elems_out = (w.B * w.C_in * w.L_in + n_off * (2 if w.mask_dist else 1) + w.C_out * (w.C_in // w.groups) * w.K
                 + w.C_out)
    return 2 * contraction, 7 * samples, 4 * (elems_in + elems_out)


def run_backward(w, steps, warmup, check=True, baseline=True):
    """Time the backward (every gradient) on the GPU; check it against the
    oracle's backward, whose run is also the CPU baseline."""
    import torch
    from deformable_convolution_amd import dc1d, inputs

    dev = torch.device("cuda:0")
    t = inputs.make_inputs(w, seed=0)
    gen = torch.Generator().manual_seed(1000)
    dout = torch.randn((w.B, w.C_out, w.L_out), generator=gen, dtype=torch.float32)
    if w.dtype == "bf16":
        dout = dout.to(torch.bfloat16)
    g = {k: (v.to(dev) if v is not None else None) for k, v in t.items()}
    gd = dout.to(dev)
    kw = dict(stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)

    nws = dc1d.backward_workspace_bytes(g["x"], g["offsets"], g["weight"], gd, g["mask"], **kw)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev) if nws else None

    def step():
        return dc1d.backward(g["x"], g["offsets"], g["weight"], gd, g["mask"], workspace=ws, **kw)

    got = step()
    torch.cuda.synchronize()
    parity, cpu = None, None
    if check or baseline:
        import oracle
        cores = len(os.sched_getaffinity(0))
        os.environ.setdefault("OMP_NUM_THREADS", str(cores))
        t0 = time.perf_counter()
        ref = oracle.backward(t["x"], t["offsets"], t["weight"], dout, t["mask"], **kw)
        el = time.perf_counter() - t0
        c2, s2, _ = work_backward(w)
        cpu = {"value": (c2 + s2) / el / 1e9, "unit": "GFLOP/s", "cores": min(int(os.environ["OMP_NUM_THREADS"]),
                                                                             cores),
               "kind": "oracle", "sample": "1 full backward (all five gradients) of the same workload, %.1f s, on %s"
               % (el, cpu_model())}
        opg, cpo = w.C_out // w.groups, w.C_in // w.G
        n = {"x": opg * w.K * 2, "offsets": cpo * opg, "mask": cpo * opg, "weight": w.B * w.L_out,
             "bias": w.B * w.L_out}
        worst = 0.0
        for k, r in ref.items():
            if r is None:
                continue
            a = got[k].double().cpu().numpy()
            if not r.size:
                continue
            rms = math.sqrt(float(np.mean(r ** 2)))
            if w.dtype == "f32":
                worst = max(worst, float(np.abs(a - r).max()) / (1e-5 * math.sqrt(n[k]) * rms + 1e-6))
            else:  # bf16 gradients: elementwise 2e-2 max(|ref|, rms(ref))
                worst = max(worst, float((np.abs(a - r) / (2e-2 * np.maximum(np.abs(r), rms) + 1e-30)).max()))
        parity = {"gradients": sorted(k for k, r in ref.items() if r is not None), "max_err_over_tol": worst,
                  "ok": bool(worst <= 1.0)}
        if not parity["ok"]:
            raise SystemExit("backward parity check failed: %r" % parity)
    tm = timed(step, steps, warmup, dev)
    return {"region_ms": tm["region_ms"], "launch_ms": tm["launch_ms"], "eager_ms": tm["eager_ms"],
            "graph": tm["graph"], "parity": parity, "cpu": cpu}


def main_backward(args, w, stream=None):
    r = run_backward(w, args.steps, args.warmup, baseline=not args.no_cpu_baseline)
    contraction, sampling, nbytes = work_backward(w)
    ms = r["region_ms"] / args.steps
    kern_ms = float(np.mean(r["launch_ms"]))  # per-launch events, as the kernel trace sees them
    if w.groups == 1:
        # (bf16 storage runs the fp32 kernels on widened copies: fp32 MFMA)
        achieved = contraction / (kern_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK["mfma_f32_TFLOPs"], "unit": "TFLOP/s",
                "frac": round(achieved / PEAK["mfma_f32_TFLOPs"], 4)}
    else:
        achieved = nbytes / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK["hbm_GBps"], "unit": "GB/s",
                "frac": round(achieved / PEAK["hbm_GBps"], 4)}
    roof["traffic"] = read_traffic(w.name, "backward", kernel_hash("backward"))
    roof["kernel"] = "backward"  # the whole backward call (all its kernels)
    roof["call_ms"] = round(kern_ms, 5)
    line = {
        "metric": "DeformConv1d bwd GFLOP/s (all five gradients)",
        "value": round((contraction + sampling) / (ms * 1e-3) / 1e9, 1),
        "unit": "GFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic, seeded (deformable_convolution_amd/inputs.py; no dataset)",
        "config": {"workload": workload_label(w), "pass": "backward", "gb_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                   "parity": r["parity"], "timing": "graph replay" if r["graph"] else "eager",
                   "forward_ms": {"warm": pct(r["launch_ms"]), "eager": pct(r["eager_ms"])}},
        "roofline": roof,
    }
    if r["cpu"] is not None:
        line["cpu_baseline"] = r["cpu"]
    print(json.dumps(line), file=stream or sys.stdout, flush=True)


def work_packed(w):
    """Work of one packed-layer forward: flops of the trunk, the heads and the
    forward's contraction and sampling; the bytes each of its kernels reads
    and writes once, and the layer's compulsory bytes (x, parameters, out).
    Kernels: where the head kernel computes the trunk itself (K <= 4,
    C_in <= 64, G*K*heads <= 128*K, L_out a multiple of 32) heads: x,
    offsets and mask; forward: x, offsets, mask, out.  Otherwise trunk: x,
    t; heads: t per head, offsets and mask; forward as before."""
    GK = w.G * w.K
    heads = 2 if w.modulated else 1
    flops = (2 * w.B * w.C_in * w.L_out * w.K + 2 * w.B * w.L_out * w.C_in * GK * heads
             + 2 * w.B * w.C_out * w.L_out * (w.C_in // w.groups) * w.K
             + (4 if w.modulated else 3) * w.B * w.C_in * w.L_out * w.K)
    x, t, out = w.B * w.C_in * w.L_in, w.B * w.C_in * w.L_out, w.B * w.C_out * w.L_out
    gen = w.B * GK * w.L_out * heads
    params = w.C_in * (w.K + 1) + (GK * w.C_in + GK) * heads + w.C_out * ((w.C_in // w.groups) * w.K + 1)
    fused = w.K <= 4 and w.C_in <= 64 and GK * heads <= 128 * w.K and w.L_out % 32 == 0
    if fused:
        pipeline = 4 * ((x + gen) + (x + gen + out) + params)
    else:
        pipeline = 4 * ((x + t) + (t * heads + gen) + (x + gen + out) + params)
    compulsory = 4 * (x + params + out)
    return flops, pipeline, compulsory


def packed_label(w):
    return "%s B%d Cin%d Cout%d L%d K%d s%d p%d d%d groups%d G%d%s f32" % (
        w.name, w.B, w.C_in, w.C_out, w.L_in, w.K, w.stride, w.padding, w.dilation, w.groups, w.G,
        " modulated" if w.modulated else "")


def run_packed(w, steps, warmup, check=True, baseline=True):
    """Time the packed layer (generator + forward) on the GPU; check every
    output against one full oracle run, which is also the CPU baseline."""
    import torch
    from deformable_convolution_amd import dc1d, inputs

    dev = torch.device("cuda:0")
    t = inputs.make_packed_inputs(w, seed=0)
    g = {k: (v.to(dev) if v is not None else None) for k, v in t.items()}
    kw = dict(stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)
    args = (g["x"], g["trunk_weight"], g["trunk_bias"], g["off_weight"], g["off_bias"], g["weight"], g["bias"],
            g["mask_weight"], g["mask_bias"])
    out = torch.empty((w.B, w.C_out, w.L_out), dtype=torch.float32, device=dev)
    nws = dc1d.packed_workspace_bytes(g["x"], g["trunk_weight"], g["off_weight"], g["weight"], g["mask_weight"], **kw)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev) if nws else None

    def step():
        dc1d.packed_forward(*args, out=out, workspace=ws, **kw)

    step()
    torch.cuda.synchronize()
    parity = cpu = None
    if check or baseline:
        import oracle
        cores = len(os.sched_getaffinity(0))
        os.environ.setdefault("OMP_NUM_THREADS", str(cores))
        t0 = time.perf_counter()
        ref, r_off, r_mask = oracle.packed_forward(t["x"], t["trunk_weight"], t["trunk_bias"], t["off_weight"],
                                                   t["off_bias"], t["weight"], t["bias"], t["mask_weight"],
                                                   t["mask_bias"], **kw)
        el = time.perf_counter() - t0
        flops, _, _ = work_packed(w)
        cpu = {"value": flops / el / 1e9, "unit": "GFLOP/s",
               "cores": min(int(os.environ["OMP_NUM_THREADS"]), cores), "kind": "oracle",
               "sample": "1 full packed-layer forward (generator and forward, all %d outputs), %.1f s, on %s"
               % (w.B * w.C_out * w.L_out, el, cpu_model())}
        # the generated offsets and mask against the oracle's generator, and
        # the output against the oracle's forward on the GPU's own offsets and
        # mask with the forward's bound, as in the packed parity tests
        o2, gen = dc1d.packed_forward(*args, with_offsets=True, **kw)
        torch.cuda.synchronize()
        g_off, g_mask = gen if w.modulated else (gen, None)
        a = out.double().cpu().numpy()
        assert np.array_equal(a, o2.double().cpu().numpy()), "packed output differs with the offsets returned"
        rms = lambda v: math.sqrt(float(np.mean(v ** 2)))
        a_off = g_off.double().cpu().numpy()
        a_m = g_mask.double().cpu().numpy() if g_mask is not None else None
        tol_o = 1e-5 * math.sqrt(w.C_in) * max(rms(r_off), 1.0)
        tol_m = tol_o / 4 + 2.0 ** -20
        gen_ok = float(np.abs(a_off - r_off).max()) <= tol_o and (a_m is None or float(np.abs(a_m - r_mask).max()) <= tol_m)
        g_ref = oracle.forward(t["x"], a_off, t["weight"], t["bias"], a_m, **kw)
        tol = 1e-5 * math.sqrt((w.C_in // w.groups) * w.K)
        err = float(np.abs(a - g_ref).max())
        err_ref = float(np.abs(a - ref).max())
        parity = {"elements": int(ref.size), "max_err": err, "tol": tol, "generator_ok": gen_ok,
                  "max_err_vs_oracle_generator": err_ref, "ok": bool(err <= tol and gen_ok)}
        if not parity["ok"]:
            raise SystemExit("packed parity check failed: %r" % parity)
    tm = timed(step, steps, warmup, dev)
    return {"region_ms": tm["region_ms"], "launch_ms": tm["launch_ms"], "eager_ms": tm["eager_ms"],
            "graph": tm["graph"], "parity": parity, "cpu": cpu}


def main_packed(args, w, stream=None):
    r = run_packed(w, args.steps, args.warmup, baseline=not args.no_cpu_baseline)
    flops, pipeline, compulsory = work_packed(w)
    ms = r["region_ms"] / args.steps
    kern_ms = float(np.mean(r["launch_ms"]))  # per-launch events, as the kernel trace sees them
    achieved = pipeline / (kern_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK["hbm_GBps"], "unit": "GB/s",
            "frac": round(achieved / PEAK["hbm_GBps"], 4), "traffic": read_traffic(w.name, "packed", kernel_hash("packed")),
            "kernel": "packed", "call_ms": round(kern_ms, 5)}  # the whole layer call (all its kernels)
    line = {
        "metric": "Packed DeformConv1d fwd GFLOP/s (offset/mask generator + forward)",
        "value": round(flops / (ms * 1e-3) / 1e9, 1),
        "unit": "GFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic, seeded (deformable_convolution_amd/inputs.py; no dataset)",
        "config": {"workload": packed_label(w), "pass": "packed forward",
                   "compulsory_gb_per_s": round(compulsory / (ms * 1e-3) / 1e9, 1),
                   "parity": r["parity"], "timing": "graph replay" if r["graph"] else "eager",
                   "forward_ms": {"warm": pct(r["launch_ms"]), "eager": pct(r["eager_ms"])}},
        "roofline": roof,
    }
    if r["cpu"] is not None:
        line["cpu_baseline"] = r["cpu"]
    print(json.dumps(line), file=stream or sys.stdout, flush=True)


def work2d(w):
    """Work of one 2D forward: contraction flops, sampling flops (the
    bilinear blend of four neighbours: 7 per sample, 8 with the mask), and
    the bytes of every input read once and the output written once."""
    T, HWo = w.kh * w.kw, w.Ho * w.Wo
    contraction = 2 * w.B * w.C_out * HWo * (w.C_in // w.groups) * T
    sampling = (8 if w.modulated else 7) * w.B * w.C_in * T * HWo
    es = 4 if w.dtype == "f32" else 2
    elems = (w.B * w.C_in * w.H * w.W + w.B * w.G * T * HWo * (3 if w.modulated else 2)
             + w.C_out * (w.C_in // w.groups) * T + w.C_out + w.B * w.C_out * HWo)
    return contraction, sampling, elems * es


def label2d(w):
    return "%s B%d Cin%d Cout%d %dx%d k%dx%d s%s p%s d%s groups%d G%d%s %s" % (
        w.name, w.B, w.C_in, w.C_out, w.H, w.W, w.kh, w.kw, w.stride, w.padding, w.dilation, w.groups, w.G,
        " mask" if w.modulated else "", w.dtype)


def run2d(w, steps, warmup, check=True, baseline=True):
    """Time the 2D forward; check whole images of the first and last batch
    against the oracle, whose run on one image is also the CPU baseline."""
    import torch
    from deformable_convolution_amd import dc1d, inputs

    dev = torch.device("cuda:0")
    t = inputs.make_inputs2d(w, seed=0)
    g = {k: (v.to(dev) if v is not None else None) for k, v in t.items()}
    kw = dict(stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)
    kern = dc1d.plan2d(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], **kw)
    nws = dc1d.workspace_bytes2d(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], **kw)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev) if nws else None
    out = torch.empty((w.B, w.C_out, w.Ho, w.Wo), dtype=g["x"].dtype, device=dev)

    def step():
        dc1d.forward2d(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], out=out, workspace=ws, **kw)

    step()
    torch.cuda.synchronize()
    parity = cpu = None
    if check or baseline:
        import oracle
        cores = len(os.sched_getaffinity(0))
        os.environ.setdefault("OMP_NUM_THREADS", str(cores))
        worst, el = 0.0, 0.0
        for b in (0, w.B - 1):
            sl = {k: (v[b:b + 1] if v is not None and k in ("x", "offsets", "mask") else v) for k, v in t.items()}
            t0 = time.perf_counter()
            ref = oracle.forward2d(sl["x"], sl["offsets"], sl["weight"], sl["bias"], sl["mask"], **kw)
            el = time.perf_counter() - t0
            a = out[b:b + 1].double().cpu().numpy()
            rms = math.sqrt(float(np.mean(ref ** 2)))
            if w.dtype == "f32":
                tol = 1e-5 * math.sqrt(w.C_in // w.groups * w.kh * w.kw)
                worst = max(worst, float(np.abs(a - ref).max()) / tol)
            else:
                worst = max(worst, float((np.abs(a - ref) / (2e-2 * np.maximum(np.abs(ref), rms))).max()))
        parity = {"images": 2, "max_err_over_tol": worst, "ok": bool(worst <= 1.0)}
        if not parity["ok"]:
            raise SystemExit("2D parity check failed: %r" % parity)
        c1, s1, _ = work2d(w.with_batch(1))
        cpu = {"value": (c1 + s1) / el / 1e9, "unit": "GFLOP/s",
               "cores": min(int(os.environ["OMP_NUM_THREADS"]), cores), "kind": "oracle",
               "sample": "1 image of the batch (all its %d outputs), %.1f s, on %s" % (w.C_out * w.Ho * w.Wo, el,
                                                                                     cpu_model())}
    tm = timed(step, steps, warmup, dev)
    return {"kernel": kern, "region_ms": tm["region_ms"], "launch_ms": tm["launch_ms"], "parity": parity, "cpu": cpu}


def main2d(args, w, stream=None):
    r = run2d(w, args.steps, args.warmup, baseline=not args.no_cpu_baseline)
    contraction, sampling, nbytes = work2d(w)
    ms = r["region_ms"] / args.steps
    kern_ms = float(np.mean(r["launch_ms"]))  # per-launch events, as the kernel trace sees them
    peak = PEAK["mfma_f32_TFLOPs"] if w.dtype == "f32" else PEAK["mfma_bf16_TFLOPs"]
    achieved = contraction / (kern_ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": read_traffic(w.name, r["kernel"], kernel_hash(r["kernel"])),
            "kernel": r["kernel"], "call_ms": round(kern_ms, 5)}  # the whole call (sampler and GEMM)
    es = 4 if w.dtype == "f32" else 2
    s_bytes = 2 * w.B * (w.C_in // w.groups) * w.kh * w.kw * w.Ho * w.Wo * es  # the sampled matrix, out and back
    line = {
        "metric": "Deformable conv2d (DCNv2) fwd GFLOP/s",
        "value": round((contraction + sampling) / (ms * 1e-3) / 1e9, 1),
        "unit": "GFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic, seeded (deformable_convolution_amd/inputs.py; no dataset)",
        "config": {"workload": label2d(w), "gb_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                   "hbm_frac_with_sampled_matrix": round((nbytes + s_bytes) / (ms * 1e-3) / 1e9 / PEAK["hbm_GBps"], 4),
                   "parity": r["parity"], "forward_ms": {"warm": pct(r["launch_ms"])}},
        "roofline": roof,
    }
    if r["cpu"] is not None:
        line["cpu_baseline"] = r["cpu"]
    print(json.dumps(line), file=stream or sys.stdout, flush=True)


def pct(v):
    """median, p10, p90 of a list of times (ms)."""
    if not v:
        return None
    q = np.percentile(np.asarray(v), [50, 10, 90])
    return {"median": round(float(q[0]), 5), "p10": round(float(q[1]), 5), "p90": round(float(q[2]), 5),
            "n": len(v)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s=12.0, max_reps=200, constrained=False):
    """The oracle, untouched, on this host's cores: full forwards of the same
    workload repeated until about budget_s seconds have passed.  Returns the
    baseline record and the last forward's output (every element, for the
    parity check of the GPU's output)."""
    import oracle
    from deformable_convolution_amd import inputs

    t = inputs.make_inputs(w, seed=0)
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    kw = dict(stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)
    contraction, sampling, _ = work(w)
    oracle.forward(t["x"], t["offsets"], t["weight"], t["bias"], t["mask"], constrained=constrained,
                   **kw)  # warm (untimed)
    reps, t0 = 0, time.perf_counter()
    while True:
        ref = oracle.forward(t["x"], t["offsets"], t["weight"], t["bias"], t["mask"], constrained=constrained,
                             **kw)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= max_reps:
            break
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    return {"value": (contraction + sampling) * reps / el / 1e9, "unit": "GFLOP/s", "cores": min(threads, cores),
            "kind": "oracle",
            "sample": "%d full forward(s) of the same workload (all %d outputs each), %.1f s, on %s" % (
                reps, w.B * w.C_out * w.L_out, el, cpu_model())}, ref


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dc1d_layer")
    ap.add_argument("--only", action="store_true",
                    help="time the named workload alone (no stderr records of the other workloads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-run", action="store_true")
    ap.add_argument("--backward", action="store_true", help="time the backward (fp32 workloads) instead")
    ap.add_argument("--constrained", action="store_true",
                    help="the forward in constrained mode (every tap kept inside its kernel window)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB")
    ap.add_argument("--summarize-profile", default=None, metavar="DIR")
    ap.add_argument("--kernel", default=None, help="the plan's kernel name, for --summarize-profile")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only; the forward shards by batch or output channel "
              "with no exchange, and no multi-GPU figure is produced.", file=sys.stderr)
        raise SystemExit(2)
    if args.summarize_profile:
        if not args.kernel:
            raise SystemExit("--summarize-profile needs --kernel (the plan's kernel name, or backward)")
        write_profile_md(args.summarize_profile, args.workload, args.kernel)
        return

    import torch
    from deformable_convolution_amd import inputs

    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        print("copied %d bytes" % n, flush=True)
        return

    if args.constrained and (args.workload in inputs.WORKLOADS_2D or args.workload in inputs.PACKED_WORKLOADS):
        raise SystemExit("--constrained times the 1D forward workloads (%s)" % ", ".join(sorted(inputs.WORKLOADS)))
    if args.workload in inputs.WORKLOADS_2D:
        w = inputs.WORKLOADS_2D[args.workload]
        if args.profile_run:
            r = run2d(w, args.steps, args.warmup, check=False, baseline=False)
            print("profile run: %s %s, %d timed launches" % (w.name, r["kernel"], args.steps), flush=True)
            return
        main2d(args, w)
        return
    if args.workload in inputs.PACKED_WORKLOADS:
        w = inputs.PACKED_WORKLOADS[args.workload]
        if args.profile_run:
            run_packed(w, args.steps, args.warmup, check=False, baseline=False)
            print("profile run: %s packed, %d timed launches" % (w.name, args.steps), flush=True)
            return
        main_packed(args, w)
        return
    w = inputs.WORKLOADS[args.workload]
    if args.backward:
        if args.constrained:
            raise SystemExit("--constrained times the forward")
        if args.profile_run:
            run_backward(w, args.steps, args.warmup, check=False, baseline=False)
            print("profile run: %s backward, %d timed launches" % (w.name, args.steps), flush=True)
            return
        main_backward(args, w)
        return
    if args.profile_run:
        r = run_gpu(w, args.steps, args.warmup, constrained=args.constrained)
        print("profile run: %s %s, %d timed launches, %.4f ms/launch" % (
            w.name, r["plan"]["kernel"], args.steps, float(np.mean(r["launch_ms"]))), flush=True)
        return

    # The other workloads first, one JSON record each on stderr (timing,
    # roofline, full-output parity against the oracle), then the headline.
    if not args.only:
        for name in inputs.WORKLOAD_ORDER:
            if name == w.name:
                continue
            rec = workload_line(inputs.WORKLOADS[name], max(10, args.steps // 2), args.warmup)
            print(json.dumps(rec), file=sys.stderr, flush=True)
        # then the scope table's other rows, one record each on stderr: the
        # backward (the layer shape and the depthwise shape), the packed
        # layer, 2D in bf16 and fp32 -- each with its own parity check and
        # CPU baseline; one that fails leaves an error record and the
        # headline is still measured
        sub = argparse.Namespace(steps=max(10, args.steps // 2), warmup=args.warmup,
                                 no_cpu_baseline=args.no_cpu_baseline)
        for mode, name in (("backward", "dc1d_layer"), ("backward", "depthwise"), ("packed", "packed"),
                           ("2d", "dcn2d_bf16"), ("2d", "dcn2d")):
            try:
                if mode == "backward":
                    main_backward(sub, inputs.WORKLOADS[name], stream=sys.stderr)
                elif mode == "packed":
                    main_packed(sub, inputs.PACKED_WORKLOADS[name], stream=sys.stderr)
                else:
                    main2d(sub, inputs.WORKLOADS_2D[name], stream=sys.stderr)
            except (Exception, SystemExit) as e:  # noqa: BLE001 -- reported, the headline still runs
                print(json.dumps({"workload": name, "pass": mode, "error": repr(e), "ok": False}), file=sys.stderr,
                      flush=True)

    t = inputs.make_inputs(w, seed=0)
    r = run_gpu(w, args.steps, args.warmup, cold_reps=20, constrained=args.constrained, t=t)
    contraction, sampling, nbytes = work(w)
    ms = r["region_ms"] / args.steps
    kern = r["plan"]["kernel"]
    roof = roofline_of(w, kern, float(np.mean(r["kernel_ms"])), float(np.mean(r["launch_ms"])),
                       constrained=args.constrained)
    # parity: every output against the oracle's, from the CPU baseline's own
    # run (or a run of its own when the baseline is not taken)
    if args.no_cpu_baseline:
        base = None
        ref, _ = oracle_reference(w, t, constrained=args.constrained)
    else:
        base, ref = cpu_baseline(w, constrained=args.constrained)
    parity = parity_of(w, r["out"].double().cpu().numpy(), ref)
    if not parity["ok"]:
        raise SystemExit("bench parity check failed: %r" % parity)
    line = {
        "metric": METRIC,
        "value": round((contraction + sampling) / (ms * 1e-3) / 1e9, 1),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.dtype == "f32" else "bf16",
        "data": "synthetic, seeded (deformable_convolution_amd/inputs.py; no dataset)",
        "config": {"workload": workload_label(w) + (" constrained" if args.constrained else ""), "plan": r["plan"],
                   "gb_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1), "parity": parity,
                   "timing": "graph replay" if r["graph"] else "eager",
                   "forward_ms": {"warm": pct(r["launch_ms"]), "kernel": pct(r["kernel_ms"]),
                                  "cold": pct(r["cold_ms"]), "eager": pct(r["eager_ms"])}},
        "roofline": roof,
    }
    if base is not None:
        line["cpu_baseline"] = base
    print(json.dumps(line), flush=True)


PROFILE_COMMANDS = """\
cd /tmp && export TMPDIR=/tmp; R=<repo root>; P=<output dir>/{wl}{suffix}
rocprofv3 --kernel-trace --stats --output-format csv -d $P/trace -o run -- \\
    python3 $R/bench.py --workload {wl}{flag} --profile-run --steps 20 --warmup 3
rocprofv3 --pmc FETCH_SIZE --output-format csv -d $P/fetch -o run -- \\
    python3 $R/bench.py --workload {wl}{flag} --profile-run --steps 5 --warmup 1
rocprofv3 --pmc WRITE_SIZE --output-format csv -d $P/write -o run -- \\
    python3 $R/bench.py --workload {wl}{flag} --profile-run --steps 5 --warmup 1
rocprofv3 --pmc FETCH_SIZE --output-format csv -d $P/copy_fetch -o run -- \\
    python3 $R/bench.py --copy-calibration 512
rocprofv3 --pmc WRITE_SIZE --output-format csv -d $P/copy_write -o run -- \\
    python3 $R/bench.py --copy-calibration 512
python3 $R/bench.py --workload {wl}{flag} --summarize-profile $P --kernel {kernel}
"""


def short(name):
    """A kernel's name without namespaces and arguments."""
    name = name.replace("(anonymous namespace)::", "").replace("dc1d::", "").replace("void ", "")
    return name.split("(")[0][:100]


def summarize_profile(d, workload):
    """Fold the rocprofv3 output of PROFILE_COMMANDS (kernel-trace stats, then
    FETCH_SIZE and WRITE_SIZE passes of the profile run and of a 512 MiB
    device copy) into profiles/<workload>__<kernel>.md.  The copy fixes the
    scale of the counters: bytes a copy of N bytes must read and write over
    what the counters report for it."""
    import csv
    import glob

    from deformable_convolution_amd import inputs

    w = (inputs.PACKED_WORKLOADS.get(workload) or inputs.WORKLOADS_2D.get(workload) or inputs.WORKLOADS[workload])

    def csvs(sub, pattern):
        out = []
        for f in sorted(glob.glob(os.path.join(d, sub, "**", pattern), recursive=True)):
            out += list(csv.DictReader(open(f)))
        return out


    def ours(name):
        return "dc1d::" in name

    stats = [r for r in csvs("trace", "*kernel_stats.csv") if ours(r["Name"])]

    def counter(sub, cname):
        acc = {}
        for r in csvs(sub, "*counter_collection.csv"):
            if r.get("Counter_Name") == cname:
                acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return acc

    fetch, write = counter("fetch", "FETCH_SIZE"), counter("write", "WRITE_SIZE")
    cf, cw = counter("copy_fetch", "FETCH_SIZE"), counter("copy_write", "WRITE_SIZE")
    copy_bytes = 512 << 20
    # the copy's dispatch is the one that moved the most
    cf_v = max((max(v) for v in cf.values()), default=0.0)
    cw_v = max((max(v) for v in cw.values()), default=0.0)
    f_scale = copy_bytes / cf_v if cf_v > 0 else None
    w_scale = copy_bytes / cw_v if cw_v > 0 else None

    # launches in the counter runs: the fewest dispatches any of our kernels
    # had (every kernel runs at least once per launch)
    ours_f = {k: v for k, v in fetch.items() if ours(k)}
    ours_w = {k: v for k, v in write.items() if ours(k)}
    nf = min((len(v) for v in ours_f.values()), default=1)
    nw = min((len(v) for v in ours_w.values()), default=1)
    rows_k = []
    total_bytes = 0.0
    for name in sorted(set(ours_f) | set(ours_w)):
        fv = float(np.sum(ours_f.get(name, [0.0]))) / nf  # counter units per launch
        wv = float(np.sum(ours_w.get(name, [0.0]))) / nw
        fb = fv * f_scale if f_scale else None
        wb = wv * w_scale if w_scale else None
        if fb is not None and wb is not None:
            total_bytes += fb + wb
        rows_k.append((short(name), fv, wv, fb, wb))
    return stats, rows_k, total_bytes, (cf_v, cw_v, f_scale, w_scale), w


def write_profile_md(d, workload, kernel):
    stats, rows_k, total_bytes, (cf_v, cw_v, f_scale, w_scale), w = summarize_profile(d, workload)
    is2d = workload in __import__("deformable_convolution_amd.inputs", fromlist=["x"]).WORKLOADS_2D
    if kernel == "packed":
        contraction, alg_bytes, _ = work_packed(w)
    elif is2d:
        contraction, sampling, alg_bytes = work2d(w)
    else:
        contraction, sampling, alg_bytes = work_backward(w) if kernel == "backward" else work(w)
    # launches in the trace run: the fewest calls of any of our kernels
    n_launch = min((int(r["Calls"]) for r in stats), default=1)
    fwd_ns = sum(float(r["TotalDurationNs"]) for r in stats) / max(n_launch, 1)
    out = []
    out.append("# %s -- %s" % (packed_label(w) if kernel == "packed" else (label2d(w) if is2d else workload_label(w)),
                               kernel))
    out.append("")
    out.append("<!-- kernel=%s -->" % kernel)
    out.append("<!-- kernel_sources=%s -->" % kernel_hash(kernel))
    if rows_k and f_scale and w_scale:
        out.append("<!-- hbm_bytes_per_launch=%.0f -->" % total_bytes)
    out.append("")
    out.append("One launch = one %s call (every kernel it enqueues, back to back on one stream)."
               % {"backward": "backward (all five gradients)", "packed": "packed-layer forward (generator and "
                  "forward)"}.get(kernel, "forward"))
    out.append("")
    out.append("Commands (rocprofv3, ROCm 7.2, one MI355X):")
    out.append("")
    out.append("```")
    bwd, con = kernel == "backward", kernel.endswith("_constrained")
    out.append(PROFILE_COMMANDS.format(wl=workload, kernel=kernel,
                                       flag=" --backward" if bwd else (" --constrained" if con else ""),
                                       suffix="_backward" if bwd else ("_constrained" if con else "")).rstrip())
    out.append("```")
    out.append("")
    out.append("## Kernel trace (--kernel-trace --stats)")
    out.append("")
    out.append("| kernel | calls | average (us) | total (us) |")
    out.append("|---|---|---|---|")
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        out.append("| %s | %s | %.2f | %.1f |" % (short(r["Name"]), r["Calls"],
                                               float(r["AverageNs"]) / 1e3, float(r["TotalDurationNs"]) / 1e3))
    out.append("")
    out.append("Kernel time per launch (all its kernels' total over %d launches): %.2f us; %s %.3f GFLOP "
               "-> %.1f TFLOP/s over that time." % (n_launch, fwd_ns / 1e3,
                                                    "all flops" if kernel == "packed" else "contraction",
                                                    contraction / 1e9,
                                                    contraction / (fwd_ns * 1e-9) / 1e12 if fwd_ns else 0.0))
    out.append("")
    out.append("## HBM traffic (--pmc FETCH_SIZE, --pmc WRITE_SIZE; counter units per launch, all dispatches)")
    out.append("")
    if f_scale and w_scale:
        out.append("Copy calibration: a 512 MiB device-to-device copy reads as FETCH_SIZE %.0f and WRITE_SIZE %.0f; "
                   "scale factors %.4f and %.4f bytes per counter unit." % (cf_v, cw_v, f_scale, w_scale))
    else:
        out.append("Copy calibration missing: traffic not scaled.")
    out.append("")
    out.append("| kernel | FETCH_SIZE | WRITE_SIZE | fetched (MB) | written (MB) |")
    out.append("|---|---|---|---|---|")
    for name, fv, wv, fb, wb in rows_k:
        out.append("| %s | %.0f | %.0f | %s | %s |" % (name, fv, wv, "%.2f" % (fb / 1e6) if fb else "-",
                                                   "%.2f" % (wb / 1e6) if wb else "-"))
    out.append("")
    out.append("Per launch: %.2f MB of HBM traffic against %.2f MB of algorithmic bytes (each tensor moved once)."
               % (total_bytes / 1e6, alg_bytes / 1e6))
    path = os.path.join(ROOT, "profiles", "%s__%s.md" % (workload, kernel))
    os.makedirs(os.path.dirname(path), exist_ok=True)
    open(path, "w").write("\n".join(out) + "\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
