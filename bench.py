"""Benchmark of the DeformConv1d forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--all]

One step is one forward (the whole hot path: position split, interpolation,
modulation, contraction, bias) over one batch of seeded synthetic inputs
that are already resident in device memory.  The default workload is the
dc1d page's layer shape (B16, C512 -> 512, K16, dilation 3, "valid", L128,
fp32).  Prints ONE JSON line (rank 0, one GPU):

  value      contraction + sampling GFLOP per step / seconds per step
  roofline   the dominant kernel's achieved rate against its roofline peak,
             from HIP events around every timed launch on the launch stream
  cpu_baseline  the CPU oracle timed on the host cores (reported baseline)

Parity is checked in the same run (sampled outputs against the oracle)
before timing; a mismatch aborts the bench.

--all additionally writes one JSON line per named workload to stderr.
--profile-run runs only the warmup + timed launches (no oracle, no JSON),
for rocprofv3; --copy-calibration MB runs one device-to-device copy of that
size (the reference kernel for scaling the HBM byte counters).
--summarize-counters DIR folds rocprofv3 counter CSVs into the markdown
summary kept under profiles/.
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


def kernel_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def workload_label(w):
    return "%s B%d Cin%d Cout%d L%d K%d s%d p%d d%d groups%d G%d%s %s" % (
        w.name, w.B, w.C_in, w.C_out, w.L_in, w.K, w.stride, w.padding, w.dilation, w.groups, w.G,
        " mask" if w.mask_dist else "", w.dtype)


def read_traffic(name, kernel, khash):
    """HBM bytes per launch of `kernel` on workload `name` from the committed
    counter summary, or None if absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "counters_%s.md" % name)
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


def run_gpu(w, steps, warmup, check=True, quiet=False):
    import torch
    from deformable_convolution_amd import dc1d, inputs

    dev = torch.device("cuda:0")
    t = inputs.make_inputs(w, seed=0)
    g = {k: (v.to(dev) if v is not None else None) for k, v in t.items()}
    kw = dict(stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)
    plan = dc1d.plan(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], **kw)
    out = torch.empty((w.B, w.C_out, w.L_out), dtype=g["x"].dtype, device=dev)
    nws = dc1d.workspace_bytes(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], **kw)
    ws = torch.zeros(max(nws, 1), dtype=torch.uint8, device=dev) if nws else None

    def step():
        dc1d.forward(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"], out=out, workspace=ws, **kw)

    step()
    torch.cuda.synchronize()
    parity = None
    if check:
        import oracle
        rng = np.random.default_rng(1)
        n = 512
        pts = np.stack([rng.integers(0, w.B, n), rng.integers(0, w.C_out, n), rng.integers(0, w.L_out, n)], 1)
        ref = oracle.forward_points(t["x"], t["offsets"], t["weight"], pts, t["bias"], t["mask"], **kw)
        got = out[pts[:, 0], pts[:, 1], pts[:, 2]].double().cpu().numpy()
        if w.dtype == "f32":
            err = float(np.abs(got - ref).max())
            tol = 1e-5 * math.sqrt(w.C_in * w.K / w.groups)
            ok = err <= tol
        else:
            rms = math.sqrt(float(np.mean(ref ** 2)))
            err = float((np.abs(got - ref) / np.maximum(np.abs(ref), rms)).max())
            tol = 2e-2
            ok = err <= tol
        parity = {"points": n, "max_err": err, "tol": tol, "ok": bool(ok)}
        if not ok:
            raise SystemExit("bench parity check failed: %r" % parity)

    stream = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    region0 = torch.cuda.Event(enable_timing=True)
    region1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    region0.record(stream)
    for i in range(steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    region1.record(stream)
    torch.cuda.synchronize()
    region_ms = region0.elapsed_time(region1)
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    return {"plan": plan, "region_ms": region_ms, "launch_ms": launch_ms, "parity": parity}


def cpu_baseline(w, budget_s=12.0, max_reps=20):
    """The oracle, untouched, on this host's cores: full forwards of the same
    workload repeated until about budget_s seconds have passed."""
    import oracle
    from deformable_convolution_amd import inputs

    t = inputs.make_inputs(w, seed=0)
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    kw = dict(stride=w.stride, padding=w.padding, dilation=w.dilation, groups=w.groups)
    contraction, sampling, _ = work(w)
    oracle.forward(t["x"], t["offsets"], t["weight"], t["bias"], t["mask"], **kw)  # warm (untimed)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(t["x"], t["offsets"], t["weight"], t["bias"], t["mask"], **kw)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= max_reps:
            break
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    return {"value": (contraction + sampling) * reps / el / 1e9, "unit": "GFLOP/s", "cores": min(threads, cores),
            "kind": "oracle",
            "sample": "%d full forward(s) of the same workload (all %d outputs each), %.1f s" % (
                reps, w.B * w.C_out * w.L_out, el)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dc1d_layer")
    ap.add_argument("--all", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-run", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB")
    ap.add_argument("--summarize-counters", default=None, metavar="DIR")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; the forward shards by batch or output channel "
              "with no exchange (see DESIGN.md), and no multi-GPU figure is produced.", file=sys.stderr)
        raise SystemExit(2)
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.workload)
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

    w = inputs.WORKLOADS[args.workload]
    if args.profile_run:
        r = run_gpu(w, args.steps, args.warmup, check=False)
        print("profile run: %s %s, %d timed launches, %.4f ms/launch" % (
            w.name, r["plan"]["kernel"], args.steps, float(np.mean(r["launch_ms"]))), flush=True)
        return

    r = run_gpu(w, args.steps, args.warmup)
    contraction, sampling, nbytes = work(w)
    ms = r["region_ms"] / args.steps
    kern_ms = float(np.mean(r["launch_ms"]))
    kern = r["plan"]["kernel"]
    if kern.startswith("mfma"):
        peak = PEAK["mfma_f32_TFLOPs"] if w.dtype == "f32" else PEAK["mfma_bf16_TFLOPs"]
        achieved = contraction / (kern_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4)}
    else:
        achieved = nbytes / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK["hbm_GBps"], "unit": "GB/s",
                "frac": round(achieved / PEAK["hbm_GBps"], 4)}
    traffic = read_traffic(w.name, kern, kernel_hash())
    roof["traffic"] = traffic
    roof["kernel"] = kern
    roof["kernel_ms"] = round(kern_ms, 5)
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
        "data": "synthetic (seeded; see DESIGN.md input recipe)",
        "config": {"workload": workload_label(w), "plan": r["plan"],
                   "gb_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1), "parity": r["parity"]},
        "roofline": roof,
    }
    if args.all:
        for name in inputs.WORKLOAD_ORDER:
            ww = inputs.WORKLOADS[name]
            rr = run_gpu(ww, max(10, args.steps // 2), args.warmup)
            c2, s2, b2 = work(ww)
            m2 = float(np.mean(rr["launch_ms"]))
            rec = {"workload": workload_label(ww), "kernel": rr["plan"]["kernel"], "plan": rr["plan"],
                   "ms": round(m2, 5), "GFLOP/s": round((c2 + s2) / (m2 * 1e-3) / 1e9, 1),
                   "GB/s": round(b2 / (m2 * 1e-3) / 1e9, 1), "parity": rr["parity"]}
            if rr["plan"]["kernel"].startswith("mfma"):
                pk = PEAK["mfma_f32_TFLOPs"] if ww.dtype == "f32" else PEAK["mfma_bf16_TFLOPs"]
                rec["mfma_frac"] = round(c2 / (m2 * 1e-3) / 1e12 / pk, 4)
            rec["hbm_frac"] = round(b2 / (m2 * 1e-3) / 1e9 / PEAK["hbm_GBps"], 4)
            print(json.dumps(rec), file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


def summarize_counters(d, workload):
    """Fold rocprofv3 --pmc output (FETCH_SIZE and WRITE_SIZE passes of the
    bench profile run and of the copy calibration) into a markdown summary
    with the per-launch HBM bytes of the dominant kernel."""
    import csv
    import glob

    def rows(sub):
        out = []
        for f in glob.glob(os.path.join(d, sub, "**", "*counter_collection.csv"), recursive=True):
            out += list(csv.DictReader(open(f)))
        return out

    def per_kernel(rs, counter):
        acc = {}
        for r in rs:
            if r.get("Counter_Name") != counter:
                continue
            name = r.get("Kernel_Name", "")
            acc.setdefault(name, []).append(float(r["Counter_Value"]))
        return acc

    res = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        res[counter] = {"bench": per_kernel(rows("bench_" + counter), counter),
                        "copy": per_kernel(rows("copy_" + counter), counter)}
    print(json.dumps({c: {k: {n: (len(v), float(np.mean(v))) for n, v in kk.items()} for k, kk in r.items()}
                      for c, r in res.items()}, indent=1))


if __name__ == "__main__":
    main()
