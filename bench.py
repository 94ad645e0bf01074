#!/usr/bin/env python3
"""Benchmark: fused RMSNorm / LayerNorm forward + backward on one MI355X.

A step is one pass of the whole path over one batch: the forward (y, saved mean/rstd)
followed by the backward (dx, and dgamma/dbeta through the two-stage column reduction).
Inputs are seeded synthetic tensors resident in HBM before timing starts.

Metric: effective bandwidth = algorithmic bytes / time, where the algorithmic bytes are
what the method must move (s = bytes per element):
    forward  RMS: 2*M*N*s + N*s + 4*M           LN: 2*M*N*s + 2*N*s + 8*M
    backward RMS: 3*M*N*s + N*s + 4*M + 4*N     LN: 3*M*N*s + N*s + 8*M + 8*N
The roofline entry is for the dominant kernel (the backward's dx + partials kernel),
timed by HIP events recorded around every launch of it inside the timed loop.

Prints ONE JSON line on stdout.  --all additionally writes a per-workload table.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "RMSNorm/LayerNorm fwd+bwd effective GB/s and % of MI355X HBM peak, bf16"
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "ln2"
MALL_BYTES = 256 << 20
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_bwd_rows_ln2.json")


def ideal_bytes(kind, M, N, s):
    if kind == "rms":
        return 2 * M * N * s + N * s + 4 * M, 3 * M * N * s + N * s + 4 * M + 4 * N
    return 2 * M * N * s + 2 * N * s + 8 * M, 3 * M * N * s + N * s + 8 * M + 8 * N


def main_bwd_kernel_bytes(kind, M, N, s):
    """Bytes the backward's main kernel must move: read x, dy, gamma, the saved statistics,
    write dx (the dgamma/dbeta output is written by the column reduce)."""
    return 3 * M * N * s + N * s + (4 if kind == "rms" else 8) * M


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "row_normalization_norm_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def describe(w):
    dist = f"N({w.x_mean:g},{w.x_std:g})"
    if w.outlier_p:
        dist += f" with {w.outlier_p:.0%} of entries x{w.outlier_scale:g}"
    kind = "RMSNorm" if w.kind == "rms" else "LayerNorm"
    return f"{kind} fwd+bwd x[{w.M},{w.N}] {w.dtype} {dist}, eps={w.eps:g}"


def to_device(a, dtype, device):
    """Host array of raw bits (uint16 bf16 / float32) -> device tensor, bit-exact."""
    import numpy as np
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


class Bench:
    """Device buffers (rotating sets when one set would fit in the MALL) for a workload."""

    def __init__(self, w, device):
        import torch
        import gen
        import row_normalization_norm_amd as rn
        self.w, self.device, self.rn = w, device, rn
        t0 = time.time()
        inputs = gen.make_inputs(w)
        s = 2 if w.dtype == "bf16" else 4
        per_set = 4 * w.M * w.N * s  # x, y, dy, dx
        self.sets = max(1, math.ceil(2 * MALL_BYTES / per_set))
        x0 = to_device(inputs["x"], w.dtype, device)
        dy0 = to_device(inputs["dy"], w.dtype, device)
        self.gamma = to_device(inputs["gamma"], w.dtype, device)
        self.beta = to_device(inputs["beta"], w.dtype, device) if w.kind == "ln" else None
        self.bufs = []
        for i in range(self.sets):
            x = x0 if i == 0 else x0.clone()
            dy = dy0 if i == 0 else dy0.clone()
            self.bufs.append(dict(
                x=x, dy=dy, y=torch.empty_like(x), dx=torch.empty_like(x),
                mean=torch.empty(w.M, device=device) if w.kind == "ln" else None,
                rstd=torch.empty(w.M, device=device)))
        self.dgamma = torch.empty(w.N, device=device)
        self.dbeta = torch.empty(w.N, device=device) if w.kind == "ln" else None
        dt = rn.NORM_DTYPE_BF16 if w.dtype == "bf16" else rn.NORM_DTYPE_F32
        ws = rn.norm_bwd_workspace_size(w.M, w.N, w.kind == "ln", dt)
        self.ws = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)
        fws = rn.norm_fwd_workspace_size(w.M, w.N, w.kind == "ln", dt)
        self.fws = torch.empty(fws, dtype=torch.uint8, device=device) if fws else None
        torch.cuda.synchronize()
        self.setup_s = time.time() - t0

    def step(self, k, fwd_opt=None, bwd_opt=None):
        rn, w, b = self.rn, self.w, self.bufs[k % self.sets]
        if w.kind == "rms":
            rn.norm_rms_fwd(b["x"], self.gamma, b["y"], b["rstd"], eps=w.eps, workspace=self.fws,
                            options=fwd_opt)
            rn.norm_rms_bwd(b["dy"], b["x"], self.gamma, b["rstd"], b["dx"], self.dgamma,
                            workspace=self.ws, options=bwd_opt)
        else:
            rn.norm_ln_fwd(b["x"], self.gamma, self.beta, b["y"], b["mean"], b["rstd"], eps=w.eps,
                           workspace=self.fws, options=fwd_opt)
            rn.norm_ln_bwd(b["dy"], b["x"], self.gamma, b["mean"], b["rstd"], b["dx"], self.dgamma,
                           self.dbeta, workspace=self.ws, options=bwd_opt)


def make_events(n):
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    s = torch.cuda.current_stream()
    for e in evs:
        e.record(s)  # create the underlying HIP event so its handle can be passed down
    torch.cuda.synchronize()
    return evs


def run_gpu(w, steps, warmup, device):
    """Two timed passes of `steps` steps each, after `warmup` untimed steps:
    pass A records events only before and after the K steps (the step time); pass B also
    records HIP events around every launch of the forward kernel and of the backward's
    main kernel on the stream they run on (per-kernel average durations).  Per-launch
    events add a few microseconds of gap each, which is why the step time comes from A."""
    import torch
    import row_normalization_norm_amd as rn
    b = Bench(w, device)
    for k in range(warmup):
        b.step(k)
    torch.cuda.synchronize()

    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record()
    for k in range(steps):
        b.step(warmup + k)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(stop)

    fev = make_events(2 * steps)
    bev = make_events(2 * steps)
    fopts = [rn.Options(ev_start=fev[2 * i].cuda_event, ev_stop=fev[2 * i + 1].cuda_event)
             for i in range(steps)]
    bopts = [rn.Options(ev_start=bev[2 * i].cuda_event, ev_stop=bev[2 * i + 1].cuda_event)
             for i in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        b.step(warmup + steps + k, fopts[k], bopts[k])
    torch.cuda.synchronize()
    fwd_ms = sum(fev[2 * i].elapsed_time(fev[2 * i + 1]) for i in range(steps)) / steps
    bwd_ms = sum(bev[2 * i].elapsed_time(bev[2 * i + 1]) for i in range(steps)) / steps
    return dict(ms_per_step=total_ms / steps, fwd_kernel_ms=fwd_ms, bwd_main_kernel_ms=bwd_ms,
                wall_s=wall, sets=b.sets, setup_s=b.setup_s)


def copy_probe(nbytes, steps, device):
    """Time a plain device copy of nbytes (torch's copy kernel): the achievable
    read+write bandwidth next to the nominal peak, and the kernel whose rocprofv3
    FETCH_SIZE / WRITE_SIZE readings scale the counters to bytes."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device=device).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "ms": round(ms, 5),
            "GBs_read_plus_write": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}


def cpu_baseline(w, target_s=12.0):
    """The oracle (as it stands) on the first rows of the same workload: forward (y, stats),
    dx, and dgamma/dbeta over the sampled rows.  Reported in the metric's unit."""
    import gen
    import oracle
    orc = oracle.get()
    rows = 64
    while True:
        sub = w.scaled(rows)
        inp = gen.make_inputs(sub)
        t0 = time.perf_counter()
        if w.kind == "rms":
            orc.rms_fwd(inp["x"], inp["gamma"], w.eps)
            orc.rms_bwd_dx(inp["dy"], inp["x"], inp["gamma"], w.eps)
            orc.rms_dgamma(inp["dy"], inp["x"], w.eps)
        else:
            orc.ln_fwd(inp["x"], inp["gamma"], inp["beta"], w.eps)
            orc.ln_bwd_dx(inp["dy"], inp["x"], inp["gamma"], w.eps)
            orc.ln_dgamma_dbeta(inp["dy"], inp["x"], w.eps)
        dt = time.perf_counter() - t0
        if dt >= target_s / 4 or rows >= w.M:
            break
        rows = min(w.M, int(rows * max(2.0, target_s / max(dt, 1e-3))))
    s = 2 if w.dtype == "bf16" else 4
    f, bwd = ideal_bytes(w.kind, rows, w.N, s)
    return {"value": round((f + bwd) / dt / 1e9, 3), "unit": "GB/s", "cores": orc.num_threads(),
            "kind": "oracle",
            "sample": f"first {rows} of {w.M} rows of the same workload (fp64 C oracle, "
                      f"forward + dx + dgamma/dbeta), {dt:.1f} s"}


def load_counters(w):
    """HBM traffic of the backward's main kernel from committed rocprofv3 counter runs,
    or None when absent or taken on different kernel sources."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    with open(COUNTERS_FILE) as f:
        c = json.load(f)
    if c.get("kernel_source_hash") != kernel_source_hash() or c.get("workload") != w.name:
        return None
    return c.get("traffic_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--all", metavar="JSON", help="also time every workload, write a table")
    ap.add_argument("--copy-probe", type=int, metavar="BYTES",
                    help="only time a plain device copy of BYTES and print it")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(rows shard over GPUs with no exchange; see the design notes). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gen
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import row_normalization_norm_amd as rn
    rn.lib()
    device = torch.device("cuda:0")
    if args.copy_probe:
        print(json.dumps(copy_probe(args.copy_probe, args.steps, device)), flush=True)
        return

    w = gen.WORKLOADS[args.workload]
    s = 2 if w.dtype == "bf16" else 4
    fwd_b, bwd_b = ideal_bytes(w.kind, w.M, w.N, s)
    r = run_gpu(w, args.steps, args.warmup, device)
    value = (fwd_b + bwd_b) / (r["ms_per_step"] * 1e-3) / 1e9

    main_bytes = main_bwd_kernel_bytes(w.kind, w.M, w.N, s)
    achieved = main_bytes / (r["bwd_main_kernel_ms"] * 1e-3) / 1e9
    plan = rn.norm_plan(True, w.kind == "ln", w.M, w.N,
                        rn.NORM_DTYPE_BF16 if w.dtype == "bf16" else rn.NORM_DTYPE_F32)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {describe(w)}", "M": w.M, "N": w.N,
                   "kind": w.kind, "eps": w.eps},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "fwd_GBs": round(fwd_b / (r["fwd_kernel_ms"] * 1e-3) / 1e9, 1),
        "bwd_GBs": round(bwd_b / ((r["ms_per_step"] - r["fwd_kernel_ms"]) * 1e-3) / 1e9, 1),
        "roofline": {
            "bound": "hbm",
            "kernel": f"bwd_rows_kernel (dx + dgamma/dbeta partials), "
                      f"{plan.lanes_per_row}x{plan.vecs_per_lane}, grid {plan.grid}",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": load_counters(w),
            "avg_launch_ms": round(r["bwd_main_kernel_ms"], 5),
            "algorithmic_bytes_per_launch": main_bytes,
            "timing": "HIP events around every launch of the kernel in a second timed "
                      "pass of the same steps",
        },
        "rotating_buffer_sets": r["sets"],
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w)
    if args.all:
        table = []
        sweep = [gen.sweep_workload(k, d, n) for k in ("rms", "ln") for d in ("bf16", "f32")
                 for n in gen.SWEEP_N]
        for wl in list(gen.WORKLOADS.values()) + sweep:
            name = wl.name
            rr = run_gpu(wl, max(5, args.steps // 2), 3, device)
            ss = 2 if wl.dtype == "bf16" else 4
            fb, bb = ideal_bytes(wl.kind, wl.M, wl.N, ss)
            table.append({"workload": name, "desc": describe(wl),
                          **{k: round(v, 5) for k, v in rr.items()},
                          "fwd_GBs": fb / (rr["fwd_kernel_ms"] * 1e-3) / 1e9,
                          "bwd_GBs": bb / ((rr["ms_per_step"] - rr["fwd_kernel_ms"]) * 1e-3) / 1e9,
                          "step_GBs": (fb + bb) / (rr["ms_per_step"] * 1e-3) / 1e9})
            print(f"# {name}: {table[-1]['step_GBs']:.0f} GB/s", file=sys.stderr, flush=True)
        with open(args.all, "w") as f:
            json.dump(table, f, indent=1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
