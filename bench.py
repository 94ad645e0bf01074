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
DEFAULT_STEPS = 50
DEFAULT_WARMUP = 100
# The untimed warm-up lasts at least this long.  Measured on MI355X (LayerNorm [65536,
# 4096] bf16, fresh process, 20 timed steps): after 5 warm-up steps the step runs at
# 5.5 TB/s, after 0.3 s of steps at 6.2 TB/s, the steady state.  The timed region is the
# same K steps either way.
DEFAULT_WARMUP_S = 0.3
MALL_BYTES = 256 << 20
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_bwd_rows_ln2.json")


def ideal_bytes(kind, M, N, s, ps=None):
    """Algorithmic bytes of the forward and of the backward call: s bytes per activation,
    ps per gamma/beta element (default s)."""
    ps = s if ps is None else ps
    if kind == "rms":
        return 2 * M * N * s + N * ps + 4 * M, 3 * M * N * s + N * ps + 4 * M + 4 * N
    return 2 * M * N * s + 2 * N * ps + 8 * M, 3 * M * N * s + N * ps + 8 * M + 8 * N


def main_bwd_kernel_bytes(kind, M, N, s, ps=None):
    """Bytes the backward's main kernel must move: read x, dy, gamma, the saved statistics,
    write dx (the dgamma/dbeta output is written by the column reduce)."""
    ps = s if ps is None else ps
    return 3 * M * N * s + N * ps + (4 if kind == "rms" else 8) * M


def main_bwd_kernel_name(w, plan):
    """The backward's main kernel for the planned call."""
    import row_normalization_norm_amd as rn
    if plan.path == rn.NORM_PATH_CLUSTER:
        return "bwd_cluster_kernel"
    if plan.path == rn.NORM_PATH_ROWS:
        return "bwd_pipe_kernel" if plan.pipelined else "bwd_rows_kernel"
    return "bwd_grows_kernel" if plan.vecs_per_lane else "colslice_kernel"


def elem_bytes(dtype):
    return 4 if dtype == "f32" else 2


def lib_dtype(w):
    """The library's dtype code for a workload (activations, and gamma/beta if different)."""
    import row_normalization_norm_amd as rn
    code = {"f32": rn.NORM_DTYPE_F32, "bf16": rn.NORM_DTYPE_BF16, "f16": rn.NORM_DTYPE_F16}
    if w.pdtype and w.pdtype != w.dtype:
        return rn.dtype_mixed(code[w.dtype], code[w.pdtype])
    return code[w.dtype]


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "row_normalization_norm_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def describe(w):
    dist = f"N({w.x_mean:g},{w.x_std:g})"
    types = w.dtype if not w.pdtype else f"{w.dtype} (gamma/beta {w.pdtype})"
    if w.outlier_p:
        dist += f" with {w.outlier_p:.0%} of entries x{w.outlier_scale:g}"
    kind = "RMSNorm" if w.kind == "rms" else "LayerNorm"
    return f"{kind} fwd+bwd x[{w.M},{w.N}] {types} {dist}, eps={w.eps:g}"


def to_device(a, dtype, device):
    """Host array of raw bits (uint16 bf16, float16, float32) -> device tensor, bit-exact."""
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    elif dtype == "f16":
        t = torch.from_numpy(a.view(np.float16))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


class Bench:
    """Device buffers (rotating sets when one set would fit in the MALL) for a workload."""

    def __init__(self, w, device, fused=False):
        import torch
        import gen
        import row_normalization_norm_amd as rn
        self.w, self.device, self.rn, self.fused = w, device, rn, fused
        t0 = time.time()
        inputs = gen.make_inputs(w, residual=fused)
        s = elem_bytes(w.dtype)
        per_set = (7 if fused else 4) * w.M * w.N * s  # x, y, dy, dx (+ res, sum, dsum)
        self.sets = max(1, math.ceil(2 * MALL_BYTES / per_set))
        x0 = to_device(inputs["x"], w.dtype, device)
        dy0 = to_device(inputs["dy"], w.dtype, device)
        self.gamma = to_device(inputs["gamma"], w.param_dtype, device)
        self.beta = to_device(inputs["beta"], w.param_dtype, device) if w.kind == "ln" else None
        self.bufs = []
        for i in range(self.sets):
            x = x0 if i == 0 else x0.clone()
            dy = dy0 if i == 0 else dy0.clone()
            self.bufs.append(dict(
                x=x, dy=dy, y=torch.empty_like(x), dx=torch.empty_like(x),
                mean=torch.empty(w.M, device=device) if w.kind == "ln" else None,
                rstd=torch.empty(w.M, device=device)))
            if fused:
                self.bufs[-1].update(res=to_device(inputs["res"], w.dtype, device),
                                     dsum=to_device(inputs["dsum"], w.dtype, device),
                                     sum=torch.empty_like(x))
        self.dgamma = torch.empty(w.N, device=device)
        self.dbeta = torch.empty(w.N, device=device) if w.kind == "ln" else None
        dt = lib_dtype(w)
        ws = rn.norm_bwd_workspace_size(w.M, w.N, w.kind == "ln", dt)
        self.ws = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)
        fws = rn.norm_fwd_workspace_size(w.M, w.N, w.kind == "ln", dt)
        self.fws = torch.empty(fws, dtype=torch.uint8, device=device) if fws else None
        torch.cuda.synchronize()
        self.setup_s = time.time() - t0

    def step(self, k, fwd_opt=None, bwd_opt=None, bwd_events=None):
        """One forward + backward on buffer set k; with bwd_events = (e0, e1), events
        recorded on the launch stream just before and just after the backward call."""
        self.forward(k, fwd_opt)
        if bwd_events:
            bwd_events[0].record()
        self.backward(k, bwd_opt)
        if bwd_events:
            bwd_events[1].record()

    def forward(self, k, opt=None):
        rn, w, b = self.rn, self.w, self.bufs[k % self.sets]
        if self.fused:
            if w.kind == "rms":
                rn.norm_rms_fwd_add(b["x"], b["res"], self.gamma, b["y"], b["sum"], b["rstd"],
                                    eps=w.eps, workspace=self.fws, options=opt)
            else:
                rn.norm_ln_fwd_add(b["x"], b["res"], self.gamma, self.beta, b["y"], b["sum"],
                                   b["mean"], b["rstd"], eps=w.eps, workspace=self.fws,
                                   options=opt)
        elif w.kind == "rms":
            rn.norm_rms_fwd(b["x"], self.gamma, b["y"], b["rstd"], eps=w.eps, workspace=self.fws,
                            options=opt)
        else:
            rn.norm_ln_fwd(b["x"], self.gamma, self.beta, b["y"], b["mean"], b["rstd"], eps=w.eps,
                           workspace=self.fws, options=opt)

    def backward(self, k, opt=None):
        rn, w, b = self.rn, self.w, self.bufs[k % self.sets]
        if self.fused:
            if w.kind == "rms":
                rn.norm_rms_bwd_add(b["dy"], b["sum"], self.gamma, b["rstd"], b["dsum"], b["dx"],
                                    self.dgamma, workspace=self.ws, options=opt)
            else:
                rn.norm_ln_bwd_add(b["dy"], b["sum"], self.gamma, b["mean"], b["rstd"], b["dsum"],
                                   b["dx"], self.dgamma, self.dbeta, workspace=self.ws,
                                   options=opt)
        elif w.kind == "rms":
            rn.norm_rms_bwd(b["dy"], b["x"], self.gamma, b["rstd"], b["dx"], self.dgamma,
                            workspace=self.ws, options=opt)
        else:
            rn.norm_ln_bwd(b["dy"], b["x"], self.gamma, b["mean"], b["rstd"], b["dx"], self.dgamma,
                           self.dbeta, workspace=self.ws, options=opt)

def make_events(n):
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    s = torch.cuda.current_stream()
    for e in evs:
        e.record(s)  # create the underlying HIP event so its handle can be passed down
    torch.cuda.synchronize()
    return evs


def run_gpu(w, steps, warmup, device, fused=False, warmup_s=0.0):
    """Two timed passes of `steps` steps each, after `warmup` untimed steps:
    pass A records events only before and after the K steps (the step time); pass B also
    records HIP events around every launch of the forward kernel and of the backward's
    main kernel on the stream they run on (per-kernel average durations).  Per-launch
    events add a few microseconds of gap each, which is why the step time comes from A."""
    import torch
    import row_normalization_norm_amd as rn
    b = Bench(w, device, fused)
    # `warmup` steps, continued (when warmup_s is set) until that much wall time has gone
    # by: on MI355X the first tens of milliseconds of sustained traffic run slower than
    # the steady state (DEFAULT_WARMUP_S)
    t0 = time.perf_counter()
    k = 0
    while k < warmup or time.perf_counter() - t0 < warmup_s:
        b.step(k)
        k += 1
        if k % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warmup = k

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
    cev = make_events(2 * steps)
    fopts = [rn.Options(ev_start=fev[2 * i].cuda_event, ev_stop=fev[2 * i + 1].cuda_event)
             for i in range(steps)]
    bopts = [rn.Options(ev_start=bev[2 * i].cuda_event, ev_stop=bev[2 * i + 1].cuda_event)
             for i in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        b.step(warmup + steps + k, fopts[k], bopts[k], (cev[2 * k], cev[2 * k + 1]))
    torch.cuda.synchronize()
    fwd_ms = sum(fev[2 * i].elapsed_time(fev[2 * i + 1]) for i in range(steps)) / steps
    bwd_ms = sum(bev[2 * i].elapsed_time(bev[2 * i + 1]) for i in range(steps)) / steps
    call_ms = sum(cev[2 * i].elapsed_time(cev[2 * i + 1]) for i in range(steps)) / steps
    return dict(ms_per_step=total_ms / steps, fwd_kernel_ms=fwd_ms, bwd_main_kernel_ms=bwd_ms,
                bwd_call_ms=call_ms, wall_s=wall, sets=b.sets, setup_s=b.setup_s,
                warmup_steps=warmup)


def workload_by_name(name):
    """A named workload, or a sweep point written sweep_{rms|ln}_{bf16|f32}_N{N}."""
    import gen
    if name in gen.WORKLOADS:
        return gen.WORKLOADS[name]
    parts = name.split("_")
    if len(parts) == 4 and parts[0] == "sweep" and parts[1] in ("rms", "ln") and \
            parts[2] in ("bf16", "f32", "f16") and parts[3].startswith("N") and parts[3][1:].isdigit():
        return gen.sweep_workload(parts[1], parts[2], int(parts[3][1:]))
    raise SystemExit(f"unknown workload {name!r}")


def graph_step_ms(w, device, fused=False, replays=20):
    """Step time with the host out of the loop: one step per rotating buffer set captured
    into a HIP graph (torch.cuda.graph), replayed `replays` times."""
    import torch
    b = Bench(w, device, fused)
    for k in range(b.sets):
        b.step(k)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(b.sets):
            b.step(k)
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / (replays * b.sets)


def stream_reference_ms(nbytes, device, two_reads=False, reps=10):
    """The library's streaming reference kernel over nbytes per stream (copy: read a,
    write d; two_reads: read a and b, write d), with rotating buffers so that the working
    set is at least twice the MALL: the achievable time for moving the forward's (copy)
    or the backward's (two reads, one write) element bytes at this size."""
    import torch
    import row_normalization_norm_amd as rn
    nbytes = (nbytes + 15) // 16 * 16
    streams = 3 if two_reads else 2
    sets = max(1, math.ceil(2 * MALL_BYTES / (streams * nbytes)))
    bufs = [[torch.empty(nbytes, dtype=torch.uint8, device=device).fill_(1)
             for _ in range(streams)] for _ in range(sets)]

    def run(bs):
        rn.norm_stream_reference(1 if two_reads else 0, bs[0], bs[1] if two_reads else None,
                                 bs[-1])

    for bs in bufs:
        run(bs)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        for bs in bufs:
            run(bs)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / (reps * sets)
    del bufs
    torch.cuda.empty_cache()
    return ms


def host_overhead(w, device, calls=2000):
    """Host time per call, in microseconds, of the workload's forward, backward and step
    through the binding and through bare ctypes calls with the arguments prepared, one
    buffer set (so the GPU keeps up at small sizes): (host-only time, time to the GPU's
    end) per entry.  The binding's share is the difference."""
    import torch
    import row_normalization_norm_amd as rn
    b = Bench(w, device)
    k = b.bufs[0]
    L = rn.lib()
    ln = w.kind == "ln"
    code = lib_dtype(w)
    st = torch.cuda.current_stream().cuda_stream
    p = lambda t: None if t is None else t.data_ptr()
    fws = (p(b.fws), 0 if b.fws is None else b.fws.numel())
    bws = (b.ws.data_ptr(), b.ws.numel())
    if ln:
        fa = (p(k["x"]), p(b.gamma), p(b.beta), p(k["y"]), p(k["mean"]), p(k["rstd"]), w.M, w.N,
              w.eps, code) + fws + (st,)
        ba = (p(k["dy"]), p(k["x"]), p(b.gamma), p(k["mean"]), p(k["rstd"]), p(k["dx"]),
              p(b.dgamma), p(b.dbeta), w.M, w.N, code) + bws + (st,)
        cf, cb = (lambda: L.norm_ln_fwd(*fa)), (lambda: L.norm_ln_bwd(*ba))
    else:
        fa = (p(k["x"]), p(b.gamma), p(k["y"]), p(k["rstd"]), w.M, w.N, w.eps, code) + fws + (st,)
        ba = (p(k["dy"]), p(k["x"]), p(b.gamma), p(k["rstd"]), p(k["dx"]), p(b.dgamma), w.M, w.N,
              code) + bws + (st,)
        cf, cb = (lambda: L.norm_rms_fwd(*fa)), (lambda: L.norm_rms_bwd(*ba))

    def timed(fn):
        for _ in range(50):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(calls):
            fn()
        t1 = time.perf_counter()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        return [round((t1 - t0) / calls * 1e6, 2), round((t2 - t0) / calls * 1e6, 2)]

    return {"workload": w.name, "calls": calls,
            "binding_fwd": timed(lambda: b.forward(0)),
            "binding_bwd": timed(lambda: b.backward(0)),
            "binding_step": timed(lambda: b.step(0)),
            "ctypes_fwd": timed(cf), "ctypes_bwd": timed(cb),
            "ctypes_step": timed(lambda: (cf(), cb()))}


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
    dx, and dgamma/dbeta over the sampled rows.  Reported in the metric's unit.  The sample
    grows until one pass takes about a quarter of target_s; when the whole workload is
    faster than that, whole passes repeat until that much time has gone by."""
    import gen
    import oracle
    orc = oracle.get()

    def one_pass(inp):
        if w.kind == "rms":
            orc.rms_fwd(inp["x"], inp["gamma"], w.eps)
            orc.rms_bwd_dx(inp["dy"], inp["x"], inp["gamma"], w.eps)
            orc.rms_dgamma(inp["dy"], inp["x"], w.eps)
        else:
            orc.ln_fwd(inp["x"], inp["gamma"], inp["beta"], w.eps)
            orc.ln_bwd_dx(inp["dy"], inp["x"], inp["gamma"], w.eps)
            orc.ln_dgamma_dbeta(inp["dy"], inp["x"], w.eps)

    rows = 64
    while True:
        inp = gen.make_inputs(w.scaled(rows))
        t0 = time.perf_counter()
        one_pass(inp)
        dt = time.perf_counter() - t0
        if dt >= target_s / 4 or rows >= w.M:
            break
        rows = min(w.M, int(rows * max(2.0, target_s / max(dt, 1e-3))))
    passes = 1
    while dt * passes < target_s / 4:
        t0 = time.perf_counter()
        one_pass(inp)
        dt = (dt * passes + time.perf_counter() - t0) / (passes + 1)
        passes += 1
    f, bwd = ideal_bytes(w.kind, rows, w.N, elem_bytes(w.dtype), elem_bytes(w.param_dtype))
    return {"value": round((f + bwd) / dt / 1e9, 3), "unit": "GB/s", "cores": orc.num_threads(),
            "kind": "oracle",
            "sample": f"first {rows} of {w.M} rows of the same workload (fp64 C oracle, "
                      f"forward + dx + dgamma/dbeta), {passes} pass(es) of {dt:.2f} s"}


def dgamma_compare(w, device, reps=5):
    """The backward call with each way of reducing dgamma/dbeta over the rows: the two-stage
    reduction (per-workgroup partial rows, then the column-reduce kernel) on the tuned plan
    and on the atomic variants' own mapping, against fp32 atomicAdd of every row's
    contribution (ATOMIC_ROW, M*N adds per output vector) and of one partial per workgroup
    (ATOMIC_WG, grid*N adds).  Each variant is timed over `reps` calls per rotating buffer
    set (HIP events around the calls, so the atomic variants' zero fill is included), after
    one forward per set has saved the statistics.  Also reports how far each variant's
    dgamma is from the tuned two-stage result."""
    import torch
    import row_normalization_norm_amd as rn
    b = Bench(w, device)
    for k in range(b.sets):
        b.step(k)
    torch.cuda.synchronize()
    dt = lib_dtype(w)
    ln = w.kind == "ln"
    s, ps = elem_bytes(w.dtype), elem_bytes(w.param_dtype)
    _, bwd_b = ideal_bytes(w.kind, w.M, w.N, s, ps)
    apl = rn.norm_plan(True, ln, w.M, w.N, dt,
                       options=rn.Options(dgamma_mode=rn.NORM_DGAMMA_ATOMIC_WG))
    variants = [
        ("two_stage", None),
        ("two_stage_same_mapping", rn.Options(path=rn.NORM_PATH_ROWS,
                                              lanes_per_row=apl.lanes_per_row,
                                              vecs_per_lane=apl.vecs_per_lane, grid=apl.grid)),
        ("atomic_wg", rn.Options(dgamma_mode=rn.NORM_DGAMMA_ATOMIC_WG)),
        ("atomic_row", rn.Options(dgamma_mode=rn.NORM_DGAMMA_ATOMIC_ROW)),
    ]

    def bwd(buf, opt, ws):
        if ln:
            rn.norm_ln_bwd(buf["dy"], buf["x"], b.gamma, buf["mean"], buf["rstd"], buf["dx"],
                           b.dgamma, b.dbeta, workspace=ws, options=opt)
        else:
            rn.norm_rms_bwd(buf["dy"], buf["x"], b.gamma, buf["rstd"], buf["dx"], b.dgamma,
                            workspace=ws, options=opt)

    # warm the device up first (sustained traffic for 0.3 s), so that the first variant
    # timed is not measured before the steady state
    ws0 = torch.empty(max(rn.norm_bwd_workspace_size(w.M, w.N, ln, dt), 1), dtype=torch.uint8,
                      device=device)
    t0 = time.perf_counter()
    k = 0
    while time.perf_counter() - t0 < 0.3:
        bwd(b.bufs[k % b.sets], None, ws0)
        k += 1
        if k % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    del ws0
    rows, ref = [], None
    for name, opt in variants:
        pl = rn.norm_plan(True, ln, w.M, w.N, dt, options=opt)
        need = rn.norm_bwd_workspace_size(w.M, w.N, ln, dt, opt)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
        bwd(b.bufs[0], opt, ws)  # warm-up
        torch.cuda.synchronize()
        dg = b.dgamma.clone()
        db = b.dbeta.clone() if ln else None
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            for buf in b.bufs:
                bwd(buf, opt, ws)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / (reps * b.sets)
        if ref is None:
            ref = (dg, db)

        def rel(a, r):
            return float(((a - r).abs().max() / r.abs().max().clamp_min(1e-30)).item())

        row = {"variant": name, "ms": round(ms, 5), "GBs": round(bwd_b / (ms * 1e-3) / 1e9, 1),
               "mapping": f"{pl.lanes_per_row}x{pl.vecs_per_lane}, grid {pl.grid}",
               "atomic_adds_per_output_vector": (w.M if name == "atomic_row" else
                                                 pl.grid if name == "atomic_wg" else 0) * w.N,
               "dgamma_max_rel_diff_vs_two_stage": rel(dg, ref[0])}
        if ln:
            row["dbeta_max_rel_diff_vs_two_stage"] = rel(db, ref[1])
        rows.append(row)
        del ws
    del b
    return {"workload": w.name, "desc": describe(w), "variants": rows}


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _short(name):
    name = name.replace("rownorm::(anonymous namespace)::", "").replace("rownorm::", "")
    return name[5:] if name.startswith("void ") else name


def summarize(d, workload, warmup, steps, copy_bytes):
    """Turn the rocprofv3 outputs of one profiling session into the text summaries kept
    under profiles/ and the counter file the benchmark reads.  Layout of d (each a
    rocprofv3 -d directory): trace/<w>_kernel_trace.csv (--kernel-trace),
    FETCH_SIZE/<w>_counter_collection.csv and WRITE_SIZE/... (--pmc on this benchmark),
    FETCH_SIZE_copy/copy_counter_collection.csv and WRITE_SIZE_copy/... (--pmc on
    --copy-probe copy_bytes), LDS/<w>_counter_collection.csv (LDS counters), and the
    benchmark's own stdout for the FETCH_SIZE run in FETCH_SIZE.log (source hash)."""
    import statistics
    w = workload
    out_dir = os.path.join(ROOT, "profiles")
    lines = []
    # kernel trace
    tr = _read_csv(os.path.join(d, "trace", f"{w}_kernel_trace.csv"))
    per = {}
    for r in sorted(tr, key=lambda r: int(r["Start_Timestamp"])):
        per.setdefault(_short(r["Kernel_Name"]), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines.append("| kernel | calls | avg us (all) | warm-up avg | pass A avg (back to back) | "
                 "pass B avg (per-launch events) | min us | max us |")
    lines.append("|---|---|---|---|---|---|---|---|")
    trace_avg = {}
    for k, v in per.items():
        if len(v) == warmup + 2 * steps:
            ph = [v[:warmup], v[warmup:warmup + steps], v[warmup + steps:]]
            phs = " | ".join(f"{statistics.fmean(p):.1f}" for p in ph)
            trace_avg[k] = statistics.fmean(ph[2])
        else:
            phs = "- | - | -"
        lines.append(f"| `{k}` | {len(v)} | {statistics.fmean(v):.1f} | {phs} | "
                     f"{min(v):.1f} | {max(v):.1f} |")
    trace_table = "\n".join(lines)

    def counter(sub, fname, name):
        vals = {}
        for r in _read_csv(os.path.join(d, sub, fname)):
            if r["Counter_Name"] == name:
                vals.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        return {k: statistics.median(v) for k, v in vals.items()}

    fetch = counter("FETCH_SIZE", f"{w}_counter_collection.csv", "FETCH_SIZE")
    write = counter("WRITE_SIZE", f"{w}_counter_collection.csv", "WRITE_SIZE")
    cf = max(counter("FETCH_SIZE_copy", "copy_counter_collection.csv", "FETCH_SIZE").values())
    cw = max(counter("WRITE_SIZE_copy", "copy_counter_collection.csv", "WRITE_SIZE").values())
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    lds = {}
    lds_path = os.path.join(d, "LDS", f"{w}_counter_collection.csv")
    if os.path.exists(lds_path):
        for name in ("SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT"):
            for k, v in counter("LDS", f"{w}_counter_collection.csv", name).items():
                lds.setdefault(k, {})[name] = v
    import gen
    wl = workload_by_name(w)
    s, ps = elem_bytes(wl.dtype), elem_bytes(wl.param_dtype)
    fwd_b, bwd_b = ideal_bytes(wl.kind, wl.M, wl.N, s, ps)
    main_b = main_bwd_kernel_bytes(wl.kind, wl.M, wl.N, s, ps)
    algo = {"fwd_rows_kernel": fwd_b, "bwd_rows_kernel": main_b,
            "fwd_pipe_kernel": fwd_b, "bwd_pipe_kernel": main_b,
            "fwd_cluster_kernel": fwd_b, "bwd_cluster_kernel": main_b,
            "colreduce_kernel": bwd_b - main_b}
    clines = ["| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | bytes read | bytes written | "
              "traffic | algorithmic | traffic / algorithmic | LDS instr | LDS bank conflicts |",
              "|---|---|---|---|---|---|---|---|---|---|"]
    bwd_traffic = None
    for k in fetch:
        if "rocclr" in k or k not in write:
            continue
        rb, wb = fetch[k] * 1024 * f_scale, write[k] * 1024 * w_scale
        a = next((v for n, v in algo.items() if k.startswith(n)), None)
        if k.startswith("bwd_rows_kernel") or k.startswith("bwd_pipe_kernel"):
            bwd_traffic = rb + wb
        li = lds.get(k, {})
        clines.append(f"| `{k}` | {fetch[k]:.0f} | {write[k]:.0f} | {rb:.4g} | {wb:.4g} | "
                      f"{rb + wb:.4g} | {a if a else '-'} | "
                      f"{(rb + wb) / a if a else float('nan'):.4f} | "
                      f"{li.get('SQ_INSTS_LDS', float('nan')):.0f} | "
                      f"{li.get('SQ_LDS_BANK_CONFLICT', float('nan')):.0f} |")
    src_hash = None
    log = os.path.join(d, f"FETCH_SIZE_{w}.log")
    if not os.path.exists(log):
        log = os.path.join(d, "FETCH_SIZE.log")
    if os.path.exists(log):
        for line in open(log):
            if line.startswith("{"):
                src_hash = json.loads(line).get("kernel_source_hash")
    return trace_table, trace_avg, "\n".join(clines), f_scale, w_scale, bwd_traffic, src_hash


PROFILE_STEPS = (
    "cd /tmp && export TMPDIR=/tmp; R=/root/repo; D=${{PROF_OUT:-$R/prof_out}}; mkdir -p $D",
    "rocprofv3 --kernel-trace --stats --output-format csv -d $D/trace -o {w} -- "
    "python3 $R/bench.py --workload {w} --no-cpu > $D/trace_{w}.log",
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $D/FETCH_SIZE -o {w} -- "
    "python3 $R/bench.py --workload {w} --steps 3 --warmup 1 --warmup-time 0 --no-cpu > $D/FETCH_SIZE_{w}.log",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $D/WRITE_SIZE -o {w} -- "
    "python3 $R/bench.py --workload {w} --steps 3 --warmup 1 --warmup-time 0 --no-cpu",
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $D/FETCH_SIZE_copy -o copy -- "
    "python3 $R/bench.py --copy-probe {c} --steps 3",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $D/WRITE_SIZE_copy -o copy -- "
    "python3 $R/bench.py --copy-probe {c} --steps 3",
    "rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS --output-format csv -d $D/LDS -o {w} -- "
    "python3 $R/bench.py --workload {w} --steps 3 --warmup 1 --warmup-time 0 --no-cpu",
    "python3 $R/bench.py --summarize $D --workload {w}",
)


def traced_run_counts(d, w, warmup, steps):
    """The warm-up and timed step counts of the traced run, from the JSON line it printed
    (trace_<w>.log beside the trace directory; the warm-up runs for a minimum time, so
    its step count varies), else the defaults."""
    log = os.path.join(d, f"trace_{w}.log")
    if os.path.exists(log):
        with open(log) as f:
            for line in f:
                if line.startswith("{") and '"warmup_steps_run"' in line:
                    j = json.loads(line)
                    return j["warmup_steps_run"], j["steps"]
    return warmup, steps


def write_summaries(d, w, warmup=DEFAULT_WARMUP, steps=DEFAULT_STEPS, copy_bytes=1 << 30):
    """--summarize: write profiles/<w>_kernel_trace.md, profiles/<w>_hbm_counters.md and
    (for the benchmark's own workload) the counter file bench.py reports traffic from."""
    warmup, steps = traced_run_counts(d, w, warmup, steps)
    tt, tavg, ct, fs, ws_, bwd_traffic, src_hash = summarize(d, w, warmup, steps, copy_bytes)
    cmds = "\n".join(c.format(w=w, c=copy_bytes) for c in PROFILE_STEPS)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"{w}_kernel_trace.md"), "w") as f:
        f.write(f"# Kernel durations, workload {w} (rocprofv3 --kernel-trace --stats)\n\n"
                f"Commands (the whole profiling session; this file comes from the first):\n\n"
                f"```\n{cmds}\n```\n\n{tt}\n\n"
                f"Kernel source hash: `{src_hash}`. The profiled run makes {warmup} warm-up "
                f"steps, then pass A ({steps} steps launched back to back: the step time) "
                f"and pass B ({steps} steps with HIP events recorded around each launch: "
                f"the per-kernel time bench.py reports as avg_launch_ms).\n")
    with open(os.path.join(ROOT, "profiles", f"{w}_hbm_counters.md"), "w") as f:
        f.write(f"# HBM traffic and LDS counters, workload {w} (rocprofv3 --pmc)\n\n"
                f"Commands:\n\n```\n{cmds}\n```\n\n"
                f"Counter scale from a {copy_bytes} B device copy: FETCH_SIZE x{fs:.4f}, "
                f"WRITE_SIZE x{ws_:.4f} (bytes = KiB x 1024 x scale). Values are the median "
                f"over the run's dispatches of each kernel.\n\n{ct}\n\n"
                f"Kernel source hash: `{src_hash}`.\n")
    if w == DEFAULT_WORKLOAD and bwd_traffic:
        with open(COUNTERS_FILE, "w") as f:
            import row_normalization_norm_amd as rn
            wl = workload_by_name(w)
            plan = rn.norm_plan(True, wl.kind == "ln", wl.M, wl.N, lib_dtype(wl))
            json.dump({"workload": w, "kernel": main_bwd_kernel_name(wl, plan),
                       "kernel_source_hash": src_hash,
                       "traffic_bytes_per_launch": round(bwd_traffic),
                       "fetch_scale": round(fs, 4), "write_scale": round(ws_, 4),
                       "trace_avg_us_pass_b": {k: round(v, 2) for k, v in tavg.items()}},
                      f, indent=1)
            f.write("\n")


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
    ap.add_argument("--steps", type=int, default=DEFAULT_STEPS)
    ap.add_argument("--warmup", type=int, default=DEFAULT_WARMUP)
    ap.add_argument("--warmup-time", type=float, default=DEFAULT_WARMUP_S, metavar="SECONDS",
                    help="after the --warmup steps, keep stepping (untimed) until this much "
                         "wall time has gone by (0: exactly --warmup steps)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-only", action="store_true",
                    help="only time the oracle CPU baseline of --workload (no GPU needed)")
    ap.add_argument("--cpu-threads", type=int, metavar="T",
                    help="host threads for the oracle (default: OpenMP's, all cores)")
    ap.add_argument("--all", metavar="JSON", help="also time every workload, write a table")
    ap.add_argument("--copy-probe", type=int, metavar="BYTES",
                    help="only time a plain device copy of BYTES and print it")
    ap.add_argument("--host-overhead", action="store_true",
                    help="only time the host side of --workload's calls (binding and bare "
                         "ctypes, microseconds per call) and print it")
    ap.add_argument("--stream-reference", type=int, metavar="BYTES",
                    help="only time the streaming reference kernel (copy, then two reads "
                         "and one write) over BYTES per stream, --steps launches per "
                         "rotating buffer set, and print it")
    ap.add_argument("--dgamma-compare", metavar="JSON",
                    help="only time the backward with the two-stage and the atomic dgamma "
                         "reductions on rms1, ln2, rms3 and sweep points up to N=8192, "
                         "write a table")
    ap.add_argument("--summarize", metavar="DIR",
                    help="only write the profiles/ summaries from a profiling session in DIR")
    args = ap.parse_args()
    if args.summarize:
        write_summaries(args.summarize, args.workload)
        return
    if args.cpu_threads:
        # read by the OpenMP runtime when the oracle library is loaded
        os.environ["OMP_NUM_THREADS"] = str(args.cpu_threads)
    if args.cpu_only:
        out = cpu_baseline(workload_by_name(args.workload))
        out["workload"] = args.workload
        print(json.dumps(out), flush=True)
        return

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
    if args.host_overhead:
        print(json.dumps(host_overhead(workload_by_name(args.workload), device)), flush=True)
        return

    if args.stream_reference:
        nb = args.stream_reference
        out = {"bytes_per_stream": nb}
        for key, two in (("copy", False), ("two_reads_one_write", True)):
            ms = stream_reference_ms(nb, device, two_reads=two, reps=args.steps)
            moved = (3 if two else 2) * ((nb + 15) // 16 * 16)
            out[key] = {"us_per_launch": round(ms * 1e3, 3),
                        "GBs": round(moved / (ms * 1e-3) / 1e9, 1)}
        print(json.dumps(out), flush=True)
        return

    if args.dgamma_compare:
        import gc
        names = ["rms1", "ln2", "rms3"] + [f"sweep_{k}_bf16_N{n}" for k in ("rms", "ln")
                                           for n in (1024, 4096, 8192)]
        res = []
        for name in names:
            gc.collect()
            torch.cuda.empty_cache()
            res.append(dgamma_compare(workload_by_name(name), device))
            print("# " + name + ": " + ", ".join(f"{v['variant']} {v['GBs']:.0f} GB/s"
                                                 for v in res[-1]["variants"]),
                  file=sys.stderr, flush=True)
        with open(args.dgamma_compare, "w") as f:
            json.dump(res, f, indent=1)
        return

    w = workload_by_name(args.workload)
    s, ps = elem_bytes(w.dtype), elem_bytes(w.param_dtype)
    fwd_b, bwd_b = ideal_bytes(w.kind, w.M, w.N, s, ps)
    r = run_gpu(w, args.steps, args.warmup, device, warmup_s=args.warmup_time)
    value = (fwd_b + bwd_b) / (r["ms_per_step"] * 1e-3) / 1e9

    main_bytes = main_bwd_kernel_bytes(w.kind, w.M, w.N, s, ps)
    achieved = main_bytes / (r["bwd_main_kernel_ms"] * 1e-3) / 1e9
    plan = rn.norm_plan(True, w.kind == "ln", w.M, w.N, lib_dtype(w))
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": r["warmup_steps"],
        "warmup_min_s": args.warmup_time,
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
        "bwd_call_GBs": round(bwd_b / (r["bwd_call_ms"] * 1e-3) / 1e9, 1),
        "roofline": {
            "bound": "hbm",
            "kernel": f"{main_bwd_kernel_name(w, plan)} (dx + dgamma/dbeta partials), "
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
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w)
    if args.all:
        table = []
        import dataclasses
        sweep = [gen.sweep_workload(k, d, n) for k in ("rms", "ln") for d in ("bf16", "f32")
                 for n in gen.SWEEP_N]
        # the benchmark workload with fp16 activations and with fp32 gamma/beta
        other = [dataclasses.replace(gen.WORKLOADS[DEFAULT_WORKLOAD], dtype=d, pdtype=p,
                                     name=f"{DEFAULT_WORKLOAD}_{d}" + (f"_{p}" if p else ""))
                 for d, p in (("f16", None), ("bf16", "f32"), ("f16", "f32"))]
        fused_names = set()
        fused = []
        for base in (DEFAULT_WORKLOAD, "rms1"):
            f = dataclasses.replace(gen.WORKLOADS[base], name=f"{base}_residual_add")
            fused.append(f)
            fused_names.add(f.name)
        import gc
        import torch
        for wl in list(gen.WORKLOADS.values()) + other + fused + sweep:
            name = wl.name
            is_fused = name in fused_names
            # release the previous workload's buffers, so each starts from the same
            # (empty) caching-allocator state
            gc.collect()
            torch.cuda.empty_cache()
            rr = run_gpu(wl, max(5, args.steps // 2), 10, device, fused=is_fused, warmup_s=0.3)
            es = elem_bytes(wl.dtype)
            fb, bb = ideal_bytes(wl.kind, wl.M, wl.N, es, elem_bytes(wl.param_dtype))
            if is_fused:  # + read residual, write sum; + read dsum
                fb, bb = fb + 2 * wl.M * wl.N * es, bb + wl.M * wl.N * es
            table.append({"workload": name,
                          "desc": describe(wl) + (", residual add fused" if is_fused else ""),
                          **{k: round(v, 5) for k, v in rr.items()},
                          "fwd_GBs": fb / (rr["fwd_kernel_ms"] * 1e-3) / 1e9,
                          "bwd_GBs": bb / ((rr["ms_per_step"] - rr["fwd_kernel_ms"]) * 1e-3) / 1e9,
                          "bwd_call_GBs": bb / (rr["bwd_call_ms"] * 1e-3) / 1e9,
                          "step_GBs": (fb + bb) / (rr["ms_per_step"] * 1e-3) / 1e9})
            # the streaming reference at the forward's (1 read + 1 write of M*N elements)
            # and the backward's (2 reads + 1 write) element bytes
            nb = wl.M * wl.N * es
            cms = stream_reference_ms(nb, device)
            tms = stream_reference_ms(nb, device, two_reads=True)
            table[-1].update(copy_ms=round(cms, 5), copy_GBs=2 * nb / (cms * 1e-3) / 1e9,
                             two_read_ms=round(tms, 5), two_read_GBs=3 * nb / (tms * 1e-3) / 1e9)
            if rr["ms_per_step"] < 0.1:
                # launch-bound: also the step replayed from a captured graph
                gms = graph_step_ms(wl, device, fused=is_fused)
                table[-1]["graph_ms_per_step"] = round(gms, 5)
                table[-1]["graph_step_GBs"] = (fb + bb) / (gms * 1e-3) / 1e9
            print(f"# {name}: {table[-1]['step_GBs']:.0f} GB/s", file=sys.stderr, flush=True)
        with open(args.all, "w") as f:
            json.dump(table, f, indent=1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
