"""Measure every compiled (path, mapping, grid) on the current GPU and write the planner
table (csrc/tuned.h) from the results.

    python -m row_normalization_norm_amd.tune --sweep sweep.jsonl      # on the GPU
    python -m row_normalization_norm_amd.tune --table sweep.jsonl > csrc/tuned.h

The sweep covers the benchmark's shape sweep: RMSNorm and LayerNorm, bf16 and fp32,
forward and backward, N in 256 ... 65536 with M = 2^27 / N rows.  For each shape it
times every register-resident (ROWS) mapping that covers the row with less than one
vector of waste per lane, at several grids, and (for rows longer than 1024 vectors)
every split-row (CLUSTER) configuration that fits on the device.  Inputs are random
device tensors (timing only); throughput is algorithmic bytes / time.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SWEEP_N = (256, 384, 512, 768, 1024, 2048, 4096, 8192, 16384, 32768, 65536)
CL_FWD = [(256, 1, 1), (256, 2, 1), (256, 4, 1), (512, 1, 1), (512, 2, 1), (512, 4, 1),
          (1024, 1, 1), (1024, 2, 1), (1024, 4, 1), (256, 1, 2), (256, 2, 2), (512, 1, 2),
          (512, 2, 2), (1024, 1, 2), (1024, 2, 2)]
CL_BWD = [(256, 1, 1), (256, 2, 1), (512, 1, 1), (512, 2, 1), (1024, 1, 1), (1024, 2, 1),
          (256, 1, 2), (512, 1, 2), (1024, 1, 2), (256, 2, 2), (512, 2, 2)]


def mappings(direction):
    """(lanes, vectors) pairs compiled for the ROWS kernels, read from launch.h."""
    with open(os.path.join(HERE, "csrc", "launch.h")) as f:
        src = f.read()
    macro = "RN_FWD_MAPPINGS" if direction == "fwd" else "RN_BWD_MAPPINGS"
    body = src[src.index(f"#define {macro}"):]
    body = body[:body.index("\n\n")]
    return [(int(a), int(b)) for a, b in re.findall(r"X\((\d+), (\d+)\)", body)]


def ideal_bytes(kind, M, N, s):
    if kind == "rms":
        return 2 * M * N * s + N * s + 4 * M, 3 * M * N * s + N * s + 4 * M + 4 * N
    return 2 * M * N * s + 2 * N * s + 8 * M, 3 * M * N * s + N * s + 8 * M + 8 * N


def _time(fn, iters=20, warm=3):
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def tune_shape(kind, dtype, M, N, grids_f=(0, 256, 512, 1024, -1), grids_b=(0, 256, 512, 1024),
               cluster=True, dirs=("fwd", "bwd"), refine=5):
    """Time every candidate for one shape; returns a list of result dicts.  A forward grid
    of -1 stands for one row group per workgroup (the grid recorded is that count)."""
    import torch
    import row_normalization_norm_amd as rn
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    code = rn.NORM_DTYPE_BF16 if dtype == "bf16" else rn.NORM_DTYPE_F32
    s = 2 if dtype == "bf16" else 4
    nvec = N // (16 // s)
    ln = kind == "ln"
    x = torch.randn(M, N, device=dev, dtype=tdt)
    dy = torch.randn(M, N, device=dev, dtype=tdt)
    y, dx = torch.empty_like(x), torch.empty_like(x)
    g = (1 + 0.1 * torch.randn(N, device=dev)).to(tdt)
    b = (0.1 * torch.randn(N, device=dev)).to(tdt)
    mean, rstd = torch.empty(M, device=dev), torch.empty(M, device=dev)
    dg, db = torch.empty(N, device=dev), torch.empty(N, device=dev)
    fb, bb = ideal_bytes(kind, M, N, s)
    res = []

    def run_fwd(opt, ws):
        if ln:
            rn.norm_ln_fwd(x, g, b, y, mean, rstd, workspace=ws, options=opt)
        else:
            rn.norm_rms_fwd(x, g, y, rstd, workspace=ws, options=opt)

    def run_bwd(opt, ws):
        if ln:
            rn.norm_ln_bwd(dy, x, g, mean, rstd, dx, dg, db, workspace=ws, options=opt)
        else:
            rn.norm_rms_bwd(dy, x, g, rstd, dx, dg, workspace=ws, options=opt)

    def record(direction, opt, path, lanes, vecs, grid, C=0, R=0, pipe=0):
        size = (rn.norm_bwd_workspace_size if direction == "bwd" else rn.norm_fwd_workspace_size)(
            M, N, ln, code, opt)
        ws = torch.empty(max(size, 1), dtype=torch.uint8, device=dev)
        fn = run_bwd if direction == "bwd" else run_fwd
        ms = _time(lambda: fn(opt, ws))
        res.append(dict(dir=direction, kind=kind, dtype=dtype, M=M, N=N, nvec=nvec, path=path,
                        lpr=lanes, vpl=vecs, grid=grid, C=C, R=R, pipe=pipe, ms=ms,
                        GBs=(bb if direction == "bwd" else fb) / ms / 1e6, reps=[ms], _opt=opt))

    run_fwd(None, torch.empty(max(rn.norm_fwd_workspace_size(M, N, ln, code), 1),
                              dtype=torch.uint8, device=dev))
    torch.cuda.synchronize()
    for direction, maps, grids, cl_list in (("fwd", mappings("fwd"), grids_f, CL_FWD),
                                            ("bwd", mappings("bwd"), grids_b, CL_BWD)):
        if direction not in dirs:
            continue
        bwd = direction == "bwd"
        for lanes, vecs in maps:
            if lanes * vecs < nvec or lanes * vecs - nvec >= lanes:
                continue
            rows_per_wg = (max(256, lanes) if not bwd else max(512, lanes)) // lanes
            groups = (M + rows_per_wg - 1) // rows_per_wg
            for grid in grids:
                if grid == -1:
                    grid = groups
                    if grid in grids:
                        continue
                opt = rn.Options(path=rn.NORM_PATH_ROWS, lanes_per_row=lanes, vecs_per_lane=vecs,
                                 grid=grid)
                try:
                    plan = rn.norm_plan(bwd, ln, M, N, code, options=opt)
                except rn.NormError:
                    break  # mapping not built for this kind and element width
                # a persistent grid runs either the plain or the pipelined kernel
                for pipe in ((1, 2) if plan.grid < groups else (0,)):
                    opt = rn.Options(path=rn.NORM_PATH_ROWS, lanes_per_row=lanes,
                                     vecs_per_lane=vecs, grid=grid, pipeline=pipe)
                    if pipe == 2 and not rn.norm_plan(bwd, ln, M, N, code, options=opt).pipelined:
                        continue  # no pipelined kernel for this mapping
                    record(direction, opt, rn.NORM_PATH_ROWS, lanes, vecs, grid,
                           pipe=int(pipe == 2))
        if not cluster or nvec <= 1024:
            continue
        for C in (2, 4, 8, 16, 32):
            if nvec % C:
                continue
            sv = nvec // C
            for T, V, R in cl_list:
                if T * V < sv or T * V - sv >= T:
                    continue
                base = rn.Options(path=rn.NORM_PATH_CLUSTER, cluster_size=C, lanes_per_row=T,
                                  vecs_per_lane=V, cluster_rows=R)
                g0 = rn.norm_plan(bwd, ln, M, N, code, options=base).grid
                for grid in (g0, 2 * g0):
                    opt = rn.Options(path=rn.NORM_PATH_CLUSTER, cluster_size=C, lanes_per_row=T,
                                     vecs_per_lane=V, grid=grid, cluster_rows=R)
                    if rn.norm_cluster_resident(bwd, ln, M, N, code, opt) != 1:
                        continue
                    record(direction, opt, rn.NORM_PATH_CLUSTER, T, V, grid, C, R)
    # The single timings differ by 1-2 % from run to run: re-time the best few of each
    # direction, interleaved, and rank them by the median of all their timings.
    for direction in dirs:
        top = sorted((r for r in res if r["dir"] == direction), key=lambda r: -r["GBs"])[:refine]
        for _ in range(3):
            for r in top:
                opt = r["_opt"]
                size = (rn.norm_bwd_workspace_size if direction == "bwd"
                        else rn.norm_fwd_workspace_size)(M, N, ln, code, opt)
                ws = torch.empty(max(size, 1), dtype=torch.uint8, device=dev)
                fn = run_bwd if direction == "bwd" else run_fwd
                r["reps"].append(_time(lambda: fn(opt, ws)))
        for r in top:
            r["ms"] = sorted(r["reps"])[len(r["reps"]) // 2]
            r["GBs"] = (bb if direction == "bwd" else fb) / r["ms"] / 1e6
    for r in res:
        r.pop("_opt", None)
    del x, dy, y, dx
    torch.cuda.empty_cache()
    return res


def sweep(out_path, ns=SWEEP_N, dirs=("fwd", "bwd"), kinds=("rms", "ln"), dtypes=("bf16", "f32")):
    with open(out_path, "w") as out:
        for kind in kinds:
            for dtype in dtypes:
                for N in ns:
                    res = tune_shape(kind, dtype, (1 << 27) // N, N, dirs=dirs)
                    for r in res:
                        out.write(json.dumps(r) + "\n")
                    out.flush()
                    for d in dirs:
                        best = max((r for r in res if r["dir"] == d), key=lambda r: r["GBs"])
                        print(f"{kind} {dtype} N={N} {d}: path {best['path']} "
                              f"{best['lpr']}x{best['vpl']} grid {best['grid']} C{best['C']} "
                              f"R{best['R']}: {best['GBs']:.0f} GB/s", flush=True)


def table(jsonl_paths):
    """C++ header with the fastest candidate per (direction, kind, dtype, row length).
    A shape measured in a later file is taken from that file alone (its kernels may have
    changed since the earlier measurement)."""
    best = {}
    compiled = {"fwd": set(mappings("fwd")), "bwd": set(mappings("bwd"))}
    for p in jsonl_paths:
        mine = {}
        with open(p) as f:
            for line in f:
                r = json.loads(line)
                if r.get("path", 1) == 1 and (r["lpr"], r["vpl"]) not in compiled[r["dir"]]:
                    continue  # a mapping no longer built
                nvec = r.get("nvec") or r["N"] // (8 if r["dtype"] == "bf16" else 4)
                key = (r["dir"] == "bwd", r["kind"] == "ln", r["dtype"] == "bf16", nvec)
                if key not in mine or r["GBs"] > mine[key][1]["GBs"]:
                    mine[key] = (r["N"], r)
        best.update(mine)
    lines = []
    for key in sorted(best, key=lambda k: (-k[0], -k[1], -k[2], k[3])):
        N, r = best[key]
        path = r.get("path", 1)
        lines.append(f"    {{{int(key[0])}, {int(key[1])}, {int(key[2])}, {key[3]}, {path}, "
                     f"{r['lpr']}, {r['vpl']}, {r['grid']}, {r.get('C', 0)}, {r.get('R', 0)}, "
                     f"{r.get('pipe', 0)}}},  // N={N}: {r['GBs']:.0f} GB/s")
    with open(os.path.join(HERE, "csrc", "tuned.h")) as f:
        src = f.read()
    head = src[:src.index("constexpr TunedPlan kTunedPlans[] = {") +
               len("constexpr TunedPlan kTunedPlans[] = {")]
    tail = src[src.index("};\n// clang-format on"):]
    return head + "\n" + "\n".join(lines) + "\n" + tail


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--sweep", metavar="OUT.jsonl", help="time the sweep on cuda:0")
    ap.add_argument("--n", type=int, nargs="+", default=list(SWEEP_N),
                    help="row lengths to sweep (default: all)")
    ap.add_argument("--dirs", nargs="+", default=["fwd", "bwd"], choices=["fwd", "bwd"],
                    help="directions to sweep (default: both)")
    ap.add_argument("--kinds", nargs="+", default=["rms", "ln"], choices=["rms", "ln"],
                    help="normalizations to sweep (default: both)")
    ap.add_argument("--dtypes", nargs="+", default=["bf16", "f32"], choices=["bf16", "f32"],
                    help="element types to sweep (default: both)")
    ap.add_argument("--table", metavar="IN.jsonl", nargs="+",
                    help="print csrc/tuned.h built from sweep results (a shape in a later "
                         "file replaces the earlier files' results for it)")
    args = ap.parse_args()
    if args.sweep:
        sys.path.insert(0, os.path.dirname(HERE))
        sweep(args.sweep, args.n, tuple(args.dirs), tuple(args.kinds), tuple(args.dtypes))
    elif args.table:
        sys.stdout.write(table(args.table))
    else:
        ap.print_help()


if __name__ == "__main__":
    main()
