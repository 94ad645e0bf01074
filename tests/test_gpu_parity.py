"""GPU parity: the HIP library against the fp64 oracle, element by element.

Small cases compare every row.  The named workloads at full size, and the N = 65536
sweep points, compare every row too (the oracle evaluates them a chunk of rows at a
time); the other sweep points and the other type pairs at full size compare sampled
rows.  dgamma/dbeta are always compared in full (the oracle sums all rows).
Tolerances are in parity.py.  All calls go through the C ABI.

Forced mappings and split-row sizes are listed only where the planner accepts them;
tests/test_abi.py checks on the CPU that exactly the others are rejected.
"""
import ctypes

import numpy as np
import pytest

import gen
import row_normalization_norm_amd as rn
from parity import (GpuRun, check_all_rows, check_backward, check_forward, full_check,
                    sample_rows, to_device)
import plan_cases

pytestmark = pytest.mark.gpu

SMALL_N = (1, 2, 3, 7, 64, 100, 256, 384, 512, 768, 770, 1000, 1024, 2048, 4095, 4096, 8190, 8192,
           8195, 16384, 32768, 65536, 131072)


# (activation type, parameter type or None for the same): the configurations' bf16 and
# fp32, fp16, and 16-bit activations with fp32 gamma/beta.
PAIRS = [("bf16", None), ("f32", None), ("f16", None), ("bf16", "f32"), ("f16", "f32")]
PAIR_IDS = ["bf16", "f32", "f16", "bf16+f32", "f16+f32"]
_CODE = {"f32": rn.NORM_DTYPE_F32, "bf16": rn.NORM_DTYPE_BF16, "f16": rn.NORM_DTYPE_F16}


def dtype_code(dtype, pdtype=None):
    return rn.dtype_mixed(_CODE[dtype], _CODE[pdtype]) if pdtype else _CODE[dtype]


def small_workload(kind, dtype, N, M=None, eps=1e-6, x_mean=0.0, x_std=1.0, pdtype=None):
    if M is None:
        # several row groups plus a ragged tail, within a few million elements
        M = max(3, min(1531, 3_000_000 // N))
    return gen.Workload(f"{kind}_{dtype}{'+' + pdtype if pdtype else ''}_{M}x{N}", kind, dtype, M,
                        N, eps, x_mean=x_mean, x_std=x_std, config=9, pdtype=pdtype)


@pytest.mark.parametrize("N", SMALL_N)
@pytest.mark.parametrize("dtype,pdtype", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("kind", ["rms", "ln"])
def test_small_shapes(device, kind, dtype, pdtype, N):
    w = small_workload(kind, dtype, N, x_mean=0.25 if kind == "ln" else 0.0, x_std=1.5,
                       pdtype=pdtype)
    full_check(w, device, rows=np.arange(w.M))


# Row lengths between the one-workgroup mappings' lengths (their forward used to be
# refused): 16-byte vectors 4097, 5000, 6500 and 7000, one-workgroup and split-row plans.
BETWEEN = [("rms", "bf16", 8 * 4097), ("ln", "bf16", 8 * 5000), ("ln", "bf16", 8 * 7000),
           ("rms", "f32", 4 * 6500), ("ln", "f32", 4 * 4097)]


@pytest.mark.parametrize("kind,dtype,N", BETWEEN, ids=[f"{k}-{d}-N{n}" for k, d, n in BETWEEN])
def test_row_lengths_between_mappings(device, kind, dtype, N):
    w = small_workload(kind, dtype, N, M=37, x_mean=0.2)
    code = dtype_code(dtype)
    p = rn.norm_plan(False, kind == "ln", w.M, N, code)
    assert p.path in (rn.NORM_PATH_ROWS, rn.NORM_PATH_CLUSTER)
    print(f"between mappings: {w.name} forward path {p.path} {p.lanes_per_row}x{p.vecs_per_lane}",
          flush=True)
    full_check(w, device, rows=np.arange(w.M))


def _all_rows(w, device):
    print(f"all-row parity: {w.name} [{w.M}x{w.N}] {w.dtype}", flush=True)
    inputs = gen.make_inputs(w)
    run = GpuRun(w, inputs, device)
    run.forward()
    run.backward()
    run.sync()
    check_all_rows(run, inputs)


@pytest.mark.parametrize("name", ["rms1", "ln2", "rms3", "rms4"])
def test_workloads_full_size(device, name):
    """The named workloads at full size, in the launch configuration the benchmark times,
    every element of y, dx and the statistics compared."""
    _all_rows(gen.WORKLOADS[name], device)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("kind", ["rms", "ln"])
def test_sweep_longest_rows_all_rows(device, kind, dtype):
    """The sweep's longest rows (N = 65536: split rows) with every element compared."""
    _all_rows(gen.sweep_workload(kind, dtype, 65536), device)


@pytest.mark.parametrize("dtype,pdtype", PAIRS[2:], ids=PAIR_IDS[2:])
@pytest.mark.parametrize("name", ["rms1", "ln2", "rms3", "rms4"])
def test_workloads_other_types(device, name, dtype, pdtype):
    """The named workloads' shapes and distributions with fp16 activations, or with fp32
    gamma/beta beside 16-bit activations."""
    import dataclasses
    w = dataclasses.replace(gen.WORKLOADS[name], dtype=dtype, pdtype=pdtype,
                            name=f"{name}_{dtype}_{pdtype}")
    full_check(w, device, rows=sample_rows(w.M, 32))


@pytest.mark.parametrize("N", gen.SWEEP_N)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("kind", ["rms", "ln"])
def test_sweep_full_size(device, kind, dtype, N):
    w = gen.sweep_workload(kind, dtype, N)
    full_check(w, device, rows=sample_rows(w.M, 24))


MAPPING_CASES = plan_cases.mapping_cases(PAIRS)


@pytest.mark.parametrize("pipeline", [0, 1, 2], ids=["one-pass", "persistent", "pipelined"])
@pytest.mark.parametrize("kind,dtype,pdtype,direction,lpr,vpl", MAPPING_CASES,
                         ids=[f"{k}-{d}{'+' + p if p else ''}-{dr}-{l}x{v}"
                              for k, d, p, dr, l, v in MAPPING_CASES])
def test_every_mapping(device, kind, dtype, pdtype, direction, lpr, vpl, pipeline):
    """Force each compiled (lanes per row, vectors per lane) mapping on a row that leaves
    the last vector slot partly empty, with a ragged final row group: with the planner's
    grid (one row group per workgroup at these sizes), and with a persistent grid of a
    third of the row groups (each workgroup takes several, unevenly) in the plain and in
    the pipelined kernel."""
    N, M = plan_cases.mapping_shape(dtype, lpr, vpl)
    w = small_workload(kind, dtype, N, M=M, x_mean=0.1, pdtype=pdtype)
    opt = rn.Options(path=rn.NORM_PATH_ROWS, lanes_per_row=lpr, vecs_per_lane=vpl)
    code = dtype_code(dtype, pdtype)
    p = rn.norm_plan(direction == "bwd", kind == "ln", M, N, code, options=opt)
    assert (p.path, p.lanes_per_row, p.vecs_per_lane) == (rn.NORM_PATH_ROWS, lpr, vpl)
    groups = -(-M // (p.block // lpr))
    if pipeline:
        assert groups >= 3
        opt.grid = groups // 3
        opt.pipeline = pipeline
        q = rn.norm_plan(direction == "bwd", kind == "ln", M, N, code, options=opt)
        assert q.grid < groups
        if pipeline == 2 and not q.pipelined:
            # 1024 lanes x 4 vectors (backward): no registers for a second stage
            assert direction == "bwd" and lpr == 1024 and vpl > 2
        else:
            assert q.pipelined == (pipeline == 2)
    inputs = gen.make_inputs(w)
    run = GpuRun(w, inputs, device)
    if direction == "fwd":
        run.forward(opt)
        run.sync()
        check_forward(run, inputs, np.arange(M))
    else:
        run.forward()
        run.backward(opt)
        run.sync()
        check_backward(run, inputs, np.arange(M))


@pytest.mark.parametrize("path", [rn.NORM_PATH_SPLIT, rn.NORM_PATH_GENERIC])
@pytest.mark.parametrize("dtype,pdtype", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("kind", ["rms", "ln"])
@pytest.mark.parametrize("N", [256, 384, 4096, 12288])
def test_forced_paths(device, kind, dtype, pdtype, N, path):
    w = small_workload(kind, dtype, N, M=517, pdtype=pdtype)
    full_check(w, device, rows=np.arange(w.M), fwd_options=rn.Options(path=path),
               bwd_options=rn.Options(path=path))


CLUSTER_CASES = plan_cases.cluster_cases(PAIRS)


@pytest.mark.parametrize("kind,dtype,pdtype,N,C,R", CLUSTER_CASES,
                         ids=[f"{k}-{d}{'+' + p if p else ''}-N{n}-C{c}-R{r}"
                              for k, d, p, n, c, r in CLUSTER_CASES])
def test_cluster_path(device, kind, dtype, pdtype, N, C, R):
    """Rows split over C workgroups, forward and backward, with a row count that leaves
    the clusters unevenly loaded."""
    M = plan_cases.cluster_rows(N)
    w = small_workload(kind, dtype, N, M=M, x_mean=0.3, x_std=1.2, pdtype=pdtype)
    opt = rn.Options(path=rn.NORM_PATH_CLUSTER, cluster_size=C, cluster_rows=R)
    code = dtype_code(dtype, pdtype)
    for bwd in (False, True):
        assert rn.norm_plan(bwd, kind == "ln", M, N, code, options=opt).path == \
            rn.NORM_PATH_CLUSTER
    for bwd in (False, True):
        assert rn.norm_cluster_resident(bwd, kind == "ln", M, N, code, opt) == 1, \
            "one cluster must fit the device (otherwise the call silently takes another path)"
    full_check(w, device, rows=np.arange(M), fwd_options=opt, bwd_options=opt)


def _cluster_mapping_cases():
    import re
    src = open(rn.__file__.replace("__init__.py", "csrc/launch.h")).read()
    cases = []
    for direction, macro in (("fwd", "RN_CLUSTER_FWD_MAPPINGS"), ("bwd", "RN_CLUSTER_BWD_MAPPINGS")):
        lines = src[src.index(f"#define {macro}"):].splitlines()
        end = next(i for i, line in enumerate(lines) if not line.rstrip().endswith("\\"))
        body = "\n".join(lines[:end + 1])
        for t, v, r in re.findall(r"X\((\d+), (\d+), (\d+)\)", body):
            cases.append((direction, int(t), int(v), int(r)))
    return cases


CLUSTER_MAPPINGS = _cluster_mapping_cases()


@pytest.mark.parametrize("direction,T,V,R", CLUSTER_MAPPINGS,
                         ids=[f"{d}-{t}x{v}r{r}" for d, t, v, r in CLUSTER_MAPPINGS])
@pytest.mark.parametrize("dtype,pdtype", [("bf16", None), ("f32", None), ("f16", "f32")],
                         ids=["bf16", "f32", "f16+f32"])
@pytest.mark.parametrize("kind", ["rms", "ln"])
def test_every_cluster_mapping(device, kind, dtype, pdtype, direction, T, V, R):
    """Force each compiled split-row mapping (threads, vectors per lane, rows per step) on
    a 2-member cluster whose slice leaves the last vector slot partly empty, with a row
    count that leaves the last step and the clusters unevenly loaded."""
    epv = 4 if dtype == "f32" else 8
    C = 2
    slice_vecs = T * V - max(1, T // 3)
    N = C * slice_vecs * epv
    M = 37
    w = small_workload(kind, dtype, N, M=M, x_mean=0.3, x_std=1.2, pdtype=pdtype)
    opt = rn.Options(path=rn.NORM_PATH_CLUSTER, cluster_size=C, lanes_per_row=T, vecs_per_lane=V,
                     cluster_rows=R)
    code = dtype_code(dtype, pdtype)
    bwd = direction == "bwd"
    try:
        rn.norm_plan(bwd, kind == "ln", M, N, code, options=opt)
    except rn.NormError:
        pytest.skip("mapping not built for this direction")
    if rn.norm_cluster_resident(bwd, kind == "ln", M, N, code, opt) != 1:
        pytest.skip("a cluster does not fit the device")
    inputs = gen.make_inputs(w)
    run = GpuRun(w, inputs, device)
    if not bwd:
        run.forward(opt)
        run.sync()
        check_forward(run, inputs, np.arange(M))
    else:
        run.forward()
        run.backward(opt)
        run.sync()
        check_backward(run, inputs, np.arange(M))


# Both kinds, fp32 (plain fmaf / adds) and 16-bit (dot-product) partial sums, one and two
# rows per exchange step; every case is accepted by the planner in both directions.
SELF_CASES = [("ln", "bf16", None, 65536, 4, 1), ("rms", "bf16", None, 131072, 8, 1),
              ("rms", "f32", None, 32768, 4, 1), ("ln", "f32", None, 65536, 8, 1),
              ("ln", "f32", None, 32768, 8, 2), ("ln", "bf16", None, 32768, 4, 2),
              ("rms", "f16", "f32", 65536, 8, 2), ("ln", "bf16", None, 262144, 16, 1)]


@pytest.mark.parametrize("fused", [False, True], ids=["plain", "residual"])
@pytest.mark.parametrize("kind,dtype,pdtype,N,C,R", SELF_CASES,
                         ids=[f"{k}-{d}{'+' + p if p else ''}-N{n}-C{c}-R{r}"
                              for k, d, p, n, c, r in SELF_CASES])
def test_cluster_partials_computed_locally(device, kind, dtype, pdtype, N, C, R, fused):
    """A split-row member that does not receive another member's partial sums computes
    them itself.  Forcing that for every member and step (cluster_wait = -1) must give
    the same bits as the exchange, forward and backward."""
    import torch
    M = 37
    w = small_workload(kind, dtype, N, M=M, x_mean=0.2, x_std=1.1, pdtype=pdtype)
    code = dtype_code(dtype, pdtype)
    outs = []
    for wait in (0, -1):
        opt = rn.Options(path=rn.NORM_PATH_CLUSTER, cluster_size=C, cluster_rows=R,
                         cluster_wait=wait)
        for bwd in (False, True):
            p = rn.norm_plan(bwd, kind == "ln", M, N, code, options=opt)
            assert (p.path, p.cluster_size, p.cluster_rows) == (rn.NORM_PATH_CLUSTER, C, R)
            # otherwise both runs would take the fallback plan and agree trivially
            assert rn.norm_cluster_resident(bwd, kind == "ln", M, N, code, opt) == 1
        inputs = gen.make_inputs(w, residual=fused)
        run = GpuRun(w, inputs, device)
        if fused:
            res = to_device(inputs["res"], dtype, device)
            dsum = to_device(inputs["dsum"], dtype, device)
            s = torch.empty_like(run.x)
            if kind == "rms":
                rn.norm_rms_fwd_add(run.x, res, run.gamma, run.y, s, run.rstd, eps=w.eps,
                                    options=opt)
                rn.norm_rms_bwd_add(run.dy, s, run.gamma, run.rstd, dsum, run.dx, run.dgamma,
                                    options=opt)
            else:
                rn.norm_ln_fwd_add(run.x, res, run.gamma, run.beta, run.y, s, run.mean,
                                   run.rstd, eps=w.eps, options=opt)
                rn.norm_ln_bwd_add(run.dy, s, run.gamma, run.mean, run.rstd, dsum, run.dx,
                                   run.dgamma, run.dbeta, options=opt)
        else:
            run.forward(opt)
            run.backward(opt)
        run.sync()
        outs.append({k: getattr(run, k).clone() for k in ("y", "dx", "rstd", "dgamma", "mean",
                                                          "dbeta") if getattr(run, k) is not None})
        if wait == 0 and not fused:
            check_forward(run, inputs, np.arange(M))
            check_backward(run, inputs, np.arange(M))
    for k in outs[0]:
        assert torch.equal(outs[0][k], outs[1][k]), f"{k}: locally computed partials differ"


@pytest.mark.parametrize("name", ["rms4"])
def test_long_rows_run_on_cluster_path(device, name):
    """The 131072-column workload splits its rows over a cluster of workgroups, forward
    and backward, and every cluster fits the device at once."""
    w = gen.WORKLOADS[name]
    code = rn.NORM_DTYPE_BF16 if w.dtype == "bf16" else rn.NORM_DTYPE_F32
    for bwd in (False, True):
        assert rn.norm_plan(bwd, w.kind == "ln", w.M, w.N, code).path == rn.NORM_PATH_CLUSTER
        assert rn.norm_cluster_resident(bwd, w.kind == "ln", w.M, w.N, code) == 1


@pytest.mark.parametrize("grid", [1, 3, 64])
@pytest.mark.parametrize("kind", ["rms", "ln"])
def test_grid_override(device, kind, grid):
    w = small_workload(kind, "bf16", 1024, M=1000)
    full_check(w, device, rows=np.arange(w.M), fwd_options=rn.Options(grid=grid),
               bwd_options=rn.Options(grid=grid))


@pytest.mark.parametrize("mode", [rn.NORM_DGAMMA_ATOMIC_ROW, rn.NORM_DGAMMA_ATOMIC_WG])
@pytest.mark.parametrize("kind", ["rms", "ln"])
def test_atomic_dgamma_variants(device, kind, mode):
    """The atomic comparison variants agree with the oracle (not bitwise with each other)."""
    w = small_workload(kind, "bf16", 4096, M=2000)
    full_check(w, device, rows=sample_rows(w.M), bwd_options=rn.Options(dgamma_mode=mode))


@pytest.mark.parametrize("name", ["ln2", "rms3", "rms4", "sweep_ln_f32_65536"])
def test_two_stage_is_deterministic(device, name):
    """Two-stage backward: bitwise identical dx, dgamma, dbeta across runs."""
    import torch
    base = gen.WORKLOADS[name] if name in gen.WORKLOADS else gen.sweep_workload("ln", "f32", 65536)
    w = base.scaled(min(base.M, 4096))
    inputs = gen.make_inputs(w)
    run = GpuRun(w, inputs, device)
    run.forward()
    outs = []
    for _ in range(3):
        run.backward()
        run.sync()
        outs.append([t.clone() for t in (run.dx, run.dgamma, run.dbeta) if t is not None])
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


@pytest.mark.parametrize("kind", ["rms", "ln"])
def test_backward_with_oracle_stats(device, kind):
    """Feed the backward the oracle's statistics rounded to fp32: isolates the backward."""
    import oracle
    import torch
    w = small_workload(kind, "bf16", 2048, M=700)
    inputs = gen.make_inputs(w)
    run = GpuRun(w, inputs, device)
    orc = oracle.get()
    if kind == "rms":
        _, rstd = orc.rms_fwd(inputs["x"], inputs["gamma"], w.eps)
        mean = None
    else:
        _, mean, rstd = orc.ln_fwd(inputs["x"], inputs["gamma"], inputs["beta"], w.eps)
        mean = torch.tensor(mean.astype(np.float32), device=device)
    rstd = torch.tensor(rstd.astype(np.float32), device=device)
    run.backward(mean=mean, rstd=rstd)
    run.sync()
    check_backward(run, inputs, np.arange(w.M))


@pytest.mark.parametrize("dtype,pdtype", [("bf16", None), ("f16", "f32")], ids=["bf16", "f16+f32"])
@pytest.mark.parametrize("offset", [1, 3])
@pytest.mark.parametrize("kind", ["rms", "ln"])
def test_misaligned_inputs(device, kind, offset, dtype, pdtype):
    w = small_workload(kind, dtype, 1024, M=300, pdtype=pdtype)
    full_check(w, device, rows=np.arange(w.M), x_offset=offset)


@pytest.mark.parametrize("kind", ["rms", "ln"])
def test_empty_batch(device, kind):
    import torch
    N = 1024
    x = torch.empty(0, N, dtype=torch.bfloat16, device=device)
    g = torch.ones(N, dtype=torch.bfloat16, device=device)
    b = torch.zeros(N, dtype=torch.bfloat16, device=device)
    y = torch.empty_like(x)
    rstd = torch.empty(0, dtype=torch.float32, device=device)
    mean = torch.empty(0, dtype=torch.float32, device=device)
    dg = torch.full((N,), 7.0, device=device)
    db = torch.full((N,), 7.0, device=device)
    if kind == "rms":
        rn.norm_rms_fwd(x, g, y, rstd)
        rn.norm_rms_bwd(x, x, g, rstd, torch.empty_like(x), dg)
    else:
        rn.norm_ln_fwd(x, g, b, y, mean, rstd)
        rn.norm_ln_bwd(x, x, g, mean, rstd, torch.empty_like(x), dg, db)
        torch.cuda.synchronize()
        assert torch.count_nonzero(db).item() == 0
    torch.cuda.synchronize()
    assert torch.count_nonzero(dg).item() == 0, "a sum over no rows is zero"


def test_degenerate_rows(device):
    """RMSNorm of a zero row is 0 (rstd = 1/sqrt(eps)); LayerNorm of a constant row is beta."""
    import torch
    N, eps = 512, 1e-5
    x = torch.zeros(3, N, dtype=torch.bfloat16, device=device)
    x[1] = 2.5
    x[2, ::2] = 1.0
    g = torch.full((N,), 1.5, dtype=torch.bfloat16, device=device)
    b = (torch.arange(N, device=device) % 7 * 0.125).to(torch.bfloat16)
    y = torch.empty_like(x)
    rstd = torch.empty(3, device=device)
    mean = torch.empty(3, device=device)
    rn.norm_rms_fwd(x, g, y, rstd, eps=eps)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y[0]).item() == 0
    assert abs(rstd[0].item() - eps ** -0.5) <= 1e-5 * eps ** -0.5
    rn.norm_ln_fwd(x, g, b, y, mean, rstd, eps=eps)
    torch.cuda.synchronize()
    assert torch.equal(y[1].float(), b.float()), "constant row must give beta"
    assert torch.equal(y[0].float(), b.float())


def test_nan_propagates_to_its_row_only(device):
    import torch
    w = small_workload("rms", "bf16", 1024, M=64)
    inputs = gen.make_inputs(w)
    run = GpuRun(w, inputs, device)
    run.x[5, 17] = float("nan")
    run.forward()
    run.sync()
    assert torch.isnan(run.y[5].float()).all()
    assert not torch.isnan(run.y[torch.arange(64, device=device) != 5].float()).any()


def test_invariants_on_gpu_outputs(device):
    """gamma = 1: RMS of each y row is 1; LayerNorm rows have mean 0, variance 1 (bf16)."""
    import torch
    M, N = 256, 4096
    x = gen.fill(M * N, "bf16", 77, 0.5, 2.0).reshape(M, N)
    from parity import to_device
    xd = to_device(x, "bf16", device)
    g = torch.ones(N, dtype=torch.bfloat16, device=device)
    b = torch.zeros(N, dtype=torch.bfloat16, device=device)
    y = torch.empty_like(xd)
    rstd = torch.empty(M, device=device)
    mean = torch.empty(M, device=device)
    rn.norm_rms_fwd(xd, g, y, rstd, eps=0.0)
    torch.cuda.synchronize()
    ms = y.double().pow(2).mean(dim=1)
    assert (ms - 1).abs().max().item() < 2 ** -7
    rn.norm_ln_fwd(xd, g, b, y, mean, rstd, eps=0.0)
    torch.cuda.synchronize()
    assert y.double().mean(dim=1).abs().max().item() < 2 ** -7
    assert (y.double().var(dim=1, unbiased=False) - 1).abs().max().item() < 2 ** -6


def test_events_and_streams(device):
    """Options' events bracket the main kernel; calls run on a side stream."""
    import torch
    w = small_workload("ln", "bf16", 4096, M=4096)
    inputs = gen.make_inputs(w)
    run = GpuRun(w, inputs, device)
    s = torch.cuda.Stream(device)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        e0.record(s)
        e1.record(s)  # materialise the handles
        s.synchronize()
        opt = rn.Options(ev_start=e0.cuda_event, ev_stop=e1.cuda_event)
        run.forward(opt)
        run.backward(opt)
    s.synchronize()
    assert e0.elapsed_time(e1) > 0
    check_forward(run, inputs, sample_rows(w.M))
    check_backward(run, inputs, sample_rows(w.M))


@pytest.mark.parametrize("kind,dtype,M,N", [("rms", "bf16", 64, 262144), ("ln", "bf16", 48, 262144),
                                             ("rms", "f32", 40, 131072), ("rms", "bf16", 2048, 131072),
                                             ("ln", "bf16", 2, (1 << 21) + 8),
                                             ("rms", "f32", 3, 100003)])
def test_forward_without_workspace(device, kind, dtype, M, N):
    """The forward's argument list without a workspace (NULL, 0 bytes) works at every row
    length: rows that the fastest plan splits over a cluster, or over the sliced passes,
    run a plan that needs none."""
    import torch
    code = dtype_code(dtype)
    assert rn.norm_fwd_workspace_size(M, N, kind == "ln", code) > 0
    w = small_workload(kind, dtype, N, M=M, x_mean=0.2)
    inputs = gen.make_inputs(w)
    run = GpuRun(w, inputs, device)
    stream = torch.cuda.current_stream(device).cuda_stream
    lib = rn.lib()
    if kind == "rms":
        st = lib.norm_rms_fwd(run.x.data_ptr(), run.gamma.data_ptr(), run.y.data_ptr(),
                              run.rstd.data_ptr(), M, N, w.eps, code, None, 0, stream)
    else:
        st = lib.norm_ln_fwd(run.x.data_ptr(), run.gamma.data_ptr(), run.beta.data_ptr(),
                             run.y.data_ptr(), run.mean.data_ptr(), run.rstd.data_ptr(), M, N,
                             w.eps, code, None, 0, stream)
    assert st == rn.NORM_OK, rn.status_string(st)
    run.sync()
    check_forward(run, inputs, np.arange(M))
    # a workspace that is too short is treated the same way
    y0 = run.y.clone()
    run.y.zero_()
    short = torch.empty(64, dtype=torch.uint8, device=device)
    if kind == "rms":
        st = lib.norm_rms_fwd(run.x.data_ptr(), run.gamma.data_ptr(), run.y.data_ptr(),
                              run.rstd.data_ptr(), M, N, w.eps, code, short.data_ptr(), 64, stream)
        assert st == rn.NORM_OK
        run.sync()
        assert torch.equal(run.y.view(torch.int16) if dtype == "bf16" else run.y,
                           y0.view(torch.int16) if dtype == "bf16" else y0)


def test_side_stream_with_binding_workspace(device):
    """The binding's own workspace stays reserved while a call on a side stream uses it,
    though torch's caching allocator tracks it on the current stream: allocations made on
    the current stream in between must not reuse it."""
    import torch
    w = small_workload("rms", "bf16", 131072, M=512)
    inputs = gen.make_inputs(w)
    run = GpuRun(w, inputs, device)
    side = torch.cuda.Stream(device)
    side.wait_stream(torch.cuda.current_stream(device))
    for _ in range(3):
        run.forward(stream=side)
        run.backward(stream=side)
        # fill fresh blocks on the current stream while the side stream may still run
        junk = [torch.full((1 << 20,), 7, dtype=torch.uint8, device=device) for _ in range(8)]
        del junk
    side.synchronize()
    run.sync()
    check_forward(run, inputs, np.arange(w.M))
    check_backward(run, inputs, np.arange(w.M))


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (1 << 20) + 48])
def test_stream_reference(device, nbytes):
    """The benchmark's streaming reference kernel: copy and a + b over 16-byte vectors,
    including a ragged last workgroup."""
    import torch
    n = nbytes // 4
    a = torch.randint(0, 1 << 30, (n,), dtype=torch.int32, device=device)
    b = torch.randint(0, 1 << 30, (n,), dtype=torch.int32, device=device)
    d = torch.full((n,), -1, dtype=torch.int32, device=device)
    rn.norm_stream_reference(0, a, None, d)
    torch.cuda.synchronize(device)
    assert torch.equal(d, a)
    rn.norm_stream_reference(1, a, b, d)
    torch.cuda.synchronize(device)
    assert torch.equal(d, a + b)
