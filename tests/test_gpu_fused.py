"""GPU parity of the residual-add entry points against the fp64 oracle.

Forward: sum = x + residual rounded to the activation type must match the oracle's sum
bit for bit (both sides round the same exact value to the nearest representable one);
y, mean and rstd follow the plain forward's tolerances on that sum.  Backward: dx is the
norm's backward at the sum plus the gradient arriving at the sum (dsum, optional);
dgamma/dbeta are those of the norm at the sum.  All calls go through the C ABI.
"""
import numpy as np
import pytest

import gen
import oracle
import row_normalization_norm_amd as rn
from parity import (TOL_DGAMMA, TOL_F32, TOL_STAT, _check, dgamma_scale, fp32_dx_scale,
                    fp32_y_scale, out_tol, rows_to_host64, to_device, to_host64)

pytestmark = pytest.mark.gpu

PAIRS = [("bf16", None), ("f32", None), ("f16", None), ("bf16", "f32"), ("f16", "f32")]
PAIR_IDS = ["bf16", "f32", "f16", "bf16+f32", "f16+f32"]
_ORC_TYPE = {"f32": oracle.F32, "bf16": oracle.BF16, "f16": oracle.F16}


def _run(device, kind, dtype, pdtype, M, N, with_dsum, fwd_opt=None, bwd_opt=None):
    import torch
    w = gen.Workload(f"fused_{kind}_{dtype}_{M}x{N}", kind, dtype, M, N, 1e-5, x_mean=0.2,
                     x_std=1.3, config=11, pdtype=pdtype)
    inp = gen.make_inputs(w, residual=True)
    res = inp["res"]
    dsum = inp["dsum"] if with_dsum else None
    x = to_device(inp["x"], dtype, device)
    r = to_device(res, dtype, device)
    g = to_device(inp["gamma"], w.param_dtype, device)
    b = to_device(inp["beta"], w.param_dtype, device) if kind == "ln" else None
    dy = to_device(inp["dy"], dtype, device)
    ds = to_device(dsum, dtype, device) if with_dsum else None
    y, s, dx = torch.empty_like(x), torch.empty_like(x), torch.empty_like(x)
    mean = torch.empty(M, device=device) if kind == "ln" else None
    rstd = torch.empty(M, device=device)
    dg = torch.empty(N, device=device)
    db = torch.empty(N, device=device) if kind == "ln" else None
    if kind == "rms":
        rn.norm_rms_fwd_add(x, r, g, y, s, rstd, eps=w.eps, options=fwd_opt)
        rn.norm_rms_bwd_add(dy, s, g, rstd, ds, dx, dg, options=bwd_opt)
    else:
        rn.norm_ln_fwd_add(x, r, g, b, y, s, mean, rstd, eps=w.eps, options=fwd_opt)
        rn.norm_ln_bwd_add(dy, s, g, mean, rstd, ds, dx, dg, db, options=bwd_opt)
    torch.cuda.synchronize(device)
    return w, inp, res, dsum, dict(y=y, s=s, dx=dx, mean=mean, rstd=rstd, dg=dg, db=db)


def _check_all(w, inp, res, dsum, out):
    orc = oracle.get()
    M, N = w.M, w.N
    rows = np.arange(M)
    s_ref = orc.residual_sum(inp["x"], res)
    s_gpu = to_host64(out["s"])
    assert np.array_equal(s_gpu, s_ref), \
        f"residual sum differs in {np.count_nonzero(s_gpu != s_ref)} elements"
    s_bits = oracle.as_type_bits(s_ref, _ORC_TYPE[w.dtype])
    # forward on the sum
    if w.kind == "rms":
        y_ref, rstd_ref = orc.rms_fwd(s_bits, inp["gamma"], w.eps)
    else:
        y_ref, mean_ref, rstd_ref = orc.ln_fwd(s_bits, inp["gamma"], inp["beta"], w.eps)
        row_rms = np.sqrt(np.mean(s_ref ** 2, axis=1))
        _check("mean", out["mean"].cpu().numpy(), mean_ref, TOL_STAT,
               scale=np.maximum(row_rms, 1e-30))
    _check("rstd", out["rstd"].cpu().numpy(), rstd_ref, TOL_STAT, scale=np.abs(rstd_ref))
    y = rows_to_host64(out["y"], rows)
    if w.dtype == "f32" and w.kind == "ln":
        _check("y", y, y_ref, TOL_F32,
               scale=fp32_y_scale(w, {**inp, "x": s_bits}, rows, y, y_ref, orc))
    else:
        _check("y", y, y_ref, out_tol(w.dtype))
    # backward at the sum, plus the gradient arriving at the sum
    if w.kind == "rms":
        dx_ref = orc.rms_bwd_dx(inp["dy"], s_bits, inp["gamma"], w.eps)
        dg_ref, sg = orc.rms_dgamma(inp["dy"], s_bits, w.eps)
    else:
        dx_ref = orc.ln_bwd_dx(inp["dy"], s_bits, inp["gamma"], w.eps)
        dg_ref, db_ref, sg, sb = orc.ln_dgamma_dbeta(inp["dy"], s_bits, w.eps)
        _check("dbeta", out["db"].cpu().numpy(), db_ref, TOL_DGAMMA,
               scale=np.maximum(np.abs(db_ref), sb))
    if dsum is not None:
        ds64 = dsum.astype(np.float64) if w.dtype != "bf16" else \
            gen.bf16_to_f32(dsum).astype(np.float64)
        dx_ref = dx_ref + ds64
    dx = rows_to_host64(out["dx"], rows)
    if w.dtype == "f32":
        # the plain backward's fp32 bound, taken at the sum
        _check("dx", dx, dx_ref, TOL_F32,
               scale=fp32_dx_scale(w, {**inp, "x": s_bits}, rows, dx, dx_ref, orc))
    else:
        _check("dx", dx, dx_ref, out_tol(w.dtype))
    dg = out["dg"].cpu().numpy()
    _check("dgamma", dg, dg_ref, TOL_DGAMMA,
           scale=dgamma_scale(w, {**inp, "x": s_bits}, dg, dg_ref, sg, orc))


@pytest.mark.parametrize("with_dsum", [False, True], ids=["no-dsum", "dsum"])
@pytest.mark.parametrize("N", [64, 384, 1000, 4096, 5003, 16384, 65536])
@pytest.mark.parametrize("dtype,pdtype", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("kind", ["rms", "ln"])
def test_fused_residual(device, kind, dtype, pdtype, N, with_dsum):
    M = max(3, min(600, 1_500_000 // N))
    _check_all(*_run(device, kind, dtype, pdtype, M, N, with_dsum))


@pytest.mark.parametrize("pipeline", [1, 2], ids=["plain", "pipelined"])
@pytest.mark.parametrize("N", [384, 4096])
@pytest.mark.parametrize("dtype,pdtype", [("bf16", None), ("f32", None), ("f16", "f32")],
                         ids=["bf16", "f32", "f16+f32"])
@pytest.mark.parametrize("kind", ["rms", "ln"])
def test_fused_residual_persistent(device, kind, dtype, pdtype, N, pipeline):
    """The residual add and gradient on a persistent grid of 3 workgroups (each taking
    many row groups), in the plain and the pipelined kernels."""
    opt = rn.Options(grid=3, pipeline=pipeline)
    _check_all(*_run(device, kind, dtype, pdtype, 333, N, True, opt, opt))


@pytest.mark.parametrize("path", [rn.NORM_PATH_SPLIT, rn.NORM_PATH_GENERIC, rn.NORM_PATH_CLUSTER])
@pytest.mark.parametrize("dtype,pdtype", [("bf16", None), ("f32", None), ("f16", "f32")],
                         ids=["bf16", "f32", "f16+f32"])
@pytest.mark.parametrize("kind", ["rms", "ln"])
def test_fused_residual_every_path(device, kind, dtype, pdtype, path):
    """The residual add and the residual gradient on the split-row, split and scalar paths."""
    N = 8192
    M = 97
    fwd_opt = rn.Options(path=path)
    if path == rn.NORM_PATH_CLUSTER:
        fwd_opt = rn.Options(path=path, cluster_size=4)
        bwd_opt = rn.Options(path=path, cluster_size=4)
    else:
        bwd_opt = rn.Options(path=path)
    _check_all(*_run(device, kind, dtype, pdtype, M, N, True, fwd_opt, bwd_opt))


@pytest.mark.parametrize("kind,dtype,M,N", [("rms", "bf16", 2, (1 << 21) + 8),
                                             ("ln", "f16", 1, (1 << 21) + 5)])
def test_fused_residual_beyond_a_cluster(device, kind, dtype, M, N):
    """The residual add and gradient on the sliced passes, at rows no cluster holds: the
    statistics pass writes the sum, the normalize pass reads it back."""
    _check_all(*_run(device, kind, dtype, None, M, N, True))


def test_fused_random_forced_plans(device):
    """The residual entry points under seeded random options (the draws of
    test_gpu_random_options with another seed), with and without the gradient at the
    sum; draws the planner or the entry point refuses are left out."""
    from test_gpu_random_options import _CODE, _cases, _describe
    rng = np.random.default_rng(7)
    ran = 0
    for i, kind, dtype, pdtype, M, N, fo, bo, _, _ in _cases(20261204, 400):
        code = rn.dtype_mixed(_CODE[dtype], _CODE[pdtype]) if pdtype else _CODE[dtype]
        try:
            for bwd, o in ((False, fo), (True, bo)):
                rn.norm_plan(bwd, kind == "ln", M, N, code, True, o)
        except rn.NormError:
            continue
        with_dsum = bool(rng.integers(2))
        name = (f"case {i}: {kind} {dtype}{'+' + pdtype if pdtype else ''} {M}x{N}, "
                f"dsum {with_dsum}; forward [{_describe(fo)}], backward [{_describe(bo)}]")
        print(name, flush=True)
        try:
            got = _run(device, kind, dtype, pdtype, M, N, with_dsum, fo, bo)
        except rn.NormError as e:
            print(f"  refused: {e}", flush=True)
            continue
        try:
            _check_all(*got)
        except AssertionError as e:
            raise AssertionError(f"{name}: {e}") from None
        ran += 1
    assert ran >= 100, f"only {ran} drawn cases ran"
