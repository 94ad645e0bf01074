"""The pipelined forward's tail workgroups: on a persistent grid of G workgroups with at
least 3G row groups, the persistent workgroups stop about G groups short of the end and
each extra workgroup takes one of the rest.  The assignment changes which workgroup
normalizes a row, never how, so every output must have the same bits as the same kernel
on a grid too large for tail workgroups (fewer than 3 groups per workgroup); one case
per mapping is also checked against the oracle.  The group counts straddle the edges:
exactly 3G (the smallest with tail workgroups), 3G - 1 (none), and counts whose tail is
between G and 2G groups; M leaves the last row group ragged where a group holds several
rows."""
import numpy as np
import pytest

import gen
import row_normalization_norm_amd as rn
from parity import GpuRun, check_forward, to_device
from test_gpu_parity import dtype_code, small_workload
import plan_cases

pytestmark = pytest.mark.gpu

# kind, dtype, lanes per row, vectors per lane, fused residual
MAPPINGS = [("ln", "bf16", 128, 4, False), ("ln", "bf16", 1024, 4, False),
            ("rms", "f32", 32, 2, False), ("ln", "bf16", 128, 4, True),
            ("rms", "bf16", 512, 2, False)]
G = 16
GROUPS = [3 * G, 3 * G - 1, 3 * G + 1, 5 * G - 3, 100]


def _forward(run, inputs, w, opt, fused, device):
    import torch
    if not fused:
        run.forward(opt)
        run.sync()
        return [run.y.clone(), run.rstd.clone()] + ([run.mean.clone()] if w.kind == "ln" else [])
    res = to_device(inputs["res"], w.dtype, device)
    s = torch.empty_like(run.x)
    if w.kind == "rms":
        rn.norm_rms_fwd_add(run.x, res, run.gamma, run.y, s, run.rstd, eps=w.eps, options=opt)
    else:
        rn.norm_ln_fwd_add(run.x, res, run.gamma, run.beta, run.y, s, run.mean, run.rstd,
                           eps=w.eps, options=opt)
    run.sync()
    return [run.y.clone(), s, run.rstd.clone()] + ([run.mean.clone()] if w.kind == "ln" else [])


@pytest.mark.parametrize("groups", GROUPS)
@pytest.mark.parametrize("kind,dtype,lpr,vpl,fused", MAPPINGS,
                         ids=[f"{k}-{d}-{l}x{v}{'-add' if f else ''}" for k, d, l, v, f in MAPPINGS])
def test_tail_workgroups_same_bits(device, kind, dtype, lpr, vpl, fused, groups):
    N, _ = plan_cases.mapping_shape(dtype, lpr, vpl)
    code = dtype_code(dtype)
    probe = rn.norm_plan(False, kind == "ln", 64, N, code,
                         options=rn.Options(path=rn.NORM_PATH_ROWS, lanes_per_row=lpr,
                                            vecs_per_lane=vpl))
    rows = probe.block // lpr
    M = groups * rows - (rows // 4 + 1 if rows > 1 else 0)  # a ragged last group
    assert -(-M // rows) == groups
    w = small_workload(kind, dtype, N, M=M, x_mean=0.2)
    inputs = gen.make_inputs(w, residual=fused)
    print(f"tail workgroups: {w.name} {lpr}x{vpl} groups {groups} grid {G}", flush=True)
    run = GpuRun(w, inputs, device)

    def opt(grid):
        o = rn.Options(path=rn.NORM_PATH_ROWS, lanes_per_row=lpr, vecs_per_lane=vpl,
                       grid=grid, pipeline=2)
        p = rn.norm_plan(False, kind == "ln", M, N, code, options=o)
        assert p.pipelined and p.grid == grid
        return o

    import torch
    with_tail = _forward(run, inputs, w, opt(G), fused, device)
    if not fused and groups == 3 * G:
        check_forward(run, inputs, np.arange(M))
    # a grid with fewer than three groups per workgroup: no tail workgroups
    without = _forward(run, inputs, w, opt(groups // 2), fused, device)
    names = ["y", "sum", "rstd", "mean"] if fused else ["y", "rstd", "mean"]
    for name, a, b in zip(names, with_tail, without):
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), \
            f"{name} differs between the grids with and without tail workgroups"
