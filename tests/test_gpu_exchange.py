"""The split-row exchange needs no clearing between calls: every call tags its words with
its own epoch, so whatever the workspace holds on entry — the words of the previous call
on the same workspace, random bytes, all ones, zeros — cannot be taken for a partner's
partial sums.  Each fill must give the same bits as the first call, whose results are
also checked against the oracle on sampled rows."""
import numpy as np
import pytest

import gen
import row_normalization_norm_amd as rn
from parity import GpuRun, check_backward, check_forward, sample_rows
from test_gpu_parity import dtype_code, small_workload

pytestmark = pytest.mark.gpu

# (kind, dtype, M, N): split rows in the backward, or in both directions
CASES = [("ln", "bf16", 1024, 32768), ("rms", "bf16", 512, 131072), ("ln", "f32", 64, 65536)]
FILLS = ["previous call", "random bytes", "all ones", "zeros", "previous call"]


def _bits(t):
    import torch
    return t.contiguous().view(torch.uint8)


@pytest.mark.parametrize("kind,dtype,M,N", CASES, ids=[f"{k}-{d}-{m}x{n}" for k, d, m, n in CASES])
def test_exchange_needs_no_clearing(device, kind, dtype, M, N):
    import torch
    code = dtype_code(dtype)
    ln = kind == "ln"
    assert rn.norm_plan(True, ln, M, N, code).path == rn.NORM_PATH_CLUSTER
    w = small_workload(kind, dtype, N, M=M, x_mean=0.2)
    inputs = gen.make_inputs(w)
    run = GpuRun(w, inputs, device)
    size = max(rn.norm_fwd_workspace_size(M, N, ln, code), rn.norm_bwd_workspace_size(M, N, ln, code))
    ws = torch.zeros(size, dtype=torch.uint8, device=device)
    gen_rng = torch.Generator(device=device)
    gen_rng.manual_seed(7)

    def outputs():
        return [t.clone() for t in (run.y, run.rstd, run.dx, run.dgamma, run.mean, run.dbeta)
                if t is not None]

    print(f"exchange: {w.name} first call", flush=True)
    _call(run, w, ws)
    run.sync()
    ref = outputs()
    rows = sample_rows(M)
    check_forward(run, inputs, rows)
    check_backward(run, inputs, rows)
    for fill in FILLS:
        print(f"exchange: {w.name} workspace holding {fill}", flush=True)
        if fill == "random bytes":
            ws.copy_(torch.randint(0, 256, (size,), dtype=torch.uint8, device=device,
                                   generator=gen_rng))
        elif fill == "all ones":
            ws.fill_(255)
        elif fill == "zeros":
            ws.zero_()
        for t in (run.y, run.rstd, run.dx, run.dgamma, run.mean, run.dbeta):
            if t is not None:
                t.zero_()
        _call(run, w, ws)
        run.sync()
        for a, b in zip(outputs(), ref):
            assert torch.equal(_bits(a), _bits(b)), f"{w.name}: outputs differ with {fill}"


def _call(run, w, ws):
    if w.kind == "rms":
        rn.norm_rms_fwd(run.x, run.gamma, run.y, run.rstd, eps=w.eps, workspace=ws)
        rn.norm_rms_bwd(run.dy, run.x, run.gamma, run.rstd, run.dx, run.dgamma, workspace=ws)
    else:
        rn.norm_ln_fwd(run.x, run.gamma, run.beta, run.y, run.mean, run.rstd, eps=w.eps,
                       workspace=ws)
        rn.norm_ln_bwd(run.dy, run.x, run.gamma, run.mean, run.rstd, run.dx, run.dgamma,
                       run.dbeta, workspace=ws)
