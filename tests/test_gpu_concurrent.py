"""Calls in flight together on two streams, each with its own workspace, give the same bits
as the same calls run one at a time.

Both workloads take the split-row path (the backward of one, forward and backward of the
other), whose members exchange partial sums through their workspace and normally run
together.  Two such grids on the device at once cannot all be resident, so members may
wait for partners that have not started; every wait is bounded, and a member that gives
up computes the missing partial sums itself with the same operations, so the outputs
cannot depend on the timing.  The serial results are also checked against the oracle on
sampled rows."""
import numpy as np
import pytest

import gen
import row_normalization_norm_amd as rn
from parity import GpuRun, check_backward, check_forward, sample_rows
from test_gpu_parity import small_workload

pytestmark = pytest.mark.gpu

# (kind, dtype, M, N): LayerNorm with a row-path forward and a split-row backward, and
# RMSNorm split over workgroups in both directions
WORKLOADS = [("ln", "bf16", 1024, 32768), ("rms", "bf16", 512, 131072)]


def _outputs(run, kind):
    out = [run.y, run.rstd, run.dx, run.dgamma]
    if kind == "ln":
        out += [run.mean, run.dbeta]
    return [t.clone() for t in out]


def _bits(t):
    import torch
    return t.contiguous().view(torch.uint8)


def test_two_streams_same_bits_as_serial(device):
    import torch
    runs = []
    for kind, dtype, M, N in WORKLOADS:
        w = small_workload(kind, dtype, N, M=M, x_mean=0.3)
        for bwd in (False, True):
            p = rn.norm_plan(bwd, kind == "ln", M, N, rn.NORM_DTYPE_BF16)
            if bwd or kind == "rms":
                assert p.path == rn.NORM_PATH_CLUSTER, (kind, bwd, p.path)
        inputs = gen.make_inputs(w)
        runs.append((w, inputs, GpuRun(w, inputs, device)))

    print("concurrent streams: serial reference", flush=True)
    refs = []
    for w, inputs, run in runs:
        run.forward()
        run.backward()
        run.sync()
        refs.append(_outputs(run, w.kind))
        rows = sample_rows(w.M)
        check_forward(run, inputs, rows)
        check_backward(run, inputs, rows)

    streams = [torch.cuda.Stream(device) for _ in runs]
    for rep in range(3):
        print(f"concurrent streams: pass {rep}", flush=True)
        for _, _, run in runs:
            for t in (run.y, run.dx, run.rstd, run.dgamma, run.mean, run.dbeta):
                if t is not None:
                    t.zero_()
        torch.cuda.synchronize(device)
        # launch everything before waiting for anything
        for (w, _, run), s in zip(runs, streams):
            with torch.cuda.stream(s):
                run.forward(stream=s.cuda_stream)
                run.backward(stream=s.cuda_stream)
        torch.cuda.synchronize(device)
        for (w, _, run), ref in zip(runs, refs):
            names = ["y", "rstd", "dx", "dgamma", "mean", "dbeta"]
            for name, a, b in zip(names, _outputs(run, w.kind), ref):
                assert torch.equal(_bits(a), _bits(b)), \
                    f"{w.name}: {name} differs from the serial run (pass {rep})"
