"""Entry points captured into a HIP graph (torch.cuda.graph, stream capture) and replayed.

Each case runs forward + backward eagerly for the reference outputs, captures the same
calls into a graph, then replays it several times with unrelated eager work and
synchronisations between the replays (the outputs are cleared by fill kernels before
each replay), and requires every replay to reproduce the eager outputs bit for bit.
The cases cover every kernel family, the pipelined row kernels, the split-row one (with
its exchange-slot fill kernel) and the sliced passes included.
"""
import numpy as np
import pytest

import gen
import row_normalization_norm_amd as rn
from parity import to_device

pytestmark = pytest.mark.gpu

CASES = [
    # kind, dtype, M, N, fused
    ("rms", "bf16", 4096, 1024, False),    # the small benchmark shape (row-resident path)
    ("ln", "bf16", 1000, 4096, False),
    ("ln", "bf16", 8192, 4096, False),     # pipelined forward and backward (persistent grids)
    ("rms", "bf16", 16384, 1024, False),   # pipelined backward, one-group forward
    ("ln", "f32", 96, 65536, False),       # backward on the split-row path
    ("ln", "bf16", 16, 131072, False),     # a whole row per workgroup forward
    ("rms", "bf16", 8, 262144, False),     # forward and backward on the split-row path
    ("ln", "bf16", 333, 1000, False),      # N not a multiple of 8: scalar and split paths
    ("rms", "bf16", 2, (1 << 21) + 8, False),  # rows past a cluster: the sliced passes
    ("ln", "bf16", 40, 5003, True),         # long rows of elements: sliced, residual add
    ("ln", "bf16", 512, 4096, True),       # residual-add entry points
    ("rms", "f32", 700, 12288, True),
]
_CODE = {"bf16": rn.NORM_DTYPE_BF16, "f32": rn.NORM_DTYPE_F32, "f16": rn.NORM_DTYPE_F16}


@pytest.mark.parametrize("kind,dtype,M,N,fused", CASES,
                         ids=[f"{k}-{d}-{m}x{n}{'-add' if f else ''}" for k, d, m, n, f in CASES])
@pytest.mark.parametrize("own_workspace", [True, False], ids=["workspace", "alloc"])
def test_graph_replay_matches_eager(device, kind, dtype, M, N, fused, own_workspace):
    w = gen.Workload(f"graph_{kind}_{dtype}_{M}x{N}", kind, dtype, M, N, 1e-5, x_mean=0.1,
                     x_std=1.1, config=21)
    _replay_check(device, w, fused, own_workspace)


def _replay_check(device, w, fused, own_workspace, fo=None, bo=None):
    """Eager forward + backward, then the same calls captured and replayed three times;
    every replay must give the eager bits."""
    import torch
    kind, dtype, M, N = w.kind, w.dtype, w.M, w.N
    inp = gen.make_inputs(w, residual=fused)
    ln = kind == "ln"
    x = to_device(inp["x"], dtype, device)
    dy = to_device(inp["dy"], dtype, device)
    g = to_device(inp["gamma"], w.param_dtype, device)
    b = to_device(inp["beta"], w.param_dtype, device) if ln else None
    res = to_device(inp["res"], dtype, device) if fused else None
    dsum = to_device(inp["dsum"], dtype, device) if fused else None
    out = dict(y=torch.empty_like(x), dx=torch.empty_like(x), rstd=torch.empty(M, device=device),
               dg=torch.empty(N, device=device))
    if ln:
        out.update(mean=torch.empty(M, device=device), db=torch.empty(N, device=device))
    if fused:
        out["s"] = torch.empty_like(x)
    code = _CODE[dtype] if w.pdtype is None else rn.dtype_mixed(_CODE[dtype], _CODE[w.pdtype])
    if own_workspace:
        fws_n = rn.norm_fwd_workspace_size(M, N, ln, code, fo)
        fws = torch.empty(fws_n, dtype=torch.uint8, device=device) if fws_n else None
        bws = torch.empty(max(rn.norm_bwd_workspace_size(M, N, ln, code, bo), 1),
                          dtype=torch.uint8, device=device)
    else:
        fws = bws = None

    def step(fo, bo):
        o = out
        if fused:
            if ln:
                rn.norm_ln_fwd_add(x, res, g, b, o["y"], o["s"], o["mean"], o["rstd"], eps=w.eps,
                                   workspace=fws, options=fo)
                rn.norm_ln_bwd_add(dy, o["s"], g, o["mean"], o["rstd"], dsum, o["dx"], o["dg"],
                                   o["db"], workspace=bws, options=bo)
            else:
                rn.norm_rms_fwd_add(x, res, g, o["y"], o["s"], o["rstd"], eps=w.eps,
                                    workspace=fws, options=fo)
                rn.norm_rms_bwd_add(dy, o["s"], g, o["rstd"], dsum, o["dx"], o["dg"],
                                    workspace=bws, options=bo)
        elif ln:
            rn.norm_ln_fwd(x, g, b, o["y"], o["mean"], o["rstd"], eps=w.eps, workspace=fws,
                           options=fo)
            rn.norm_ln_bwd(dy, x, g, o["mean"], o["rstd"], o["dx"], o["dg"], o["db"],
                           workspace=bws, options=bo)
        else:
            rn.norm_rms_fwd(x, g, o["y"], o["rstd"], eps=w.eps, workspace=fws, options=fo)
            rn.norm_rms_bwd(dy, x, g, o["rstd"], o["dx"], o["dg"], workspace=bws, options=bo)

    step(fo, bo)
    torch.cuda.synchronize(device)
    ref = {k: v.clone() for k, v in out.items()}

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(fo, bo)
    scratch = torch.empty(1 << 20, device=device)
    for rep in range(3):
        for v in out.values():
            v.zero_()
        scratch.normal_()  # unrelated eager work between replays
        torch.cuda.synchronize(device)
        graph.replay()
        torch.cuda.synchronize(device)
        for k, v in out.items():
            assert torch.equal(v, ref[k]), f"replay {rep}: {k} differs from the eager result"
    assert np.isfinite(out["dg"].cpu().numpy()).all()


def test_graph_replay_random_forced_plans(device):
    """Capture and replay under seeded random options (the draws of
    test_gpu_random_options with another seed; the deterministic dgamma reduction only,
    since the atomic ones need not repeat their bits), with or without the residual add
    and with the caller's workspace or the binding's."""
    from test_gpu_random_options import _cases, _describe
    rng = np.random.default_rng(11)
    ran = 0
    for i, kind, dtype, pdtype, M, N, fo, bo, x_mean, x_std in _cases(20261205, 300):
        for o in (fo, bo):
            if o is not None:
                o.dgamma_mode = rn.NORM_DGAMMA_TWO_STAGE
        code = _CODE[dtype] if pdtype is None else rn.dtype_mixed(_CODE[dtype], _CODE[pdtype])
        try:
            for bwd, o in ((False, fo), (True, bo)):
                rn.norm_plan(bwd, kind == "ln", M, N, code, True, o)
        except rn.NormError:
            continue
        fused, own = bool(rng.integers(2)), bool(rng.integers(2))
        w = gen.Workload(f"graph_{kind}_{dtype}_{M}x{N}", kind, dtype, M, N, 1e-5,
                         x_mean=x_mean, x_std=x_std, config=21, pdtype=pdtype)
        name = (f"case {i}: {kind} {dtype}{'+' + pdtype if pdtype else ''} {M}x{N}, fused "
                f"{fused}, own workspace {own}; forward [{_describe(fo)}], backward "
                f"[{_describe(bo)}]")
        print(name, flush=True)
        try:
            _replay_check(device, w, fused, own, fo, bo)
        except AssertionError as e:
            raise AssertionError(f"{name}: {e}") from None
        ran += 1
    assert ran >= 60, f"only {ran} drawn cases ran"
