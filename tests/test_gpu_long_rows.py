"""Rows past the reach of a cluster, and long rows that are not whole 16-byte vectors: the
sliced passes (a (slice, row block) grid with a per-row merge between the passes), which
spread even a single row over the whole chip.  Every row and every dgamma/dbeta column
is compared with the oracle.

The slice of a 16-byte-vector row is 256 lanes x 2 vectors; of an element row, 256
lanes x 8 elements.  The shapes below leave the last slice ragged, give a row block
rows that the next one does not have, and (with M = 1) put a single row on thousands
of workgroups."""
import numpy as np
import pytest

import gen
import row_normalization_norm_amd as rn
from parity import GpuRun, check_all_rows, full_check
from test_gpu_parity import PAIRS, PAIR_IDS, dtype_code, small_workload

pytestmark = pytest.mark.gpu

SPLIT = rn.Options(path=rn.NORM_PATH_SPLIT)
GENERIC = rn.Options(path=rn.NORM_PATH_GENERIC)

# (kind, dtype, pdtype, M, N): rows beyond the longest cluster (2^17 vectors), taken by
# the default plan in both directions.
BEYOND = [
    ("rms", "bf16", None, 1, (1 << 21) + 8),
    ("ln", "bf16", None, 3, (1 << 21) + 8),
    ("ln", "f32", None, 2, (1 << 19) + 4),
    ("rms", "f16", None, 2, (1 << 21) + 3),      # not whole vectors: element slices
    ("ln", "bf16", "f32", 1, 3 * (1 << 20) + 8),
    ("ln", "bf16", None, 5, (1 << 20) + 1000),
    ("rms", "f32", None, 1, (1 << 20) + 1),      # odd fp32 row
]


@pytest.mark.parametrize("kind,dtype,pdtype,M,N", BEYOND,
                         ids=[f"{k}-{d}{'+' + p if p else ''}-{m}x{n}" for k, d, p, m, n in BEYOND])
def test_rows_beyond_a_cluster(device, kind, dtype, pdtype, M, N):
    code = dtype_code(dtype, pdtype)
    for bwd in (False, True):
        p = rn.norm_plan(bwd, kind == "ln", M, N, code)
        vec = N % (4 if dtype == "f32" else 8) == 0
        assert p.path == (rn.NORM_PATH_SPLIT if vec or not bwd else rn.NORM_PATH_GENERIC), \
            (bwd, p.path)
        assert p.grid >= 256, "one row must spread over the chip"
    w = small_workload(kind, dtype, N, M=M, x_mean=0.25, pdtype=pdtype)
    full_check(w, device, rows=np.arange(M))


# Forced sliced passes at lengths the oracle checks quickly: several slices with a ragged
# last one, one row block and several (517 rows over up to 256 blocks leaves the last
# block short), 16-byte vectors and element loads.
FORCED_N = [5000, 4100, 12289, 40000]


@pytest.mark.parametrize("N", FORCED_N)
@pytest.mark.parametrize("dtype,pdtype", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("kind", ["rms", "ln"])
def test_forced_sliced_passes(device, kind, dtype, pdtype, N):
    M = 37 if N > 20000 else 517
    vec = N % (4 if dtype == "f32" else 8) == 0
    w = small_workload(kind, dtype, N, M=M, x_mean=0.3, pdtype=pdtype)
    # the backward's sliced passes over elements are its GENERIC plan
    full_check(w, device, rows=np.arange(M), fwd_options=SPLIT,
               bwd_options=SPLIT if vec else GENERIC)


@pytest.mark.parametrize("N", FORCED_N)
@pytest.mark.parametrize("kind", ["rms", "ln"])
def test_forced_sliced_passes_one_row(device, kind, N):
    w = small_workload(kind, "bf16", N, M=1, x_mean=-0.4)
    vec = N % 8 == 0
    full_check(w, device, rows=np.arange(1), fwd_options=SPLIT,
               bwd_options=SPLIT if vec else GENERIC)


@pytest.mark.parametrize("row_blocks", [1, 2, 7, 64])
def test_sliced_row_blocks(device, row_blocks):
    """The options' grid sets the number of row blocks: each covers ceil(M / blocks) rows."""
    M, N = 131, 9000
    w = small_workload("ln", "bf16", N, M=M, x_mean=0.1)
    opt = rn.Options(path=rn.NORM_PATH_SPLIT, grid=row_blocks)
    p = rn.norm_plan(True, True, M, N, rn.NORM_DTYPE_BF16, options=opt)
    assert p.partial_rows == -(-M // -(-M // row_blocks))
    full_check(w, device, rows=np.arange(M), fwd_options=opt, bwd_options=opt)


def test_sliced_passes_are_deterministic(device):
    """Two runs give the same bits: every sum of the sliced passes and of the merge is
    taken in a fixed order."""
    import torch
    M, N = 3, (1 << 21) + 8
    w = small_workload("ln", "bf16", N, M=M, x_mean=0.5)
    inputs = gen.make_inputs(w)
    outs = []
    for _ in range(2):
        run = GpuRun(w, inputs, device)
        run.forward()
        run.backward()
        run.sync()
        outs.append([t.clone() for t in (run.y, run.mean, run.rstd, run.dx, run.dgamma,
                                         run.dbeta)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    check_all_rows(run, inputs)


@pytest.mark.parametrize("N", [5000, 5003])
def test_sliced_degenerate_rows_and_nan(device, N):
    """On the sliced passes: RMSNorm of a zero row is 0, LayerNorm of a constant row is
    beta, and a NaN reaches its own row's outputs only."""
    import torch
    eps = 1e-5
    M = 5
    x = torch.randn(M, N, device=device).to(torch.bfloat16)
    x[0] = 0.0
    x[1] = 2.5
    x[3, N // 2] = float("nan")
    g = torch.full((N,), 1.5, dtype=torch.bfloat16, device=device)
    b = (torch.arange(N, device=device) % 7 * 0.125).to(torch.bfloat16)
    y = torch.empty_like(x)
    rstd = torch.empty(M, device=device)
    mean = torch.empty(M, device=device)
    rn.norm_rms_fwd(x, g, y, rstd, eps=eps, options=SPLIT)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y[0]).item() == 0
    assert abs(rstd[0].item() - eps ** -0.5) <= 1e-5 * eps ** -0.5
    assert torch.isnan(y[3].float()).all()
    others = torch.tensor([0, 1, 2, 4], device=device)
    assert not torch.isnan(y[others].float()).any()
    rn.norm_ln_fwd(x, g, b, y, mean, rstd, eps=eps, options=SPLIT)
    torch.cuda.synchronize()
    assert torch.equal(y[0].float(), b.float()), "a zero row gives beta"
    # a constant 2.5: its mean is 2.5 only up to the rounding of sum * (1/N) when 1/N is
    # not a power of two, so beta within the bf16 bound
    assert torch.all((y[1].float() - b.float()).abs() <= 2.0 ** -7), "a constant row gives beta"
    assert torch.isnan(y[3].float()).all()
    assert not torch.isnan(y[others].float()).any()


def test_sliced_empty_batch(device):
    """No rows at a length the sliced passes would take: nothing is written but the
    column sums, which are zero."""
    import torch
    N = (1 << 21) + 8
    x = torch.empty(0, N, dtype=torch.bfloat16, device=device)
    g = torch.ones(N, dtype=torch.bfloat16, device=device)
    b = torch.zeros(N, dtype=torch.bfloat16, device=device)
    y = torch.empty_like(x)
    mean = torch.empty(0, device=device)
    rstd = torch.empty(0, device=device)
    dg = torch.full((N,), 7.0, device=device)
    db = torch.full((N,), 7.0, device=device)
    rn.norm_ln_fwd(x, g, b, y, mean, rstd)
    rn.norm_ln_bwd(x, x, g, mean, rstd, torch.empty_like(x), dg, db)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dg).item() == 0 and torch.count_nonzero(db).item() == 0
