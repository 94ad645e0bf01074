"""The largest shapes the interface takes: a single row of 2^31 - 1 elements (the longest
N), and tensors of more than 4 GiB (row offsets past 32 bits), forward and backward.

Neither fits the fp64 oracle whole, so the inputs are periodic and the expected values
come from properties that hold at any size:

* the longest row repeats short patterns, so every sum the definitions need (the
  pages' RMSNorm and LayerNorm, "Fused RMSNorm", "What it is"; the backward as the
  torch.compile page's "Why Is Peak Vectorization Your New Best Friend?" states it) is
  a whole number of pattern periods plus a remainder, computed exactly in fp64 here;
* the > 4 GiB tensors repeat a block of rows drawn by the input generator: each row's
  outputs are the oracle's for its block row, and the column sums dgamma/dbeta are the
  oracle's sums over the block times the number of whole blocks plus the oracle's sums
  over the rows left over.

Tolerances are those of the other parity tests where the arithmetic is the same, and
worst-case bounds of fp32 summation where a sum runs over far more terms than in any
configuration: recursive summation of n terms errs by at most (n - 1) u sum |t_i|
(u = 2^-24), and the kernels' sums are trees of such runs."""
import numpy as np
import pytest

import gen
import oracle
import row_normalization_norm_amd as rn
from parity import TOL_BF16, to_device, to_host64

pytestmark = pytest.mark.gpu

U = 2.0 ** -24

# ----------------------------------------------------------------- the longest row
N_MAX = (1 << 31) - 1
PX = np.array([-3, -2, -1, 0, 1, 2, 3], np.float64) * 0.25   # x, period 7
PG = np.array([1.0, 0.5, 2.0, 1.5, 0.75])                     # gamma, period 5
PB = np.array([0.0, 0.25, -0.5])                               # beta, period 3
PD = np.array([0.5, -1.0, 0.25])                               # dy, period 3
L = 105  # a common period of all four


def _periodic_sum(f):
    """sum over j < N_MAX of f(j) for f given over one common period."""
    full, rem = divmod(N_MAX, L)
    return full * f.sum() + f[:rem].sum()


def _tiled(pattern, n, device):
    import torch
    reps = -(-n // len(pattern))
    t = torch.tensor(pattern, dtype=torch.float32, device=device).to(torch.bfloat16)
    return t.repeat(reps)[:n].contiguous()


def _at(pattern, j):
    return pattern[np.asarray(j) % len(pattern)]


@pytest.mark.parametrize("kind", ["rms", "ln"])
def test_longest_row(device, kind):
    import torch
    ln = kind == "ln"
    eps = 1e-5
    N = N_MAX
    # one period of each pattern, laid over the common period
    j = np.arange(L)
    x, g, b, d = _at(PX, j), _at(PG, j), _at(PB, j), _at(PD, j)
    if ln:
        mean = _periodic_sum(x) / N
        m2 = _periodic_sum(x * x) - 2 * mean * _periodic_sum(x) + N * mean * mean
    else:
        mean = 0.0
        m2 = _periodic_sum(x * x)
    rstd = 1.0 / np.sqrt(m2 / N + eps)
    # backward row sums: c1 = sum g xhat / N, c2 = sum g / N with g = dy * gamma
    gg = d * g
    c1 = rstd * (_periodic_sum(gg * x) - mean * _periodic_sum(gg)) / N
    c2 = _periodic_sum(gg) / N if ln else 0.0

    xt = _tiled(PX, N, device).view(1, N)
    gt = _tiled(PG, N, device)
    bt = _tiled(PB, N, device) if ln else None
    dyt = _tiled(PD, N, device).view(1, N)
    y = torch.empty_like(xt)
    dx = torch.empty_like(xt)
    rs = torch.empty(1, device=device)
    mu = torch.empty(1, device=device) if ln else None
    dg = torch.empty(N, device=device)
    db = torch.empty(N, device=device) if ln else None
    code = rn.NORM_DTYPE_BF16
    for bwd in (False, True):
        p = rn.norm_plan(bwd, ln, 1, N, code)
        assert p.path in (rn.NORM_PATH_SPLIT, rn.NORM_PATH_GENERIC) and p.grid >= 256
    if ln:
        rn.norm_ln_fwd(xt, gt, bt, y, mu, rs, eps=eps)
        rn.norm_ln_bwd(dyt, xt, gt, mu, rs, dx, dg, db)
    else:
        rn.norm_rms_fwd(xt, gt, y, rs, eps=eps)
        rn.norm_rms_bwd(dyt, xt, gt, rs, dx, dg)
    torch.cuda.synchronize(device)

    # the statistics: sums over 2^31 terms; the merge's longest run of fp32 additions is
    # one lane's share of the ~2^20 slices plus the slices' own and the wavefront's trees
    n_run = N // (256 * 8) // 64 + 64 + 256 + 8
    tol_stat = n_run * U
    assert abs(rs.item() - rstd) <= tol_stat * rstd, (rs.item(), rstd)
    if ln:
        assert abs(mu.item() - mean) <= tol_stat * np.sqrt(m2 / N), (mu.item(), mean)

    rng = np.random.default_rng(31)
    idx = np.unique(np.concatenate([
        np.arange(64), N - 1 - np.arange(64), (1 << 30) + np.arange(-32, 32),
        (1 << 31) - (1 << 20) + np.arange(64), rng.integers(0, N, 512)]))
    it = torch.as_tensor(idx, device=device)
    xs, gs, ds = _at(PX, idx), _at(PG, idx), _at(PD, idx)
    xh = (xs - mean) * rstd
    y_ref = xh * gs + (_at(PB, idx) if ln else 0.0)
    dx_ref = rstd * (ds * gs - c2 - xh * c1)
    # y and dx: the bf16 output bound of every parity test; the statistics' error above
    # adds at most about 1e-3 of a unit value, well inside it
    y_got = to_host64(y.view(-1).index_select(0, it))
    dx_got = to_host64(dx.view(-1).index_select(0, it))
    assert np.all(np.abs(y_got - y_ref) <= TOL_BF16 * np.maximum(1.0, np.abs(y_ref)))
    assert np.all(np.abs(dx_got - dx_ref) <= TOL_BF16 * np.maximum(1.0, np.abs(dx_ref)))
    # one row: dgamma_j = dy_j * xhat_j (xhat carries rstd's error), dbeta_j = dy_j exactly
    dg_got = dg.index_select(0, it).double().cpu().numpy()
    dg_ref = ds * xh
    assert np.all(np.abs(dg_got - dg_ref) <= (tol_stat + 4 * U) * np.abs(dg_ref) + 1e-30)
    if ln:
        assert np.array_equal(db.index_select(0, it).double().cpu().numpy(), ds)


# ------------------------------------------------------------ tensors beyond 4 GiB
@pytest.mark.parametrize("kind", ["rms", "ln"])
def test_tensors_beyond_4gib(device, kind):
    """[2^20 + 7, 4096] bf16: 8 GiB per tensor, rows past the 4 GiB byte offset; the
    rows repeat a block of 13 generated rows."""
    import torch
    ln = kind == "ln"
    B, M, N = 13, (1 << 20) + 7, 4096
    w = gen.Workload(f"big_{kind}", kind, "bf16", B, N, 1e-5, x_mean=0.2, x_std=1.1,
                     config=12)
    inp = gen.make_inputs(w)
    orc = oracle.get()
    reps = -(-M // B)
    x = to_device(inp["x"], "bf16", device).repeat(reps, 1)[:M].contiguous()
    dy = to_device(inp["dy"], "bf16", device).repeat(reps, 1)[:M].contiguous()
    g = to_device(inp["gamma"], "bf16", device)
    b = to_device(inp["beta"], "bf16", device) if ln else None
    y, dx = torch.empty_like(x), torch.empty_like(x)
    rs = torch.empty(M, device=device)
    mu = torch.empty(M, device=device) if ln else None
    dg = torch.empty(N, device=device)
    db = torch.empty(N, device=device) if ln else None
    if ln:
        rn.norm_ln_fwd(x, g, b, y, mu, rs, eps=w.eps)
        rn.norm_ln_bwd(dy, x, g, mu, rs, dx, dg, db)
    else:
        rn.norm_rms_fwd(x, g, y, rs, eps=w.eps)
        rn.norm_rms_bwd(dy, x, g, rs, dx, dg)
    torch.cuda.synchronize(device)

    # rows around the 4 GiB byte offset (row 2^19) and the last ones
    rows = np.unique(np.concatenate([np.arange(B), (1 << 19) + np.arange(-3, 4),
                                     M - 1 - np.arange(B), [(1 << 20) - 1, 1 << 20]]))
    it = torch.as_tensor(rows, device=device)
    br = rows % B
    if ln:
        y_ref, mean_ref, rstd_ref = orc.ln_fwd(inp["x"], inp["gamma"], inp["beta"], w.eps)
        dx_ref = orc.ln_bwd_dx(inp["dy"], inp["x"], inp["gamma"], w.eps)
    else:
        y_ref, rstd_ref = orc.rms_fwd(inp["x"], inp["gamma"], w.eps)
        dx_ref = orc.rms_bwd_dx(inp["dy"], inp["x"], inp["gamma"], w.eps)
    y_got = to_host64(y.index_select(0, it))
    dx_got = to_host64(dx.index_select(0, it))
    assert np.all(np.abs(y_got - y_ref[br]) <= TOL_BF16 * np.maximum(1.0, np.abs(y_ref[br])))
    assert np.all(np.abs(dx_got - dx_ref[br]) <= TOL_BF16 * np.maximum(1.0, np.abs(dx_ref[br])))
    rs_got = rs.index_select(0, it).double().cpu().numpy()
    assert np.all(np.abs(rs_got - rstd_ref[br]) <= 1e-5 * rstd_ref[br])

    # column sums over all M rows: whole blocks plus the rows left over
    full, rem = divmod(M, B)
    if ln:
        gb, bb, _, _ = orc.ln_dgamma_dbeta(inp["dy"], inp["x"], w.eps)
        gr, br_, _, _ = orc.ln_dgamma_dbeta(inp["dy"][:rem], inp["x"][:rem], w.eps)
        refs = [(dg, full * gb + gr), (db, full * bb + br_)]
        mean_b, rstd_b = mean_ref, rstd_ref
    else:
        gb, _ = orc.rms_dgamma(inp["dy"], inp["x"], w.eps)
        gr, _ = orc.rms_dgamma(inp["dy"][:rem], inp["x"][:rem], w.eps)
        refs = [(dg, full * gb + gr)]
        mean_b, rstd_b = np.zeros(B), rstd_ref
    # worst-case fp32 bound: the longest run of additions behind one output is a
    # workgroup's rows (one partial row per workgroup of the plan) plus the reduction of
    # the partial rows and the trees inside a workgroup
    p = rn.norm_plan(True, ln, M, N, rn.NORM_DTYPE_BF16)
    n_run = -(-M // p.partial_rows) + p.partial_rows + 64
    x64 = gen.bf16_to_f32(inp["x"]).astype(np.float64)
    d64 = gen.bf16_to_f32(inp["dy"]).astype(np.float64)
    t = [np.abs(d64 * (x64 - mean_b[:, None]) * rstd_b[:, None]), np.abs(d64)]
    for (got, ref), ta in zip(refs, t):
        abs_sum = full * ta.sum(axis=0) + ta[:rem].sum(axis=0)
        err = np.abs(got.double().cpu().numpy() - ref)
        assert np.all(err <= n_run * U * abs_sum + 1e-30), float(np.max(err / (abs_sum + 1e-30)))
