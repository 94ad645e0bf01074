"""The C ABI on a host without a GPU: the library loads, exports what include/rownorm.h
declares, rejects every invalid argument before any HIP call, and plans/sizes
workspaces as a pure function.  Every call below fails validation (or is a pure query),
so no kernel is ever launched."""
import ctypes
import os
import re

import pytest

import row_normalization_norm_amd as rn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rownorm.h")

BF16, F32, F16 = rn.NORM_DTYPE_BF16, rn.NORM_DTYPE_F32, rn.NORM_DTYPE_F16
A = 0x10000  # a 16-byte-aligned fake address: only ever passed to calls that fail validation


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_][a-z0-9_]*\s*\*?\s*(norm_[a-z0-9_]+)\s*\(",
                                 text, flags=re.M)))


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) == 21, names
    lib = rn.lib()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in rownorm.h but not exported"
    assert set(names) == set(rn.SIGNATURES), "binding signatures out of sync with the header"


def test_stream_reference_validation():
    """The measurement aid checks its arguments on the host like the norm entry points."""
    f = rn.lib().norm_stream_reference
    assert f(2, A, A, A, 16, None) == rn.NORM_ERR_BAD_OPTION
    assert f(0, A, None, A, -1, None) == rn.NORM_ERR_BAD_SHAPE
    assert f(0, A, None, A, 0, None) == rn.NORM_OK  # nothing to do, nothing enqueued
    assert f(0, None, None, A, 16, None) == rn.NORM_ERR_NULL_PTR
    assert f(1, A, None, A, 16, None) == rn.NORM_ERR_NULL_PTR
    assert f(0, A + 8, None, A, 16, None) == rn.NORM_ERR_MISALIGNED
    assert f(1, A, A + 4, A, 16, None) == rn.NORM_ERR_MISALIGNED


def test_status_strings():
    for s in range(0, 10):
        assert rn.status_string(s)
    assert rn.status_string(0) == "ok"
    assert rn.status_string(99) == "unknown status"


CLUSTER = rn.Options(path=rn.NORM_PATH_CLUSTER)
SPLIT = rn.Options(path=rn.NORM_PATH_SPLIT)


def rms_fwd(**kw):
    a = dict(x=A, gamma=A, y=A, rstd=A, M=4, N=64, eps=1e-6, dtype=BF16, ws=None, ws_bytes=0,
             opt=None)
    a.update(kw)
    args = (a["x"], a["gamma"], a["y"], a["rstd"], a["M"], a["N"], a["eps"], a["dtype"], a["ws"],
            a["ws_bytes"], None)
    if a["opt"] is not None:
        return rn.lib().norm_rms_fwd_ex(*args, ctypes.byref(a["opt"]))
    return rn.lib().norm_rms_fwd(*args)


def ln_fwd(**kw):
    a = dict(x=A, gamma=A, beta=A, y=A, mean=A, rstd=A, M=4, N=64, eps=1e-6, dtype=BF16, ws=None,
             ws_bytes=0)
    a.update(kw)
    return rn.lib().norm_ln_fwd(a["x"], a["gamma"], a["beta"], a["y"], a["mean"], a["rstd"],
                                a["M"], a["N"], a["eps"], a["dtype"], a["ws"], a["ws_bytes"], None)


def rms_bwd(**kw):
    a = dict(dy=A, x=A, gamma=A, rstd=A, dx=A, dgamma=A, M=4, N=64, dtype=BF16, ws=A,
             ws_bytes=1 << 30)
    a.update(kw)
    return rn.lib().norm_rms_bwd(a["dy"], a["x"], a["gamma"], a["rstd"], a["dx"], a["dgamma"],
                                 a["M"], a["N"], a["dtype"], a["ws"], a["ws_bytes"], None)


def ln_bwd(**kw):
    a = dict(dy=A, x=A, gamma=A, mean=A, rstd=A, dx=A, dgamma=A, dbeta=A, M=4, N=64, dtype=BF16,
             ws=A, ws_bytes=1 << 30)
    a.update(kw)
    return rn.lib().norm_ln_bwd(a["dy"], a["x"], a["gamma"], a["mean"], a["rstd"], a["dx"],
                                a["dgamma"], a["dbeta"], a["M"], a["N"], a["dtype"], a["ws"],
                                a["ws_bytes"], None)


@pytest.mark.parametrize("call,kw,status", [
    (rms_fwd, dict(x=None), rn.NORM_ERR_NULL_PTR),
    (rms_fwd, dict(gamma=None), rn.NORM_ERR_NULL_PTR),
    (rms_fwd, dict(y=None), rn.NORM_ERR_NULL_PTR),
    (rms_fwd, dict(M=-1), rn.NORM_ERR_BAD_SHAPE),
    (rms_fwd, dict(N=0), rn.NORM_ERR_BAD_SHAPE),
    (rms_fwd, dict(N=1 << 31), rn.NORM_ERR_BAD_SHAPE),
    (rms_fwd, dict(M=1 << 60, N=1 << 20), rn.NORM_ERR_BAD_SHAPE),
    (rms_fwd, dict(dtype=7), rn.NORM_ERR_BAD_DTYPE),
    (rms_fwd, dict(eps=-1e-6), rn.NORM_ERR_BAD_EPS),
    (rms_fwd, dict(eps=float("nan")), rn.NORM_ERR_BAD_EPS),
    (rms_fwd, dict(eps=float("inf")), rn.NORM_ERR_BAD_EPS),
    (rms_fwd, dict(x=A + 1), rn.NORM_ERR_MISALIGNED),
    (rms_fwd, dict(rstd=A + 2), rn.NORM_ERR_MISALIGNED),
    (rms_fwd, dict(dtype=F32, y=A + 2), rn.NORM_ERR_MISALIGNED),
    (ln_fwd, dict(beta=None), rn.NORM_ERR_NULL_PTR),
    (ln_fwd, dict(mean=A + 1), rn.NORM_ERR_MISALIGNED),
    # the split-row forward, when asked for, needs its workspace (without options a
    # missing or short forward workspace selects a plan that needs none)
    (rms_fwd, dict(M=1024, N=262144, opt=CLUSTER), rn.NORM_ERR_NULL_PTR),
    (rms_fwd, dict(M=4, N=4096, opt=SPLIT), rn.NORM_ERR_NULL_PTR),
    (rms_fwd, dict(M=4, N=5001, ws=A, ws_bytes=64, opt=SPLIT), rn.NORM_ERR_WORKSPACE_TOO_SMALL),
    (rms_fwd, dict(M=1024, N=262144, ws=A, ws_bytes=64, opt=CLUSTER),
     rn.NORM_ERR_WORKSPACE_TOO_SMALL),
    (ln_fwd, dict(M=1024, N=262144, ws=A + 8, ws_bytes=1 << 20), rn.NORM_ERR_MISALIGNED),
    (rms_bwd, dict(dy=None), rn.NORM_ERR_NULL_PTR),
    (rms_bwd, dict(rstd=None), rn.NORM_ERR_NULL_PTR),
    (rms_bwd, dict(dgamma=None), rn.NORM_ERR_NULL_PTR),
    (rms_bwd, dict(ws=None), rn.NORM_ERR_NULL_PTR),
    (rms_bwd, dict(ws_bytes=16), rn.NORM_ERR_WORKSPACE_TOO_SMALL),
    (rms_bwd, dict(ws=A + 4), rn.NORM_ERR_MISALIGNED),
    (rms_bwd, dict(N=-5), rn.NORM_ERR_BAD_SHAPE),
    (rms_bwd, dict(dtype=-1), rn.NORM_ERR_BAD_DTYPE),
    (ln_bwd, dict(mean=None), rn.NORM_ERR_NULL_PTR),
    (ln_bwd, dict(dbeta=None), rn.NORM_ERR_NULL_PTR),
    (ln_bwd, dict(dbeta=A + 1), rn.NORM_ERR_MISALIGNED),
    (ln_bwd, dict(ws_bytes=0), rn.NORM_ERR_WORKSPACE_TOO_SMALL),
    # type pairs: 16-bit activations may take fp32 gamma/beta; nothing else mixes
    (rms_fwd, dict(dtype=rn.dtype_mixed(F32, BF16)), rn.NORM_ERR_BAD_DTYPE),
    (rms_fwd, dict(dtype=rn.dtype_mixed(BF16, F16)), rn.NORM_ERR_BAD_DTYPE),
    (rms_fwd, dict(dtype=rn.dtype_mixed(F16, BF16)), rn.NORM_ERR_BAD_DTYPE),
    (rms_fwd, dict(dtype=rn.dtype_mixed(BF16, 3)), rn.NORM_ERR_BAD_DTYPE),
    (rms_fwd, dict(dtype=3), rn.NORM_ERR_BAD_DTYPE),
    (rms_fwd, dict(dtype=BF16 | (1 << 16)), rn.NORM_ERR_BAD_DTYPE),
    (ln_bwd, dict(dtype=rn.dtype_mixed(F32, F16)), rn.NORM_ERR_BAD_DTYPE),
    # fp32 parameters need 4-byte alignment even with 2-byte activations
    (rms_fwd, dict(dtype=rn.dtype_mixed(BF16, F32), gamma=A + 2), rn.NORM_ERR_MISALIGNED),
    (ln_fwd, dict(dtype=rn.dtype_mixed(F16, F32), beta=A + 2), rn.NORM_ERR_MISALIGNED),
    (ln_bwd, dict(dtype=rn.dtype_mixed(F16, F32), gamma=A + 2), rn.NORM_ERR_MISALIGNED),
    (rms_fwd, dict(dtype=F16, x=A + 1), rn.NORM_ERR_MISALIGNED),
])
def test_validation_rejects(call, kw, status):
    assert call(**kw) == status


def test_fused_residual_validation():
    """The residual-add entry points check their extra pointers like the others."""
    lib = rn.lib()
    fwd = lambda **kw: lib.norm_rms_fwd_add(kw.get("x", A), kw.get("res", A), A, A,
                                            kw.get("sum", A), A, kw.get("M", 4), 64, 1e-6, BF16,
                                            None, 0, None, None)
    lnf = lambda **kw: lib.norm_ln_fwd_add(A, kw.get("res", A), A, A, A, kw.get("sum", A), A, A,
                                           kw.get("M", 4), 64, 1e-6, BF16, None, 0, None, None)
    bwd = lambda **kw: lib.norm_rms_bwd_add(A, A, A, A, kw.get("dsum", A), A, A, 4, 64, BF16, A,
                                            1 << 30, None, None)
    lnb = lambda **kw: lib.norm_ln_bwd_add(A, A, A, A, A, kw.get("dsum", A), A, A, A, 4, 64,
                                           kw.get("dtype", BF16), A, 1 << 30, None, None)
    assert fwd(res=None) == rn.NORM_ERR_NULL_PTR
    assert fwd(sum=None) == rn.NORM_ERR_NULL_PTR
    assert lnf(res=None) == rn.NORM_ERR_NULL_PTR
    assert fwd(res=A + 1) == rn.NORM_ERR_MISALIGNED
    assert lnf(sum=A + 1) == rn.NORM_ERR_MISALIGNED
    assert bwd(dsum=A + 1) == rn.NORM_ERR_MISALIGNED
    assert lnb(dtype=rn.dtype_mixed(F32, F16)) == rn.NORM_ERR_BAD_DTYPE
    # an empty batch needs no residual buffers and enqueues nothing
    assert fwd(M=0, x=None, res=None, sum=None) == rn.NORM_OK


def test_bad_options_rejected():
    lib = rn.lib()
    bad = [rn.Options(path=9), rn.Options(lanes_per_row=-1),
           rn.Options(path=rn.NORM_PATH_ROWS, lanes_per_row=48, vecs_per_lane=1),
           rn.Options(path=rn.NORM_PATH_ROWS, lanes_per_row=8, vecs_per_lane=1),  # cannot cover N
           rn.Options(dgamma_mode=5),
           rn.Options(cluster_size=64),  # above the largest cluster
           rn.Options(path=rn.NORM_PATH_CLUSTER, cluster_size=3)]  # not a power of two
    for o in bad:
        st = lib.norm_rms_fwd_ex(A, A, A, A, 4, 4096, 1e-6, BF16, None, 0, None, ctypes.byref(o))
        assert st == rn.NORM_ERR_BAD_OPTION, (o.path, o.lanes_per_row, o.vecs_per_lane)
    # atomic dgamma is only offered on the ROWS path
    o = rn.Options(path=rn.NORM_PATH_SPLIT, dgamma_mode=rn.NORM_DGAMMA_ATOMIC_ROW)
    st = lib.norm_rms_bwd_ex(A, A, A, A, A, A, 4, 4096, BF16, A, 1 << 30, None, ctypes.byref(o))
    assert st == rn.NORM_ERR_BAD_OPTION
    # a larger backward grid means more partial rows: the default-sized workspace is then
    # rejected instead of overflowed
    o = rn.Options(grid=4096)
    need_default = rn.norm_bwd_workspace_size(1 << 20, 1024, False, BF16)
    need = rn.norm_bwd_workspace_size(1 << 20, 1024, False, BF16, o)
    assert need > need_default
    st = lib.norm_rms_bwd_ex(A, A, A, A, A, A, 1 << 20, 1024, BF16, A, need_default, None,
                             ctypes.byref(o))
    assert st == rn.NORM_ERR_WORKSPACE_TOO_SMALL


def test_plan_shape_classes():
    # non-power-of-2 N = 384 (bf16): 48 vectors, less than one vector of padding per lane;
    # the forward packs several rows per wavefront (16 lanes x 3 vectors).  The backward's
    # tuned mapping is one 64-lane row per wavefront, one vector per lane (measured 4 %
    # faster on MI355X than 16 x 3 in the pipelined kernel, 16 lanes idle); the rules
    # without the table still pack rows.
    for bwd in (False, True):
        p = rn.norm_plan(bwd, False, 262144, 384, BF16)
        cover = p.lanes_per_row * p.vecs_per_lane
        assert p.path == rn.NORM_PATH_ROWS and 48 <= cover < 48 + p.lanes_per_row
        assert p.lanes_per_row <= (64 if bwd else 32)
        q = rn.norm_plan(bwd, False, 262144 + 1, 384, BF16, options=rn.Options(grid=256))
        assert q.lanes_per_row <= 64
    # very long rows are split over a cluster of workgroups (the backward from 131072
    # bf16 columns, the forward beyond one workgroup's 16 vectors per lane)
    for bwd, N in ((False, 262144), (True, 131072)):
        p = rn.norm_plan(bwd, False, 2048, N, BF16)
        assert p.path == rn.NORM_PATH_CLUSTER and p.cluster_size >= 2 and p.cluster_rows >= 1
    # the two-pass column-sliced backward remains available
    p = rn.norm_plan(True, False, 2048, 131072, BF16, options=rn.Options(path=rn.NORM_PATH_SPLIT))
    assert p.path == rn.NORM_PATH_SPLIT and p.partial_rows >= 1
    # misaligned pointers or N not a multiple of the vector fall back to element loads:
    # the register-resident scalar kernels for short rows, the sliced passes beyond
    assert rn.norm_plan(False, True, 100, 3000, BF16, aligned16=False).path == rn.NORM_PATH_GENERIC
    assert rn.norm_plan(False, True, 100, 3071, BF16).path == rn.NORM_PATH_GENERIC
    assert rn.norm_plan(True, True, 100, 7, F32).path == rn.NORM_PATH_GENERIC
    for N, aligned in ((4096, False), (4095, True), (1 << 22, False)):
        p = rn.norm_plan(False, True, 100, N, BF16, aligned16=aligned)
        slices = -(-N // 2048)  # 256 lanes x 8 elements per slice
        # about 8192 workgroups in all, each with 4 rows or more
        row_blocks = min(-(-8192 // slices), -(-100 // 4))
        assert p.path == rn.NORM_PATH_SPLIT and p.grid == slices * row_blocks, (N, p.grid)
        assert p.workspace_bytes > 0
    # long rows past the reach of a cluster take the sliced passes in both directions,
    # spread over many workgroups even for a single row
    for bwd in (False, True):
        p = rn.norm_plan(bwd, False, 1, 1 << 22, BF16)
        assert p.path == rn.NORM_PATH_SPLIT and p.grid == (1 << 22) // 4096, (bwd, p.grid)
    # every plan's lanes x vectors covers the row with less than one vector slot of padding
    for N in (256, 384, 512, 768, 1024, 2048, 4096, 8192, 16384, 65536):
        for dt, epv in ((BF16, 8), (F32, 4)):
            for bwd in (False, True):
                p = rn.norm_plan(bwd, True, (1 << 27) // N, N, dt)
                if p.path == rn.NORM_PATH_ROWS:
                    cover = p.lanes_per_row * p.vecs_per_lane
                    assert N // epv <= cover < N // epv + p.lanes_per_row


def test_workspace_size():
    ws = rn.norm_bwd_workspace_size
    for ln in (False, True):
        for dt in (BF16, F32):
            prev = 0
            for M in (0, 1, 7, 100, 4096, 65536, 1 << 20):
                s = ws(M, 4096, ln, dt)
                assert s >= prev, "workspace size must not shrink as M grows"
                prev = s
            # per-shape query: every row length needs room for its partial rows
            for N in (1, 8, 384, 1000, 4096, 32768, 131072):
                assert ws(4096, N, ln, dt) >= N * 4 * (2 if ln else 1)
    # LayerNorm needs room for dbeta partials too
    assert ws(4096, 1024, True, BF16) > ws(4096, 1024, False, BF16)
    # the query is enough for the aligned plan and for the scalar plan
    for (M, N) in ((4096, 1024), (65536, 4096), (2048, 131072), (333, 7)):
        need = ws(M, N, True, BF16)
        for al in (True, False):
            assert rn.norm_plan(True, True, M, N, BF16, aligned16=al).workspace_bytes <= need
    # atomic comparison modes need no workspace
    o = rn.Options(dgamma_mode=rn.NORM_DGAMMA_ATOMIC_ROW)
    assert ws(4096, 1024, True, BF16, o) == 0
    # an invalid shape sizes to 0
    assert ws(-1, 1024, True, BF16) == 0


def test_cluster_plans():
    """Rows longer than one workgroup's registers are split over a cluster of workgroups,
    each owning a column slice; forward and backward both, bf16 and fp32."""
    cases = [(False, BF16, 262144), (False, F32, 131072), (True, BF16, 131072), (True, BF16, 65536),
             (True, BF16, 32768), (True, F32, 65536), (True, F32, 32768)]
    for bwd, dt, N in cases:
            M = (1 << 27) // N
            p = rn.norm_plan(bwd, True, M, N, dt)
            assert p.path == rn.NORM_PATH_CLUSTER, (bwd, dt, N, p.path)
            epv = 8 if dt == BF16 else 4
            slice_vecs = N // epv // p.cluster_size
            assert slice_vecs <= p.lanes_per_row * p.vecs_per_lane < slice_vecs + p.lanes_per_row
            assert p.grid % p.cluster_size == 0
            if bwd:
                assert p.partial_rows == p.grid // p.cluster_size
            ws = (rn.norm_bwd_workspace_size if bwd else rn.norm_fwd_workspace_size)(M, N, True, dt)
            assert ws >= p.workspace_bytes > 0
    # shorter rows stay in one workgroup's registers (no forward workspace); the forward
    # can keep a whole 256 KiB row (1024 lanes x 16 vectors), though at these lengths the
    # tuned planner splits it over a cluster
    assert rn.norm_plan(False, True, 8192, 16384, BF16).path == rn.NORM_PATH_ROWS
    for dt, N in ((BF16, 131072), (F32, 65536)):
        p = rn.norm_plan(False, True, 2048, N, dt, options=rn.Options(path=rn.NORM_PATH_ROWS))
        assert (p.path, p.lanes_per_row, p.vecs_per_lane) == (rn.NORM_PATH_ROWS, 1024, 16)
        assert rn.norm_plan(False, True, 2048, N, dt).path == rn.NORM_PATH_CLUSTER
    # untuned: 12000 vectors fit 1024 x 12; 10000 vectors fit no wide mapping
    assert rn.norm_plan(False, True, 64, 12000 * 8, BF16).vecs_per_lane == 12
    assert rn.norm_plan(False, True, 64, 10000 * 8, BF16).path == rn.NORM_PATH_CLUSTER
    assert rn.norm_plan(True, True, 16384, 8192, BF16).path == rn.NORM_PATH_ROWS


def test_lds_partial_mappings():
    """1024-lane backward mappings with 2 or 4 vectors per lane keep their per-column
    partials in LDS; they exist where those partials fit in 160 KiB (4 bytes x 1024 lanes
    x vectors x elements per vector x 1 or 2 sums), and the planner uses them for rows
    up to 4096 vectors, else splits the row over a cluster."""
    rows = rn.NORM_PATH_ROWS

    def built(ln, dt, lpr, vpl):
        epv = 8 if dt == BF16 else 4
        N = (lpr * vpl - 7) * epv
        try:
            rn.norm_plan(True, ln, 1000, N, dt,
                         options=rn.Options(path=rows, lanes_per_row=lpr, vecs_per_lane=vpl))
            return True
        except rn.NormError:
            return False

    for ln in (False, True):
        for dt in (BF16, F32):
            epv = 8 if dt == BF16 else 4
            for vpl in (2, 4):
                lds = 4 * 1024 * vpl * epv * (2 if ln else 1)
                assert built(ln, dt, 1024, vpl) == (lds <= 160 * 1024 and vpl * epv * (2 if ln else 1) >= 16), \
                    (ln, dt, vpl)
    # tuned long rows that now stay in one workgroup
    p = rn.norm_plan(True, True, 8192, 16384, BF16)
    assert (p.path, p.lanes_per_row, p.vecs_per_lane) == (rows, 1024, 2)
    p = rn.norm_plan(True, False, 8192, 16384, BF16)
    assert p.path == rows and p.lanes_per_row * p.vecs_per_lane == 2048
    # untuned lengths: 3500 vectors fit 1024 x 4 where it is built (RMSNorm bf16), not for
    # LayerNorm bf16; 2500 vectors have no 1024 x 3 mapping
    assert rn.norm_plan(True, False, 4096, 3500 * 8, BF16).path == rows
    assert rn.norm_plan(True, True, 4096, 3500 * 8, BF16).path == rn.NORM_PATH_CLUSTER
    assert rn.norm_plan(True, False, 4096, 2500 * 8, BF16).path == rn.NORM_PATH_CLUSTER
    # the aligned forward of 4096 bf16 columns needs no workspace; the size query covers
    # misaligned pointers too, whose plan (element loads, the sliced passes) needs one
    assert rn.norm_plan(False, True, 65536, 4096, BF16).workspace_bytes == 0
    assert rn.norm_fwd_workspace_size(65536, 4096, True, BF16) == \
        rn.norm_plan(False, True, 65536, 4096, BF16, aligned16=False).workspace_bytes > 0


def test_type_pairs_plan_like_their_activations():
    """The plan and the workspace depend on the activations' element size only: fp16 plans
    like bf16, and fp32 gamma/beta beside 16-bit activations change neither."""
    for bwd in (False, True):
        for ln in (False, True):
            for M, N in ((4096, 1024), (65536, 4096), (262144, 384), (2048, 131072), (77, 1000)):
                ref = rn.norm_plan(bwd, ln, M, N, BF16)
                for code in (F16, rn.dtype_mixed(BF16, F32), rn.dtype_mixed(F16, F32)):
                    p = rn.norm_plan(bwd, ln, M, N, code)
                    assert (p.path, p.lanes_per_row, p.vecs_per_lane, p.grid, p.cluster_size) == \
                        (ref.path, ref.lanes_per_row, ref.vecs_per_lane, ref.grid, ref.cluster_size)
                    size = rn.norm_bwd_workspace_size if bwd else rn.norm_fwd_workspace_size
                    assert size(M, N, ln, code) == size(M, N, ln, BF16)


def test_rejected_forced_plans_are_the_unbuilt_ones():
    """The GPU parity tests force only plans the planner accepts (tests/plan_cases.py);
    the rest must be exactly the combinations with no compiled kernel."""
    import plan_cases as pc
    pairs = [("bf16", None), ("f32", None), ("f16", None), ("bf16", "f32"), ("f16", "f32")]
    # Row mappings: a 1024-lane backward mapping with more than one vector per lane exists
    # only with its per-column partials in LDS, which needs >= 16 of them per lane and
    # 1024 lanes x 4 bytes x that many to fit in 160 KiB.
    def unbuilt(k, d, dr, lpr, vpl):
        sums = vpl * pc.epv(d) * (2 if k == "ln" else 1)
        return dr == "bwd" and lpr == 1024 and vpl > 1 and not (
            sums >= 16 and 1024 * sums * 4 <= 160 * 1024)
    rejected = pc.mapping_cases(pairs, accepted=False)
    expect = [c for c in pc.all_mapping_cases(pairs) if unbuilt(c[0], c[1], c[3], c[4], c[5])]
    assert sorted(rejected, key=str) == sorted(expect, key=str)
    assert len(rejected) == 5  # RMSNorm fp32 1024x2; LayerNorm 16-bit 1024x4 (four pairs)
    # Split rows: a member's slice (N / elements per vector / C vectors) must be covered by
    # a compiled (threads x vectors) member mapping for the step's row count, with less
    # than one vector of padding per lane and at most 4 (forward) / 2 (backward) vectors.
    maps = pc.compiled_cluster_mappings()

    def covered(direction, sv, R):
        vmax = 4 if direction == "fwd" else 2
        return any(t * v >= sv and t * v - sv < t for dr, t, v, r in maps
                   if dr == direction and r == R and v <= vmax)
    rejected = pc.cluster_cases(pairs, accepted=False)
    expect = [c for c in pc.all_cluster_cases(pairs)
              if not all(covered(dr, c[3] // pc.epv(c[1]) // c[4], c[5]) for dr in ("fwd", "bwd"))]
    assert sorted(rejected, key=str) == sorted(expect, key=str)
    assert rejected and all(c[3] == 65536 for c in rejected)


def test_noalloc_validation():
    """The entry point that allocates nothing validates like norm_ln_bwd, and rejects a
    shape whose plan needs more than its 32 MiB static scratch, all before any HIP call."""
    f = rn.lib().norm_ln_bwd_noalloc
    ok = dict(dy=A, x=A, g=A, mean=A, rstd=A, dx=A, dg=A, db=A, M=4096, N=4096, dt=BF16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["dy"], a["x"], a["g"], a["mean"], a["rstd"], a["dx"], a["dg"], a["db"], a["M"],
                 a["N"], a["dt"], None)
    assert call(db=None) == rn.NORM_ERR_NULL_PTR
    assert call(mean=None) == rn.NORM_ERR_NULL_PTR
    assert call(x=A + 1) == rn.NORM_ERR_MISALIGNED
    assert call(N=0) == rn.NORM_ERR_BAD_SHAPE
    assert call(dt=9) == rn.NORM_ERR_BAD_DTYPE
    # LayerNorm bf16 N = 131072 splits rows: 32 clusters x 131072 x 8 bytes of partial
    # rows alone is 32 MiB, plus the exchange words
    assert rn.norm_bwd_workspace_size(2048, 131072, True, BF16) > 32 << 20
    assert call(M=2048, N=131072) == rn.NORM_ERR_SCRATCH_TOO_SMALL
    # the benchmark's LayerNorm [65536, 4096] fits (its 16-byte-aligned plan: 8 MiB of
    # partial rows; the size query also covers misaligned pointers, which need more)
    assert rn.norm_plan(True, True, 65536, 4096, BF16).workspace_bytes <= 32 << 20


def test_binding_rejects_host_tensors():
    """The binding's first check, made before any GPU call: activations must live on a GPU."""
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    g = torch.ones(64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        rn.norm_rms_fwd(x, g, torch.empty_like(x))
    with pytest.raises(ValueError, match="2-D"):
        rn.norm_rms_fwd(x.view(-1), g, x.view(-1))
