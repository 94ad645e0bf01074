"""Every row length has a plan, and the forward keeps 16-byte vectors up to 8192 of them.

A forward row whose length fell between the compiled one-workgroup mappings used to be
refused (NORM_ERR_BAD_OPTION) instead of taking a longer-row plan; this walks every
length of whole 16-byte vectors up to 12000 vectors (bf16 N up to 96000, fp32 N up to
48000), both kinds and directions, for one row and for the sweep's row count.  No GPU
is needed: the planner is host code."""
import pytest

import row_normalization_norm_amd as rn

DTYPES = [("bf16", rn.NORM_DTYPE_BF16, 8), ("f32", rn.NORM_DTYPE_F32, 4)]


@pytest.mark.parametrize("dtype,code,epv", DTYPES, ids=[d[0] for d in DTYPES])
@pytest.mark.parametrize("kind", ["rms", "ln"])
@pytest.mark.parametrize("backward", [False, True], ids=["fwd", "bwd"])
def test_every_row_length_has_a_plan(dtype, code, epv, kind, backward):
    failures = []
    for nvec in range(1, 12001):
        N = nvec * epv
        for M in (1, max(1, (1 << 27) // N)):
            try:
                p = rn.norm_plan(backward, kind == "ln", M, N, code)
            except rn.NormError as e:
                failures.append((N, M, str(e)))
                continue
            if not backward and nvec <= 8192:
                # one workgroup or a cluster holds the row in 16-byte vectors
                assert p.path in (rn.NORM_PATH_ROWS, rn.NORM_PATH_CLUSTER), (N, M, p.path)
    assert not failures, failures[:10]


@pytest.mark.parametrize("backward", [False, True], ids=["fwd", "bwd"])
def test_sliced_plan_geometry(backward):
    """The sliced passes' plan at row lengths past a cluster and at long rows of elements:
    the grid covers every (slice, row) once within the grid's y limit, and the workspace
    holds the per-row table, the per-(row, slice) terms and (backward) the partial rows."""
    import random
    rnd = random.Random(7)
    shapes = [(1, (1 << 31) - 1), (3, (1 << 22) + 8), (65536, 4100), (70000, 5001), (1, 3073),
              (2, (1 << 20) + 8), (1 << 20, 4099)]
    shapes += [(rnd.randint(1, 1 << 18), rnd.randint(3073, 1 << 23)) for _ in range(200)]
    for M, N in shapes:
        for code, size, epv in ((rn.NORM_DTYPE_BF16, 2, 8), (rn.NORM_DTYPE_F32, 4, 4)):
            for ln in (False, True):
                for aligned in (False, True):
                    p = rn.norm_plan(backward, ln, M, N, code, aligned16=aligned)
                    vec = aligned and N % epv == 0
                    if p.path not in (rn.NORM_PATH_SPLIT, rn.NORM_PATH_GENERIC) or p.block != 256:
                        continue  # a row, cluster or register-resident scalar plan
                    units = N // epv if vec else N
                    slices = -(-units // (512 if vec else 2048))
                    assert p.grid % slices == 0, (M, N, p.grid, slices)
                    row_blocks = p.grid // slices
                    assert 1 <= row_blocks <= min(M, 65535)
                    need = 8 * M + 8 * M * slices
                    if backward:
                        assert 1 <= p.partial_rows <= min(M, 65535)
                        need += 4 * p.partial_rows * N * (2 if ln else 1)
                    assert p.workspace_bytes >= need, (M, N, p.workspace_bytes, need)


def test_forced_options_are_honoured():
    """The seeded draws of forced options the GPU tests run (test_gpu_random_options):
    every draw the planner accepts takes the path, mapping, cluster size and rows per
    step it was given, and enough of them are accepted for those tests to mean something.
    A forced cluster may still end on the sliced passes only when the cluster does not
    fit the device, which the planner reports through norm_cluster_resident."""
    from test_gpu_random_options import _CODE, _cases
    accepted = 0
    for i, kind, dtype, pdtype, M, N, fo, bo, _, _ in _cases(20261203, 600):
        code = rn.dtype_mixed(_CODE[dtype], _CODE[pdtype]) if pdtype else _CODE[dtype]
        plans = []
        try:
            for bwd, o in ((False, fo), (True, bo)):
                plans.append((bwd, o, rn.norm_plan(bwd, kind == "ln", M, N, code, True, o)))
        except rn.NormError as e:
            assert e.status == rn.NORM_ERR_BAD_OPTION, (i, str(e))
            continue
        accepted += 1
        for bwd, o, p in plans:
            if o is None or o.path == rn.NORM_PATH_AUTO:
                continue
            where = (i, bwd, kind, dtype, M, N)
            if o.path == rn.NORM_PATH_GENERIC and bwd:
                # the backward's long rows of elements take the sliced passes over elements
                assert p.path in (rn.NORM_PATH_GENERIC, rn.NORM_PATH_SPLIT), where
            else:
                assert p.path == o.path, (where, p.path)
            if o.path == rn.NORM_PATH_ROWS:
                if o.lanes_per_row:
                    assert p.lanes_per_row == o.lanes_per_row, where
                if o.vecs_per_lane:
                    assert p.vecs_per_lane == o.vecs_per_lane, where
            if o.path == rn.NORM_PATH_CLUSTER:
                if o.cluster_size:
                    assert p.cluster_size == o.cluster_size, where
                if o.cluster_rows:
                    assert p.cluster_rows == o.cluster_rows, where
    assert accepted >= 150, accepted
