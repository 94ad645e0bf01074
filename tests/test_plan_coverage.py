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
