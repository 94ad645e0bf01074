"""The planner's measured table (csrc/tuned.h) is what the planner actually uses: at each
entry's own row length (M = 2^27 / N rows, the shape it was measured at) the plan has the
entry's path, mapping, kernel (plain or pipelined) and, where the entry fixes one, its
grid.  An entry that stopped
fitting (a mapping no longer built, a cluster that no longer fits the workspace rules)
would otherwise fall through to the rules without notice.  No GPU is needed."""
import os
import re

import pytest

import row_normalization_norm_amd as rn

TUNED = os.path.join(os.path.dirname(rn.__file__), "csrc", "tuned.h")
ENTRY = re.compile(r"^\s*\{(-?\d+), (-?\d+), (-?\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), "
                   r"(\d+)\},")


def entries():
    out = []
    with open(TUNED) as f:
        for line in f:
            m = ENTRY.match(line)
            if m:
                out.append(tuple(int(g) for g in m.groups()))
    return out


def test_table_parses():
    e = entries()
    assert len(e) >= 80
    # one entry per (direction, kind, element size, row length)
    assert len({t[:4] for t in e}) == len(e)


@pytest.mark.parametrize("t", entries(), ids=lambda t: "bwd%d_ln%d_b16%d_nvec%d" % t[:4])
def test_entry_is_the_plan_at_its_shape(t):
    bwd, ln, b16, nvec, path, lanes, vecs, grid, cluster, rows, pipelined = t
    dt = rn.NORM_DTYPE_BF16 if b16 else rn.NORM_DTYPE_F32
    N = nvec * (8 if b16 else 4)
    M = max(1, (1 << 27) // N)
    p = rn.norm_plan(bool(bwd), bool(ln), M, N, dt)
    assert (p.path, p.lanes_per_row, p.vecs_per_lane) == (path, lanes, vecs)
    if path == rn.NORM_PATH_CLUSTER:
        assert (p.cluster_size, p.cluster_rows) == (cluster, rows)
    if grid:
        # an explicit grid is kept, or clamped to the row groups there are
        assert 0 < p.grid <= grid
    assert p.pipelined == pipelined
