"""Parity under options drawn at random (seeded): a forced path (register rows with a
drawn mapping and kernel, sliced passes, element loads, cluster with a drawn size, rows
per step and wait), a drawn grid, now and then an atomic dgamma, on drawn shapes, type
pairs and data (means up to 5, spreads from 0.05 to 3), x and dy now and then at an
element offset (not 16-byte aligned).  Draws the planner refuses are
left out; every other one must match the oracle on every row, forward and backward.
One test walks the cases in order and names the first that fails."""
import numpy as np

import row_normalization_norm_amd as rn
from parity import full_check
from test_gpu_parity import PAIRS, small_workload

import pytest

pytestmark = pytest.mark.gpu

_CODE = {"bf16": rn.NORM_DTYPE_BF16, "f32": rn.NORM_DTYPE_F32, "f16": rn.NORM_DTYPE_F16}


def _options(rng):
    r = rng.random()
    if r < 0.15:
        return None
    o = rn.Options()
    if r < 0.45:
        o.path = rn.NORM_PATH_ROWS
        o.lanes_per_row = int(rng.choice([0, 8, 16, 32, 64, 128, 256, 512, 1024]))
        o.vecs_per_lane = int(rng.choice([0, 1, 2, 3, 4, 5, 6, 7, 8]))
        o.pipeline = int(rng.choice([0, 1, 2]))
    elif r < 0.6:
        o.path = rn.NORM_PATH_SPLIT
    elif r < 0.72:
        o.path = rn.NORM_PATH_GENERIC
    else:
        o.path = rn.NORM_PATH_CLUSTER
        o.cluster_size = int(rng.choice([0, 2, 4, 8, 16, 32]))
        o.cluster_rows = int(rng.choice([0, 1, 2]))
        o.cluster_wait = int(rng.choice([0, 0, -1]))
    if rng.random() < 0.4:
        o.grid = int(rng.integers(1, 1025))
    if rng.random() < 0.1:
        o.dgamma_mode = int(rng.choice([rn.NORM_DGAMMA_ATOMIC_ROW, rn.NORM_DGAMMA_ATOMIC_WG]))
    return o


def _describe(o):
    if o is None:
        return "planner"
    return ", ".join(f"{f}={getattr(o, f)}" for f, _ in rn.Options._fields_
                     if f not in ("ev_start", "ev_stop") and getattr(o, f))


def _cases(seed, n):
    rng = np.random.default_rng(seed)
    for i in range(n):
        kind = ("rms", "ln")[int(rng.integers(2))]
        dtype, pdtype = PAIRS[int(rng.integers(len(PAIRS)))]
        N = int(np.exp(rng.uniform(0.0, np.log(1 << 17))))
        if rng.random() < 0.6:
            N = max(8, N // 8 * 8)
        M = int(rng.integers(1, max(2, min(600, 1_500_000 // N)) + 1))
        fo = _options(rng)
        bo = fo if rng.random() < 0.5 else _options(rng)
        x_mean = float(rng.choice([0.0, 0.3, -2.0, 5.0]))
        x_std = float(rng.choice([1.0, 1.0, 0.05, 3.0]))
        yield i, kind, dtype, pdtype, M, N, fo, bo, x_mean, x_std


def test_random_forced_plans(device):
    ran = 0
    offsets = np.random.default_rng(5)
    for i, kind, dtype, pdtype, M, N, fo, bo, x_mean, x_std in _cases(20261203, 600):
        code = rn.dtype_mixed(_CODE[dtype], _CODE[pdtype]) if pdtype else _CODE[dtype]
        # one case in five puts x and dy at an element offset: not 16-byte aligned
        off = int(offsets.integers(1, 8)) if offsets.random() < 0.2 else 0
        aligned = off * (4 if dtype == "f32" else 2) % 16 == 0
        try:
            for bwd, o in ((False, fo), (True, bo)):
                rn.norm_plan(bwd, kind == "ln", M, N, code, aligned, o)
        except rn.NormError:
            continue  # a draw the planner refuses (a mapping that does not cover N, ...)
        name = (f"case {i}: {kind} {dtype}{'+' + pdtype if pdtype else ''} {M}x{N}, "
                f"x ~ N({x_mean}, {x_std}), x and dy offset by {off}; forward "
                f"[{_describe(fo)}], backward [{_describe(bo)}]")
        print(name, flush=True)
        w = small_workload(kind, dtype, N, M=M, x_mean=x_mean, x_std=x_std, pdtype=pdtype)
        try:
            full_check(w, device, rows=np.arange(M), fwd_options=fo, bwd_options=bo,
                       x_offset=off)
        except AssertionError as e:
            raise AssertionError(f"{name}: {e}") from None
        ran += 1
    assert ran >= 150, f"only {ran} drawn cases were accepted by the planner"
