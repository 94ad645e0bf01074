"""Forced-plan test cases, split by whether the planner accepts them.

The GPU parity tests force every compiled row mapping and a grid of split-row (cluster)
sizes.  Some combinations have no compiled kernel (a 1024-lane backward mapping whose
per-column partials fit neither registers nor LDS; a split-row slice longer than any
compiled member mapping covers), and the planner rejects them with NORM_ERR_BAD_OPTION.
The GPU tests take only the accepted cases; tests/test_abi.py checks on the CPU that the
rejected ones are exactly those the rules above predict.  Asking the planner needs
librownorm.so (a pure host function); without it every case is listed, so the tests
still collect.
"""
from __future__ import annotations

import re

import row_normalization_norm_amd as rn

KINDS = ("rms", "ln")
CODE = {"f32": rn.NORM_DTYPE_F32, "bf16": rn.NORM_DTYPE_BF16, "f16": rn.NORM_DTYPE_F16}


def code_of(dtype, pdtype=None):
    return rn.dtype_mixed(CODE[dtype], CODE[pdtype]) if pdtype else CODE[dtype]


def epv(dtype):
    return 4 if dtype == "f32" else 8


def _launch_h():
    return open(rn.__file__.replace("__init__.py", "csrc/launch.h")).read()


def compiled_row_mappings():
    """(direction, lanes per row, vectors per lane) of RN_FWD_MAPPINGS / RN_BWD_MAPPINGS."""
    src = _launch_h()
    out = []
    for direction, macro in (("fwd", "RN_FWD_MAPPINGS"), ("bwd", "RN_BWD_MAPPINGS")):
        body = src[src.index(f"#define {macro}"):]
        body = body[:body.index("\n\n")]
        for lpr, vpl in re.findall(r"X\((\d+), (\d+)\)", body):
            out.append((direction, int(lpr), int(vpl)))
    return out


def compiled_cluster_mappings():
    """(direction, threads, vectors per lane, rows per step) of the split-row lists."""
    src = _launch_h()
    out = []
    for direction, macro in (("fwd", "RN_CLUSTER_FWD_MAPPINGS"), ("bwd", "RN_CLUSTER_BWD_MAPPINGS")):
        lines = src[src.index(f"#define {macro}"):].splitlines()
        end = next(i for i, line in enumerate(lines) if not line.rstrip().endswith("\\"))
        for t, v, r in re.findall(r"X\((\d+), (\d+), (\d+)\)", "\n".join(lines[:end + 1])):
            out.append((direction, int(t), int(v), int(r)))
    return out


def mapping_shape(dtype, lpr, vpl):
    """A row that leaves the last vector slot partly empty, and a ragged row count."""
    nvec = lpr * vpl - max(1, lpr // 3) if lpr * vpl > 1 else 1
    N = nvec * epv(dtype)
    return N, max(5, min(301, 400_000 // N))


def cluster_rows(N):
    return max(3, min(997, 2_000_000 // N))


def _accepted(bwd, kind, M, N, code, opt):
    try:
        rn.norm_plan(bwd, kind == "ln", M, N, code, options=opt)
        return True
    except rn.NormError as e:
        if e.status != rn.NORM_ERR_BAD_OPTION:
            raise
        return False


def _have_lib():
    try:
        rn.lib()
        return True
    except RuntimeError:
        return False


def all_mapping_cases(pairs):
    return [(k, d, p, dr, l, v) for k in KINDS for d, p in pairs
            for dr, l, v in compiled_row_mappings()]


def mapping_cases(pairs, accepted=True):
    """Forced row-mapping cases the planner accepts (or, accepted=False, rejects)."""
    cases = all_mapping_cases(pairs)
    if not _have_lib():
        return cases if accepted else []
    out = []
    for k, d, p, dr, l, v in cases:
        N, M = mapping_shape(d, l, v)
        opt = rn.Options(path=rn.NORM_PATH_ROWS, lanes_per_row=l, vecs_per_lane=v)
        if _accepted(dr == "bwd", k, M, N, code_of(d, p), opt) == accepted:
            out.append((k, d, p, dr, l, v))
    return out


def all_cluster_cases(pairs):
    """Row lengths x cluster sizes x rows per step whose rows split evenly over C."""
    sizes = [(N, C) for N in (2048, 8192, 65536) for C in (2, 4, 8, 16, 32)
             if (N // 8) % C == 0 and (N // 8) // C <= 4096]
    return [(k, d, p, N, C, R) for k in KINDS for d, p in pairs for N, C in sizes
            for R in (1, 2) if (N // epv(d)) % C == 0]


def cluster_cases(pairs, accepted=True):
    """Forced split-row cases the planner accepts in both directions (or, accepted=False,
    rejects in at least one)."""
    cases = all_cluster_cases(pairs)
    if not _have_lib():
        return cases if accepted else []
    out = []
    for k, d, p, N, C, R in cases:
        opt = rn.Options(path=rn.NORM_PATH_CLUSTER, cluster_size=C, cluster_rows=R)
        ok = all(_accepted(bwd, k, cluster_rows(N), N, code_of(d, p), opt) for bwd in (False, True))
        if ok == accepted:
            out.append((k, d, p, N, C, R))
    return out
