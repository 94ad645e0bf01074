"""Build librownorm.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Each kernel translation unit is compiled separately (the row kernels once per
(kind, dtype)), in parallel, then linked into one shared library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "librownorm.so")
BUILD_DIR = os.path.join(HERE, "_build")

ARCH = "gfx950"
# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU instructions.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def _units():
    units = []
    # kind (0 RMSNorm, 1 LayerNorm) x type pair (TypeCombo in csrc/launch.h)
    for k in (0, 1):
        for tc in range(5):
            for name in ("fwd_rows", "bwd_rows", "cluster", "grows"):
                units.append((os.path.join(CSRC, f"{name}.hip"),
                              os.path.join(BUILD_DIR, f"{name}_k{k}_t{tc}.o"),
                              [f"-DRN_KIND={k}", f"-DRN_TC={tc}"]))
    units.append((os.path.join(CSRC, "aux_kernels.hip"), os.path.join(BUILD_DIR, "aux.o"), []))
    units.append((os.path.join(CSRC, "split_rows.hip"), os.path.join(BUILD_DIR, "split.o"), []))
    units.append((os.path.join(CSRC, "plan.cpp"), os.path.join(BUILD_DIR, "plan.o"), ["-x", "hip"]))
    units.append((os.path.join(CSRC, "api.cpp"), os.path.join(BUILD_DIR, "api.o"), ["-x", "hip"]))
    return units


def _compile(unit, verbose):
    src, obj, extra = unit
    cmd = ["hipcc"] + COMMON + extra + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; drop that warning only.
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda u: _compile(u, verbose), _units()))
    tmp = LIB_PATH + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB_PATH)
