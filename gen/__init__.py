"""Seeded synthetic inputs shared by the oracle checks, the GPU tests and the benchmark.

This package holds no normalization arithmetic: it draws numbers (``gen.c``) and
describes the workloads (shapes, value distributions, eps) as plain data.  Both the
CPU oracle and the GPU library consume the exact bits produced here.

Workloads (the row-normalization shapes this library is measured on; the pages give no
shapes of their own, so these are synthetic stand-ins):

=====  ======  ==================  =================================  ======
name   kind    x shape / dtype     x distribution                     eps
=====  ======  ==================  =================================  ======
rms1   rms     [4096, 1024] bf16   N(0, 1)                            1e-6
ln2    ln      [65536, 4096] bf16  N(0.5, sd 2)                       1e-5
rms3   rms     [262144, 384] bf16  N(0, 1)                            1e-6
rms4   rms     [2048, 131072] bf16 N(0, 1), 1% of entries x50         1e-6
sweep  both    [floor(2^27/N), N]  N(0, 1); bf16 and fp32             1e-6
=====  ======  ==================  =================================  ======

gamma = 1 + 0.1*N(0,1), beta = 0.1*N(0,1), dy = N(0,1), all in the dtype of x.
Seeds: ``0x5EED0000 + 16*config + tensor_id`` with tensor ids x=0, gamma=1, beta=2, dy=3,
and for the residual-add entry points res=4 (the residual, N(0, 1)) and dsum=5 (the
gradient arriving at the sum, 0.5*N(0, 1)).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgen.so")

F32 = 0
BF16 = 1
F16 = 2
_DTYPES = {"f32": F32, "fp32": F32, "float32": F32, "bf16": BF16, "bfloat16": BF16,
           "f16": F16, "fp16": F16, "float16": F16}
# host array dtype of each element type: bf16 as raw uint16 bits, fp16 as numpy float16
_NP = {F32: np.float32, BF16: np.uint16, F16: np.float16}

TENSOR_IDS = {"x": 0, "gamma": 1, "beta": 2, "dy": 3, "res": 4, "dsum": 5}
SEED_BASE = 0x5EED0000


def build(verbose: bool = False) -> str:
    """Compile gen.c into libgen.so next to this file (gcc, OpenMP)."""
    src = os.path.join(_HERE, "gen.c")
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", src, "-o", _LIB_PATH, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.gen_fill.restype = ctypes.c_int
        lib.gen_fill.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64,
                                 ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_double]
        for name in ("gen_round_bf16", "gen_round_f16"):
            getattr(lib, name).restype = None
            getattr(lib, name).argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        _lib = lib
    return _lib


def dtype_code(dtype: str) -> int:
    try:
        return _DTYPES[dtype]
    except KeyError:
        raise ValueError(f"unknown dtype {dtype!r}") from None


def fill(n: int, dtype: str, seed: int, mean: float = 0.0, std: float = 1.0,
         outlier_p: float = 0.0, outlier_scale: float = 1.0) -> np.ndarray:
    """n draws of mean + std*N(0,1): float32, uint16 bfloat16 bits (bf16) or float16."""
    code = dtype_code(dtype)
    out = np.empty(n, dtype=_NP[code])
    rc = _load().gen_fill(out.ctypes.data, code, n, seed & (2**64 - 1), mean, std,
                          outlier_p, outlier_scale)
    if rc != 0:
        raise ValueError("gen_fill rejected its arguments")
    return out


def round_bf16(values) -> np.ndarray:
    """float values -> uint16 bfloat16 bits, round-to-nearest-even."""
    a = np.ascontiguousarray(values, dtype=np.float32).ravel()
    out = np.empty(a.size, dtype=np.uint16)
    _load().gen_round_bf16(a.ctypes.data, out.ctypes.data, a.size)
    return out.reshape(np.shape(values))


def round_f16(values) -> np.ndarray:
    """float values -> float16 (binary16 bits), round-to-nearest-even."""
    a = np.ascontiguousarray(values, dtype=np.float32).ravel()
    out = np.empty(a.size, dtype=np.uint16)
    _load().gen_round_f16(a.ctypes.data, out.ctypes.data, a.size)
    return out.view(np.float16).reshape(np.shape(values))


def round_to(values, dtype: str) -> np.ndarray:
    """float values as host arrays of `dtype` (the form make_inputs returns)."""
    code = dtype_code(dtype)
    if code == BF16:
        return round_bf16(values)
    if code == F16:
        return round_f16(values)
    return np.ascontiguousarray(values, dtype=np.float32)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of uint16 bfloat16 bits to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "rms" or "ln"
    dtype: str           # activations: "bf16", "f16" or "f32"
    M: int
    N: int
    eps: float
    x_mean: float = 0.0
    x_std: float = 1.0
    outlier_p: float = 0.0
    outlier_scale: float = 1.0
    config: int = 0      # seed namespace
    extra: dict = field(default_factory=dict, compare=False)
    pdtype: str | None = None  # gamma/beta type when it differs from the activations

    @property
    def param_dtype(self) -> str:
        return self.pdtype or self.dtype

    def seed(self, tensor: str) -> int:
        return SEED_BASE + 16 * self.config + TENSOR_IDS[tensor]

    def scaled(self, M: int, name: str | None = None) -> "Workload":
        """Same distributions and seeds with a different row count."""
        return Workload(name or f"{self.name}_M{M}", self.kind, self.dtype, M, self.N, self.eps,
                        self.x_mean, self.x_std, self.outlier_p, self.outlier_scale, self.config,
                        pdtype=self.pdtype)


SWEEP_N = (256, 384, 512, 768, 1024, 2048, 4096, 8192, 16384, 32768, 65536)

WORKLOADS = {
    "rms1": Workload("rms1", "rms", "bf16", 4096, 1024, 1e-6, config=1),
    "ln2": Workload("ln2", "ln", "bf16", 65536, 4096, 1e-5, x_mean=0.5, x_std=2.0, config=2),
    "rms3": Workload("rms3", "rms", "bf16", 262144, 384, 1e-6, config=3),
    "rms4": Workload("rms4", "rms", "bf16", 2048, 131072, 1e-6, outlier_p=0.01,
                     outlier_scale=50.0, config=4),
}


def sweep_workload(kind: str, dtype: str, N: int) -> Workload:
    """A sweep point: M = floor(2^27 / N) rows."""
    return Workload(f"sweep_{kind}_{dtype}_N{N}", kind, dtype, (1 << 27) // N, N, 1e-6, config=5)


def make_inputs(w: Workload, rows: int | None = None, residual: bool = False) -> dict:
    """Host arrays x [M,N], gamma [N], beta [N] (LayerNorm only), dy [M,N]; with
    ``residual`` also res [M,N] and dsum [M,N].

    ``rows`` limits x and dy to their first ``rows`` rows (the draws are counter based,
    so the first rows of a larger workload are bit-identical to the full one's).
    """
    M = w.M if rows is None else min(rows, w.M)
    n = M * w.N
    out = {
        "x": fill(n, w.dtype, w.seed("x"), w.x_mean, w.x_std, w.outlier_p, w.outlier_scale
                  ).reshape(M, w.N),
        "gamma": fill(w.N, w.param_dtype, w.seed("gamma"), 1.0, 0.1),
        "dy": fill(n, w.dtype, w.seed("dy"), 0.0, 1.0).reshape(M, w.N),
    }
    if w.kind == "ln":
        out["beta"] = fill(w.N, w.param_dtype, w.seed("beta"), 0.0, 0.1)
    if residual:
        out["res"] = fill(n, w.dtype, w.seed("res"), 0.0, 1.0).reshape(M, w.N)
        out["dsum"] = fill(n, w.dtype, w.seed("dsum"), 0.0, 0.5).reshape(M, w.N)
    return out
