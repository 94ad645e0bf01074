"""fp64 CPU oracle for RMSNorm / LayerNorm forward and backward (ctypes wrapper of oracle.c).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` import this package.  The GPU library never
imports, links or calls it, and it never imports the GPU library.

Arrays passed in are host numpy arrays of raw element bits: ``uint16`` for bfloat16,
``float16`` for IEEE binary16 and ``float32`` for fp32 (as produced by :mod:`gen`).
x and dy share a type; gamma and beta share a type, which may differ from x's.
Results are float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

F32 = 0
BF16 = 1
F16 = 2


def build(src: str = SRC_PATH, out: str = LIB_PATH, verbose: bool = False) -> str:
    """Compile the oracle (gcc, -O2, OpenMP, strict IEEE double: no -ffast-math)."""
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-ffp-contract=off",
           "-I", _HERE, src, "-o", out, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return out


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_D = ctypes.c_double
_INT = ctypes.c_int


def _ptr(a):
    return None if a is None else a.ctypes.data


def _dtype_of(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float16:
        return F16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"oracle inputs are uint16 (bf16 bits), float16 or float32, got {a.dtype}")


class Oracle:
    """Handle on one compiled oracle library (the real one, or a test mutant)."""

    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(path)
        lib.oracle_rms_fwd.argtypes = [_P, _P, _INT, _INT, _I64, _D, _P, _I64, _P, _P]
        lib.oracle_ln_fwd.argtypes = [_P, _P, _P, _INT, _INT, _I64, _D, _P, _I64, _P, _P, _P]
        lib.oracle_rms_bwd_dx.argtypes = [_P, _P, _P, _INT, _INT, _I64, _D, _P, _I64, _P]
        lib.oracle_ln_bwd_dx.argtypes = [_P, _P, _P, _INT, _INT, _I64, _D, _P, _I64, _P]
        lib.oracle_rms_bwd_dgamma.argtypes = [_P, _P, _INT, _I64, _I64, _D, _P, _P]
        lib.oracle_ln_bwd_dgamma_dbeta.argtypes = [_P, _P, _INT, _I64, _I64, _D, _P, _P, _P, _P]
        lib.oracle_residual_sum.argtypes = [_P, _P, _INT, _I64, _P, _I64, _P]
        lib.oracle_residual_sum.restype = None
        for name in ("oracle_rms_fwd", "oracle_ln_fwd", "oracle_rms_bwd_dx", "oracle_ln_bwd_dx",
                     "oracle_rms_bwd_dgamma", "oracle_ln_bwd_dgamma_dbeta"):
            getattr(lib, name).restype = None
        lib.oracle_num_threads.restype = _INT
        lib.oracle_num_threads.argtypes = []
        self.lib = lib
        self.path = path

    # ----------------------------------------------------------------- helpers
    @staticmethod
    def _prep(x, *others):
        """x and the arrays of x's type (dy)."""
        x = np.ascontiguousarray(x)
        if x.ndim != 2:
            raise ValueError("x must be 2-D [M, N]")
        dt = _dtype_of(x)
        outs = []
        for o in others:
            if o is None:
                outs.append(None)
                continue
            o = np.ascontiguousarray(o)
            if _dtype_of(o) != dt:
                raise TypeError("dy must share x's dtype")
            outs.append(o)
        return x, dt, outs

    @staticmethod
    def _params(gamma, beta=None):
        """gamma (and beta) and their shared type."""
        gamma = np.ascontiguousarray(gamma)
        gdt = _dtype_of(gamma)
        if beta is not None:
            beta = np.ascontiguousarray(beta)
            if _dtype_of(beta) != gdt:
                raise TypeError("beta must share gamma's dtype")
        return gamma, beta, gdt

    @staticmethod
    def _rows(rows, M):
        if rows is None:
            return None, M
        r = np.ascontiguousarray(rows, dtype=np.int64)
        if r.size and (r.min() < 0 or r.max() >= M):
            raise IndexError("row index out of range")
        return r, r.size

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    # ----------------------------------------------------------------- forward
    def rms_fwd(self, x, gamma, eps, rows=None):
        """-> (y [k, N] float64, rstd [k] float64) for the selected rows."""
        x, dt, _ = self._prep(x)
        gamma, _, gdt = self._params(gamma)
        M, N = x.shape
        r, k = self._rows(rows, M)
        y = np.empty((k, N), np.float64)
        rstd = np.empty(k, np.float64)
        self.lib.oracle_rms_fwd(_ptr(x), _ptr(gamma), dt, gdt, N, float(eps), _ptr(r), k,
                                _ptr(y), _ptr(rstd))
        return y, rstd

    def ln_fwd(self, x, gamma, beta, eps, rows=None):
        """-> (y, mean, rstd) float64 for the selected rows."""
        x, dt, _ = self._prep(x)
        gamma, beta, gdt = self._params(gamma, beta)
        M, N = x.shape
        r, k = self._rows(rows, M)
        y = np.empty((k, N), np.float64)
        mean = np.empty(k, np.float64)
        rstd = np.empty(k, np.float64)
        self.lib.oracle_ln_fwd(_ptr(x), _ptr(gamma), _ptr(beta), dt, gdt, N, float(eps), _ptr(r),
                               k, _ptr(y), _ptr(mean), _ptr(rstd))
        return y, mean, rstd

    # ---------------------------------------------------------------- backward
    def rms_bwd_dx(self, dy, x, gamma, eps, rows=None):
        x, dt, (dy,) = self._prep(x, dy)
        gamma, _, gdt = self._params(gamma)
        M, N = x.shape
        r, k = self._rows(rows, M)
        dx = np.empty((k, N), np.float64)
        self.lib.oracle_rms_bwd_dx(_ptr(dy), _ptr(x), _ptr(gamma), dt, gdt, N, float(eps), _ptr(r),
                                   k, _ptr(dx))
        return dx

    def ln_bwd_dx(self, dy, x, gamma, eps, rows=None):
        x, dt, (dy,) = self._prep(x, dy)
        gamma, _, gdt = self._params(gamma)
        M, N = x.shape
        r, k = self._rows(rows, M)
        dx = np.empty((k, N), np.float64)
        self.lib.oracle_ln_bwd_dx(_ptr(dy), _ptr(x), _ptr(gamma), dt, gdt, N, float(eps), _ptr(r),
                                  k, _ptr(dx))
        return dx

    def residual_sum(self, x, res, rows=None):
        """Rows of s = x + res rounded to x's type, float64 [k, N]."""
        x, dt, (res,) = self._prep(x, res)
        M, N = x.shape
        r, k = self._rows(rows, M)
        s = np.empty((k, N), np.float64)
        self.lib.oracle_residual_sum(_ptr(x), _ptr(res), dt, N, _ptr(r), k, _ptr(s))
        return s

    def rms_dgamma(self, dy, x, eps):
        """-> (dgamma [N], scale [N]) float64."""
        x, dt, (dy,) = self._prep(x, dy)
        M, N = x.shape
        dg = np.empty(N, np.float64)
        sc = np.empty(N, np.float64)
        self.lib.oracle_rms_bwd_dgamma(_ptr(dy), _ptr(x), dt, M, N, float(eps), _ptr(dg), _ptr(sc))
        return dg, sc

    def ln_dgamma_dbeta(self, dy, x, eps):
        """-> (dgamma, dbeta, dgamma_scale, dbeta_scale), each [N] float64."""
        x, dt, (dy,) = self._prep(x, dy)
        M, N = x.shape
        dg, db, sg, sb = (np.empty(N, np.float64) for _ in range(4))
        self.lib.oracle_ln_bwd_dgamma_dbeta(_ptr(dy), _ptr(x), dt, M, N, float(eps), _ptr(dg),
                                            _ptr(db), _ptr(sg), _ptr(sb))
        return dg, db, sg, sb


def as_type_bits(values: np.ndarray, dtype: int) -> np.ndarray:
    """float64 values that are exactly representable in `dtype` -> host arrays of raw bits
    (uint16 bfloat16, float16, float32), as the oracle's inputs expect."""
    v = np.asarray(values, np.float64)
    f = v.astype(np.float32)
    if dtype == F32:
        out = f
    elif dtype == F16:
        out = v.astype(np.float16)
    else:
        out = (f.view(np.uint32) >> 16).astype(np.uint16)
    back = out.astype(np.float64) if dtype != BF16 else \
        (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ok = (back == v) | (np.isnan(back) & np.isnan(v))
    if not np.all(ok):
        raise ValueError("values are not representable in the element type")
    return out


_default = None


def get() -> Oracle:
    """The oracle built next to this file."""
    global _default
    if _default is None:
        _default = Oracle(LIB_PATH)
    return _default
