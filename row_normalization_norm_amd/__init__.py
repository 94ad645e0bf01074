"""Python binding of librownorm.so: fused RMSNorm / LayerNorm forward and backward on
MI355X (gfx950).

The functions carry the C entry points' names (include/rownorm.h) and only marshal
arguments: they read shapes, dtypes and device pointers off torch tensors, pass the
current HIP stream, and raise :class:`NormError` on a non-OK status.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.  torch is used for
device memory and streams only.

Raw ctypes access to the library is available through :func:`lib`.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librownorm.so")

# norm_dtype_t
NORM_DTYPE_F32 = 0
NORM_DTYPE_BF16 = 1
NORM_DTYPE_F16 = 2


def dtype_mixed(act: int, param: int) -> int:
    """NORM_DTYPE_MIXED: activations of type `act` with gamma/beta of type `param`."""
    return act | ((param + 1) << 8)
# norm_status_t
NORM_OK = 0
NORM_ERR_NULL_PTR = 1
NORM_ERR_BAD_SHAPE = 2
NORM_ERR_BAD_DTYPE = 3
NORM_ERR_BAD_EPS = 4
NORM_ERR_WORKSPACE_TOO_SMALL = 5
NORM_ERR_HIP = 6
NORM_ERR_MISALIGNED = 7
NORM_ERR_BAD_OPTION = 8
NORM_ERR_SCRATCH_TOO_SMALL = 9
# norm_dgamma_mode_t
NORM_DGAMMA_TWO_STAGE = 0
NORM_DGAMMA_ATOMIC_ROW = 1
NORM_DGAMMA_ATOMIC_WG = 2
# norm_path_t
NORM_PATH_AUTO = 0
NORM_PATH_ROWS = 1
NORM_PATH_SPLIT = 2
NORM_PATH_GENERIC = 3
NORM_PATH_CLUSTER = 4


class NormError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class Options(ctypes.Structure):
    """norm_options_t."""
    _fields_ = [("path", ctypes.c_int), ("lanes_per_row", ctypes.c_int),
                ("vecs_per_lane", ctypes.c_int), ("dgamma_mode", ctypes.c_int),
                ("grid", ctypes.c_int), ("cluster_size", ctypes.c_int),
                ("cluster_rows", ctypes.c_int), ("ev_start", ctypes.c_void_p),
                ("ev_stop", ctypes.c_void_p), ("cluster_wait", ctypes.c_int),
                ("pipeline", ctypes.c_int)]


class PlanInfo(ctypes.Structure):
    """norm_plan_info_t."""
    _fields_ = [("path", ctypes.c_int), ("lanes_per_row", ctypes.c_int),
                ("vecs_per_lane", ctypes.c_int), ("block", ctypes.c_int),
                ("grid", ctypes.c_int), ("partial_rows", ctypes.c_int),
                ("cluster_size", ctypes.c_int), ("cluster_rows", ctypes.c_int),
                ("workspace_bytes", ctypes.c_size_t), ("pipelined", ctypes.c_int)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t
_OPT = ctypes.POINTER(Options)

SIGNATURES = {
    "norm_fwd_workspace_size": (_SZ, [_I64, _I64, _INT, _INT]),
    "norm_rms_fwd": (_INT, [_P, _P, _P, _P, _I64, _I64, _F, _INT, _P, _SZ, _P]),
    "norm_ln_fwd": (_INT, [_P, _P, _P, _P, _P, _P, _I64, _I64, _F, _INT, _P, _SZ, _P]),
    "norm_bwd_workspace_size": (_SZ, [_I64, _I64, _INT, _INT]),
    "norm_rms_bwd": (_INT, [_P, _P, _P, _P, _P, _P, _I64, _I64, _INT, _P, _SZ, _P]),
    "norm_ln_bwd": (_INT, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _INT, _P, _SZ, _P]),
    "norm_status_string": (ctypes.c_char_p, [_INT]),
    "norm_plan": (_INT, [_INT, _INT, _I64, _I64, _INT, _INT, _OPT, ctypes.POINTER(PlanInfo)]),
    "norm_cluster_resident": (_INT, [_INT, _INT, _I64, _I64, _INT, _OPT]),
    "norm_fwd_workspace_size_ex": (_SZ, [_I64, _I64, _INT, _INT, _OPT]),
    "norm_bwd_workspace_size_ex": (_SZ, [_I64, _I64, _INT, _INT, _OPT]),
    "norm_rms_fwd_ex": (_INT, [_P, _P, _P, _P, _I64, _I64, _F, _INT, _P, _SZ, _P, _OPT]),
    "norm_ln_fwd_ex": (_INT, [_P, _P, _P, _P, _P, _P, _I64, _I64, _F, _INT, _P, _SZ, _P, _OPT]),
    "norm_rms_bwd_ex": (_INT, [_P, _P, _P, _P, _P, _P, _I64, _I64, _INT, _P, _SZ, _P, _OPT]),
    "norm_ln_bwd_ex": (_INT, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _INT, _P, _SZ, _P,
                              _OPT]),
    "norm_rms_fwd_add": (_INT, [_P, _P, _P, _P, _P, _P, _I64, _I64, _F, _INT, _P, _SZ, _P, _OPT]),
    "norm_ln_fwd_add": (_INT, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _F, _INT, _P, _SZ, _P,
                               _OPT]),
    "norm_rms_bwd_add": (_INT, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _INT, _P, _SZ, _P, _OPT]),
    "norm_ln_bwd_add": (_INT, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _INT, _P, _SZ, _P,
                               _OPT]),
    "norm_stream_reference": (_INT, [_INT, _P, _P, _P, _I64, _P]),
    "norm_ln_bwd_noalloc": (_INT, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _INT, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded librownorm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                f"g.build()'` (hipcc, gfx950)")
        # torch ships its own HIP runtime under the soname libamdhip64.so.7 but links it
        # by another name, so the dynamic loader would load a second runtime if this
        # library (which names the soname) came first: torch's device pointers and
        # streams would then be foreign to it.  Importing torch first makes this library
        # bind to torch's runtime.
        torch = _torch()
        global _F32, _RAW_STREAM
        _F32 = torch.float32
        _RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None) or \
            (lambda d: torch.cuda.current_stream(d).cuda_stream)
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().norm_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != NORM_OK:
        raise NormError(status, where)


# ------------------------------------------------------------------- marshalling
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return NORM_DTYPE_BF16
    if t.dtype == torch.float32:
        return NORM_DTYPE_F32
    if t.dtype == torch.float16:
        return NORM_DTYPE_F16
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16, float16 or float32)")


_TYPES = {}
_F32 = None


def _types(xd, gd):
    """The library's dtype code for activations of dtype xd and parameters of dtype gd."""
    key = (xd, gd)
    code = _TYPES.get(key)
    if code is not None:
        return code
    torch = _torch()
    codes = {torch.bfloat16: NORM_DTYPE_BF16, torch.float32: NORM_DTYPE_F32,
             torch.float16: NORM_DTYPE_F16}
    for d in (xd, gd):
        if d not in codes:
            raise TypeError(f"unsupported dtype {d} (bfloat16, float16 or float32)")
    act, par = codes[xd], codes[gd]
    if par == act:
        code = act
    elif par == NORM_DTYPE_F32 and act in (NORM_DTYPE_BF16, NORM_DTYPE_F16):
        code = dtype_mixed(act, par)
    else:
        raise TypeError(f"gamma/beta of {gd} with activations of {xd}: use "
                        f"the activations' type or float32")
    _TYPES[key] = code
    return code


def _need(t, name, numel, dtype, dev):
    """The device address of t (None when t is None) after checking that it is a
    contiguous tensor of numel elements of dtype on GPU dev (an index).  One combined
    test on the common path: these checks run on every call."""
    if t is None:
        return None
    if t.dtype is not dtype or t.numel() != numel or t.get_device() != dev or \
            not t.is_contiguous():
        if t.get_device() != dev:
            raise ValueError(f"{name} must be on cuda:{dev}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return t.data_ptr()


def _shape(x):
    """(M, N, device index) of the activations x."""
    shape = x.shape
    if len(shape) != 2:
        raise ValueError("x must be 2-D [M, N] (reshape leading dimensions into M)")
    dev = x.get_device()
    if dev < 0:
        raise ValueError("x must be a GPU tensor")
    return shape[0], shape[1], dev


_RAW_STREAM = None


def _stream(dev, stream):
    """The raw HIP stream: the given one, else torch's current stream on GPU dev."""
    if stream is None:
        return _RAW_STREAM(dev)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _opt(options):
    return None if options is None else ctypes.byref(options)


def _keep_for_stream(ws, dev, stream):
    """A workspace the binding allocated lives in torch's caching allocator, which
    tracks it on the current stream.  When the call runs on another stream, mark the
    block as used there too, so that it is not handed to a later allocation before
    the kernels reading it have finished."""
    if ws is None or stream is None:
        return
    torch = _torch()
    ptr = _stream(dev, stream)
    if ptr != _stream(dev, None):
        ws.record_stream(torch.cuda.ExternalStream(ptr, device=dev))


# ------------------------------------------------------------------- entry points
def norm_fwd_workspace_size(M: int, N: int, is_layernorm: bool, dtype: int, options=None) -> int:
    if options is None:
        return int(lib().norm_fwd_workspace_size(M, N, int(bool(is_layernorm)), dtype))
    return int(lib().norm_fwd_workspace_size_ex(M, N, int(bool(is_layernorm)), dtype,
                                                _opt(options)))


_FWD_WS = {}


def _fwd_workspace(M, N, ln, dtype, dev, workspace, options, stream, aligned):
    """(address, bytes, tensor) of the caller's workspace (the library checks its size),
    or of a new one of the size the call needs with its pointers' alignment (None, 0,
    None when it needs none)."""
    if workspace is not None:
        return workspace.data_ptr(), workspace.numel() * workspace.element_size(), workspace
    key = (M, N, ln, dtype, aligned)
    need = _FWD_WS.get(key) if options is None else None
    if need is None:
        need = int(norm_plan(False, ln, M, N, dtype, aligned, options).workspace_bytes)
        if options is None:
            _FWD_WS[key] = need
    if need == 0:
        return None, 0, None
    torch = _torch()
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _keep_for_stream(ws, dev, stream)
    return ws.data_ptr(), need, ws


def _fail(status, where):
    raise NormError(status, where)


def norm_rms_fwd(x, gamma, y, rstd=None, eps: float = 1e-6, workspace=None, stream=None,
                 options=None):
    """y = x * rstd * gamma with rstd = 1/sqrt(mean(x^2) + eps) per row; rstd saved if given."""
    L = _lib or lib()
    M, N, dev = _shape(x)
    xd = x.dtype
    gd = xd if gamma is None else gamma.dtype
    px = _need(x, "x", M * N, xd, dev)
    py = _need(y, "y", M * N, xd, dev)
    pg = _need(gamma, "gamma", N, gd, dev)
    pr = _need(rstd, "rstd", M, _F32, dev)
    dt = _types(xd, gd)
    pw, nw, keep = _fwd_workspace(M, N, False, dt, dev, workspace, options, stream,
                                  ((px or 0) | (pg or 0) | (py or 0)) & 15 == 0)
    st = _stream(dev, stream)
    if options is None:
        status = L.norm_rms_fwd(px, pg, py, pr, M, N, float(eps), dt, pw, nw, st)
        if status:
            _fail(status, "norm_rms_fwd")
    else:
        status = L.norm_rms_fwd_ex(px, pg, py, pr, M, N, float(eps), dt, pw, nw, st,
                                   _opt(options))
        if status:
            _fail(status, "norm_rms_fwd_ex")
    return y


def norm_ln_fwd(x, gamma, beta, y, mean=None, rstd=None, eps: float = 1e-5, workspace=None,
                stream=None, options=None):
    """y = (x - mean) * rstd * gamma + beta per row; mean and rstd saved if given."""
    L = _lib or lib()
    M, N, dev = _shape(x)
    xd = x.dtype
    gd = xd if gamma is None else gamma.dtype
    px = _need(x, "x", M * N, xd, dev)
    py = _need(y, "y", M * N, xd, dev)
    pg = _need(gamma, "gamma", N, gd, dev)
    pb = _need(beta, "beta", N, gd, dev)
    pm = _need(mean, "mean", M, _F32, dev)
    pr = _need(rstd, "rstd", M, _F32, dev)
    dt = _types(xd, gd)
    pw, nw, keep = _fwd_workspace(M, N, True, dt, dev, workspace, options, stream,
                                  ((px or 0) | (pg or 0) | (pb or 0) | (py or 0)) & 15 == 0)
    st = _stream(dev, stream)
    if options is None:
        status = L.norm_ln_fwd(px, pg, pb, py, pm, pr, M, N, float(eps), dt, pw, nw, st)
        if status:
            _fail(status, "norm_ln_fwd")
    else:
        status = L.norm_ln_fwd_ex(px, pg, pb, py, pm, pr, M, N, float(eps), dt, pw, nw, st,
                                  _opt(options))
        if status:
            _fail(status, "norm_ln_fwd_ex")
    return y


def norm_bwd_workspace_size(M: int, N: int, is_layernorm: bool, dtype: int, options=None) -> int:
    if options is None:
        return int(lib().norm_bwd_workspace_size(M, N, int(bool(is_layernorm)), dtype))
    return int(lib().norm_bwd_workspace_size_ex(M, N, int(bool(is_layernorm)), dtype,
                                                _opt(options)))


_BWD_WS = {}


def _workspace(M, N, ln, dtype, dev, workspace, options, stream):
    """(address, bytes, tensor) of the caller's workspace (the library checks its size),
    or of a new one of the size the call needs."""
    if workspace is None:
        key = (M, N, ln, dtype)
        need = _BWD_WS.get(key) if options is None else None
        if need is None:
            need = norm_bwd_workspace_size(M, N, ln, dtype, options)
            if options is None:
                _BWD_WS[key] = need
        torch = _torch()
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        _keep_for_stream(workspace, dev, stream)
    return workspace.data_ptr(), workspace.numel() * workspace.element_size(), workspace


def norm_rms_bwd(dy, x, gamma, rstd, dx, dgamma, workspace=None, stream=None, options=None):
    """dx and dgamma (overwritten) of RMSNorm from the forward's saved rstd."""
    L = _lib or lib()
    M, N, dev = _shape(x)
    xd = x.dtype
    gd = xd if gamma is None else gamma.dtype
    pdy = _need(dy, "dy", M * N, xd, dev)
    px = _need(x, "x", M * N, xd, dev)
    pdx = _need(dx, "dx", M * N, xd, dev)
    pg = _need(gamma, "gamma", N, gd, dev)
    pr = _need(rstd, "rstd", M, _F32, dev)
    pdg = _need(dgamma, "dgamma", N, _F32, dev)
    dt = _types(xd, gd)
    pw, nw, keep = _workspace(M, N, False, dt, dev, workspace, options, stream)
    st = _stream(dev, stream)
    if options is None:
        status = L.norm_rms_bwd(pdy, px, pg, pr, pdx, pdg, M, N, dt, pw, nw, st)
        if status:
            _fail(status, "norm_rms_bwd")
    else:
        status = L.norm_rms_bwd_ex(pdy, px, pg, pr, pdx, pdg, M, N, dt, pw, nw, st,
                                   _opt(options))
        if status:
            _fail(status, "norm_rms_bwd_ex")
    return dx, dgamma


def norm_ln_bwd(dy, x, gamma, mean, rstd, dx, dgamma, dbeta, workspace=None, stream=None,
                options=None):
    """dx, dgamma and dbeta (overwritten) of LayerNorm from the saved mean and rstd."""
    L = _lib or lib()
    M, N, dev = _shape(x)
    xd = x.dtype
    gd = xd if gamma is None else gamma.dtype
    pdy = _need(dy, "dy", M * N, xd, dev)
    px = _need(x, "x", M * N, xd, dev)
    pdx = _need(dx, "dx", M * N, xd, dev)
    pg = _need(gamma, "gamma", N, gd, dev)
    pm = _need(mean, "mean", M, _F32, dev)
    pr = _need(rstd, "rstd", M, _F32, dev)
    pdg = _need(dgamma, "dgamma", N, _F32, dev)
    pdb = _need(dbeta, "dbeta", N, _F32, dev)
    dt = _types(xd, gd)
    pw, nw, keep = _workspace(M, N, True, dt, dev, workspace, options, stream)
    st = _stream(dev, stream)
    if options is None:
        status = L.norm_ln_bwd(pdy, px, pg, pm, pr, pdx, pdg, pdb, M, N, dt, pw, nw, st)
        if status:
            _fail(status, "norm_ln_bwd")
    else:
        status = L.norm_ln_bwd_ex(pdy, px, pg, pm, pr, pdx, pdg, pdb, M, N, dt, pw, nw, st,
                                  _opt(options))
        if status:
            _fail(status, "norm_ln_bwd_ex")
    return dx, dgamma, dbeta


def norm_ln_bwd_noalloc(dy, x, gamma, mean, rstd, dx, dgamma, dbeta, stream=None):
    """norm_ln_bwd on the library's static scratch: no workspace, no allocation (the
    binding allocates nothing either).  Calls that overlap on one device race."""
    L = _lib or lib()
    M, N, dev = _shape(x)
    xd = x.dtype
    gd = xd if gamma is None else gamma.dtype
    pdy = _need(dy, "dy", M * N, xd, dev)
    px = _need(x, "x", M * N, xd, dev)
    pdx = _need(dx, "dx", M * N, xd, dev)
    pg = _need(gamma, "gamma", N, gd, dev)
    pm = _need(mean, "mean", M, _F32, dev)
    pr = _need(rstd, "rstd", M, _F32, dev)
    pdg = _need(dgamma, "dgamma", N, _F32, dev)
    pdb = _need(dbeta, "dbeta", N, _F32, dev)
    status = L.norm_ln_bwd_noalloc(pdy, px, pg, pm, pr, pdx, pdg, pdb, M, N, _types(xd, gd),
                                   _stream(dev, stream))
    if status:
        _fail(status, "norm_ln_bwd_noalloc")
    return dx, dgamma, dbeta


def norm_plan(is_backward: bool, is_layernorm: bool, M: int, N: int, dtype: int,
              aligned16: bool = True, options=None) -> PlanInfo:
    info = PlanInfo()
    _check(lib().norm_plan(int(bool(is_backward)), int(bool(is_layernorm)), M, N, dtype,
                           int(bool(aligned16)), _opt(options), ctypes.byref(info)), "norm_plan")
    return info


def norm_cluster_resident(is_backward: bool, is_layernorm: bool, M: int, N: int, dtype: int,
                          options=None) -> int:
    """1 if the call would run on the CLUSTER path on the current device, else 0."""
    return int(lib().norm_cluster_resident(int(bool(is_backward)), int(bool(is_layernorm)), M, N,
                                           dtype, _opt(options)))


# ------------------------------------------------------------- residual add fused
def norm_rms_fwd_add(x, residual, gamma, y, sum_out, rstd=None, eps: float = 1e-6,
                     workspace=None, stream=None, options=None):
    """sum_out = x + residual (rounded to x's type); y = RMSNorm(sum_out)."""
    L = _lib or lib()
    M, N, dev = _shape(x)
    xd = x.dtype
    gd = xd if gamma is None else gamma.dtype
    px = _need(x, "x", M * N, xd, dev)
    pres = _need(residual, "residual", M * N, xd, dev)
    py = _need(y, "y", M * N, xd, dev)
    ps = _need(sum_out, "sum_out", M * N, xd, dev)
    pg = _need(gamma, "gamma", N, gd, dev)
    pr = _need(rstd, "rstd", M, _F32, dev)
    dt = _types(xd, gd)
    pw, nw, keep = _fwd_workspace(
        M, N, False, dt, dev, workspace, options, stream,
        ((px or 0) | (pres or 0) | (pg or 0) | (py or 0) | (ps or 0)) & 15 == 0)
    status = L.norm_rms_fwd_add(px, pres, pg, py, ps, pr, M, N, float(eps), dt, pw, nw,
                                _stream(dev, stream), _opt(options))
    if status:
        _fail(status, "norm_rms_fwd_add")
    return y, sum_out


def norm_ln_fwd_add(x, residual, gamma, beta, y, sum_out, mean=None, rstd=None,
                    eps: float = 1e-5, workspace=None, stream=None, options=None):
    """sum_out = x + residual (rounded to x's type); y = LayerNorm(sum_out)."""
    L = _lib or lib()
    M, N, dev = _shape(x)
    xd = x.dtype
    gd = xd if gamma is None else gamma.dtype
    px = _need(x, "x", M * N, xd, dev)
    pres = _need(residual, "residual", M * N, xd, dev)
    py = _need(y, "y", M * N, xd, dev)
    ps = _need(sum_out, "sum_out", M * N, xd, dev)
    pg = _need(gamma, "gamma", N, gd, dev)
    pb = _need(beta, "beta", N, gd, dev)
    pm = _need(mean, "mean", M, _F32, dev)
    pr = _need(rstd, "rstd", M, _F32, dev)
    dt = _types(xd, gd)
    pw, nw, keep = _fwd_workspace(
        M, N, True, dt, dev, workspace, options, stream,
        ((px or 0) | (pres or 0) | (pg or 0) | (pb or 0) | (py or 0) | (ps or 0)) & 15 == 0)
    status = L.norm_ln_fwd_add(px, pres, pg, pb, py, ps, pm, pr, M, N, float(eps), dt, pw, nw,
                               _stream(dev, stream), _opt(options))
    if status:
        _fail(status, "norm_ln_fwd_add")
    return y, sum_out


def norm_rms_bwd_add(dy, sum_in, gamma, rstd, dsum, dx, dgamma, workspace=None, stream=None,
                     options=None):
    """dx = RMSNorm backward at sum_in (+ dsum, the gradient arriving at the sum, if given);
    dgamma overwritten."""
    L = _lib or lib()
    M, N, dev = _shape(sum_in)
    xd = sum_in.dtype
    gd = xd if gamma is None else gamma.dtype
    pdy = _need(dy, "dy", M * N, xd, dev)
    ps = _need(sum_in, "sum_in", M * N, xd, dev)
    pds = _need(dsum, "dsum", M * N, xd, dev)
    pdx = _need(dx, "dx", M * N, xd, dev)
    pg = _need(gamma, "gamma", N, gd, dev)
    pr = _need(rstd, "rstd", M, _F32, dev)
    pdg = _need(dgamma, "dgamma", N, _F32, dev)
    dt = _types(xd, gd)
    pw, nw, keep = _workspace(M, N, False, dt, dev, workspace, options, stream)
    status = L.norm_rms_bwd_add(pdy, ps, pg, pr, pds, pdx, pdg, M, N, dt, pw, nw,
                                _stream(dev, stream), _opt(options))
    if status:
        _fail(status, "norm_rms_bwd_add")
    return dx, dgamma


def norm_ln_bwd_add(dy, sum_in, gamma, mean, rstd, dsum, dx, dgamma, dbeta, workspace=None,
                    stream=None, options=None):
    """dx = LayerNorm backward at sum_in (+ dsum if given); dgamma, dbeta overwritten."""
    L = _lib or lib()
    M, N, dev = _shape(sum_in)
    xd = sum_in.dtype
    gd = xd if gamma is None else gamma.dtype
    pdy = _need(dy, "dy", M * N, xd, dev)
    ps = _need(sum_in, "sum_in", M * N, xd, dev)
    pds = _need(dsum, "dsum", M * N, xd, dev)
    pdx = _need(dx, "dx", M * N, xd, dev)
    pg = _need(gamma, "gamma", N, gd, dev)
    pm = _need(mean, "mean", M, _F32, dev)
    pr = _need(rstd, "rstd", M, _F32, dev)
    pdg = _need(dgamma, "dgamma", N, _F32, dev)
    pdb = _need(dbeta, "dbeta", N, _F32, dev)
    dt = _types(xd, gd)
    pw, nw, keep = _workspace(M, N, True, dt, dev, workspace, options, stream)
    status = L.norm_ln_bwd_add(pdy, ps, pg, pm, pr, pds, pdx, pdg, pdb, M, N, dt, pw, nw,
                               _stream(dev, stream), _opt(options))
    if status:
        _fail(status, "norm_ln_bwd_add")
    return dx, dgamma, dbeta


# ------------------------------------------------------------------ measurement aid
def norm_stream_reference(kind: int, a, b, dst, stream=None):
    """Streaming reference kernel over dst's bytes (16-byte vectors): kind 0 copies a
    into dst, kind 1 writes a + b (32-bit lanes).  Not part of the normalization path:
    the achievable-bandwidth reference for the benchmark."""
    nbytes = dst.numel() * dst.element_size()
    if nbytes % 16:
        raise ValueError("dst must hold a whole number of 16-byte vectors")
    for t, n in ((a, "a"), (b, "b")):
        if t is None:
            continue
        if t.numel() * t.element_size() < nbytes or not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous and at least as large as dst")
    _check(lib().norm_stream_reference(int(kind), a.data_ptr(),
                                       b.data_ptr() if b is not None else None, dst.data_ptr(),
                                       nbytes // 16, _stream(dst.get_device(), stream)),
           "norm_stream_reference")
