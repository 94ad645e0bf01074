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
        _torch()
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


def _pdtype(x, gamma):
    return x.dtype if gamma is None else gamma.dtype


_TYPES = {}


def _types(x, gamma):
    """The library's dtype code for activations like x and parameters like gamma."""
    key = (x.dtype, None if gamma is None else gamma.dtype)
    code = _TYPES.get(key)
    if code is not None:
        return code
    act = _dtype_code(x)
    par = act if gamma is None else _dtype_code(gamma)
    if par == act:
        code = act
    elif par == NORM_DTYPE_F32 and act in (NORM_DTYPE_BF16, NORM_DTYPE_F16):
        code = dtype_mixed(act, par)
    else:
        raise TypeError(f"gamma/beta of {gamma.dtype} with activations of {x.dtype}: use "
                        f"the activations' type or float32")
    _TYPES[key] = code
    return code


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, name, numel, dtype, dev):
    """t (unless None) is a contiguous tensor of numel elements of dtype on GPU dev (an
    index).  One combined test on the common path: these checks run on every call."""
    if t is None:
        return
    if t.dtype is not dtype or t.numel() != numel or t.get_device() != dev or \
            not t.is_contiguous():
        if t.get_device() != dev:
            raise ValueError(f"{name} must be on cuda:{dev}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")


def _shape(x):
    """(M, N, device index) of the activations x."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, N] (reshape leading dimensions into M)")
    dev = x.get_device()
    if dev < 0 or not x.is_cuda:
        raise ValueError("x must be a GPU tensor")
    M, N = x.shape
    return M, N, dev


_RAW_STREAM = None


def _stream(dev, stream):
    """The raw HIP stream: the given one, else torch's current stream on GPU dev."""
    global _RAW_STREAM
    if stream is None:
        if _RAW_STREAM is None:
            torch = _torch()
            _RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None) or \
                (lambda d: torch.cuda.current_stream(d).cuda_stream)
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


def _aligned16(*tensors):
    bits = 0
    for t in tensors:
        if t is not None:
            bits |= t.data_ptr()
    return bits & 15 == 0


def _fwd_workspace(M, N, ln, dtype, dev, workspace, options, stream, aligned):
    """The caller's workspace (the library checks its size), or a new one of the size the
    call needs with its pointers' alignment (None when it needs none)."""
    if workspace is not None:
        return workspace, workspace.numel() * workspace.element_size()
    key = (M, N, ln, dtype, aligned)
    need = _FWD_WS.get(key) if options is None else None
    if need is None:
        need = int(norm_plan(False, ln, M, N, dtype, aligned, options).workspace_bytes)
        if options is None:
            _FWD_WS[key] = need
    if need == 0:
        return None, 0
    ws = _torch().empty(need, dtype=_torch().uint8, device=dev)
    _keep_for_stream(ws, dev, stream)
    return ws, need


def norm_rms_fwd(x, gamma, y, rstd=None, eps: float = 1e-6, workspace=None, stream=None,
                 options=None):
    """y = x * rstd * gamma with rstd = 1/sqrt(mean(x^2) + eps) per row; rstd saved if given."""
    torch = _torch()
    M, N, dev = _shape(x)
    _need(x, "x", M * N, x.dtype, dev)
    _need(y, "y", M * N, x.dtype, dev)
    _need(gamma, "gamma", N, _pdtype(x, gamma), dev)
    _need(rstd, "rstd", M, torch.float32, dev)
    dt = _types(x, gamma)
    ws, ws_bytes = _fwd_workspace(M, N, False, dt, dev, workspace, options, stream,
                                  _aligned16(x, gamma, y))
    args = (_ptr(x), _ptr(gamma), _ptr(y), _ptr(rstd), M, N, float(eps), dt, _ptr(ws), ws_bytes,
            _stream(dev, stream))
    if options is None:
        _check(lib().norm_rms_fwd(*args), "norm_rms_fwd")
    else:
        _check(lib().norm_rms_fwd_ex(*args, _opt(options)), "norm_rms_fwd_ex")
    return y


def norm_ln_fwd(x, gamma, beta, y, mean=None, rstd=None, eps: float = 1e-5, workspace=None,
                stream=None, options=None):
    """y = (x - mean) * rstd * gamma + beta per row; mean and rstd saved if given."""
    torch = _torch()
    M, N, dev = _shape(x)
    _need(x, "x", M * N, x.dtype, dev)
    _need(y, "y", M * N, x.dtype, dev)
    _need(gamma, "gamma", N, _pdtype(x, gamma), dev)
    _need(beta, "beta", N, _pdtype(x, gamma), dev)
    _need(mean, "mean", M, torch.float32, dev)
    _need(rstd, "rstd", M, torch.float32, dev)
    dt = _types(x, gamma)
    ws, ws_bytes = _fwd_workspace(M, N, True, dt, dev, workspace, options, stream,
                                  _aligned16(x, gamma, beta, y))
    args = (_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), _ptr(mean), _ptr(rstd), M, N, float(eps),
            dt, _ptr(ws), ws_bytes, _stream(dev, stream))
    if options is None:
        _check(lib().norm_ln_fwd(*args), "norm_ln_fwd")
    else:
        _check(lib().norm_ln_fwd_ex(*args, _opt(options)), "norm_ln_fwd_ex")
    return y


def norm_bwd_workspace_size(M: int, N: int, is_layernorm: bool, dtype: int, options=None) -> int:
    if options is None:
        return int(lib().norm_bwd_workspace_size(M, N, int(bool(is_layernorm)), dtype))
    return int(lib().norm_bwd_workspace_size_ex(M, N, int(bool(is_layernorm)), dtype,
                                                _opt(options)))


def _workspace(M, N, ln, dtype, dev, workspace, options, stream):
    """The caller's workspace (the library checks its size), or a new one of the size the
    call needs."""
    if workspace is None:
        torch = _torch()
        need = norm_bwd_workspace_size(M, N, ln, dtype, options)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        _keep_for_stream(workspace, dev, stream)
    return workspace, workspace.numel() * workspace.element_size()


def norm_rms_bwd(dy, x, gamma, rstd, dx, dgamma, workspace=None, stream=None, options=None):
    """dx and dgamma (overwritten) of RMSNorm from the forward's saved rstd."""
    torch = _torch()
    M, N, dev = _shape(x)
    for t, n, k in ((dy, "dy", M * N), (x, "x", M * N), (dx, "dx", M * N)):
        _need(t, n, k, x.dtype, dev)
    _need(gamma, "gamma", N, _pdtype(x, gamma), dev)
    _need(rstd, "rstd", M, torch.float32, dev)
    _need(dgamma, "dgamma", N, torch.float32, dev)
    dt = _types(x, gamma)
    ws, ws_bytes = _workspace(M, N, False, dt, dev, workspace, options, stream)
    args = (_ptr(dy), _ptr(x), _ptr(gamma), _ptr(rstd), _ptr(dx), _ptr(dgamma), M, N, dt,
            _ptr(ws), ws_bytes, _stream(dev, stream))
    if options is None:
        _check(lib().norm_rms_bwd(*args), "norm_rms_bwd")
    else:
        _check(lib().norm_rms_bwd_ex(*args, _opt(options)), "norm_rms_bwd_ex")
    return dx, dgamma


def norm_ln_bwd(dy, x, gamma, mean, rstd, dx, dgamma, dbeta, workspace=None, stream=None,
                options=None):
    """dx, dgamma and dbeta (overwritten) of LayerNorm from the saved mean and rstd."""
    torch = _torch()
    M, N, dev = _shape(x)
    for t, n, k in ((dy, "dy", M * N), (x, "x", M * N), (dx, "dx", M * N)):
        _need(t, n, k, x.dtype, dev)
    _need(gamma, "gamma", N, _pdtype(x, gamma), dev)
    for t, n, k in ((mean, "mean", M), (rstd, "rstd", M), (dgamma, "dgamma", N),
                    (dbeta, "dbeta", N)):
        _need(t, n, k, torch.float32, dev)
    dt = _types(x, gamma)
    ws, ws_bytes = _workspace(M, N, True, dt, dev, workspace, options, stream)
    args = (_ptr(dy), _ptr(x), _ptr(gamma), _ptr(mean), _ptr(rstd), _ptr(dx), _ptr(dgamma),
            _ptr(dbeta), M, N, dt, _ptr(ws), ws_bytes, _stream(dev, stream))
    if options is None:
        _check(lib().norm_ln_bwd(*args), "norm_ln_bwd")
    else:
        _check(lib().norm_ln_bwd_ex(*args, _opt(options)), "norm_ln_bwd_ex")
    return dx, dgamma, dbeta


def norm_ln_bwd_noalloc(dy, x, gamma, mean, rstd, dx, dgamma, dbeta, stream=None):
    """norm_ln_bwd on the library's static scratch: no workspace, no allocation (the
    binding allocates nothing either).  Calls that overlap on one device race."""
    torch = _torch()
    M, N, dev = _shape(x)
    for t, n, k in ((dy, "dy", M * N), (x, "x", M * N), (dx, "dx", M * N)):
        _need(t, n, k, x.dtype, dev)
    _need(gamma, "gamma", N, _pdtype(x, gamma), dev)
    for t, n, k in ((mean, "mean", M), (rstd, "rstd", M), (dgamma, "dgamma", N),
                    (dbeta, "dbeta", N)):
        _need(t, n, k, torch.float32, dev)
    _check(lib().norm_ln_bwd_noalloc(_ptr(dy), _ptr(x), _ptr(gamma), _ptr(mean), _ptr(rstd),
                                     _ptr(dx), _ptr(dgamma), _ptr(dbeta), M, N,
                                     _types(x, gamma), _stream(dev, stream)),
           "norm_ln_bwd_noalloc")
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
    torch = _torch()
    M, N, dev = _shape(x)
    for t, n in ((x, "x"), (residual, "residual"), (y, "y"), (sum_out, "sum_out")):
        _need(t, n, M * N, x.dtype, dev)
    _need(gamma, "gamma", N, _pdtype(x, gamma), dev)
    _need(rstd, "rstd", M, torch.float32, dev)
    dt = _types(x, gamma)
    ws, ws_bytes = _fwd_workspace(M, N, False, dt, dev, workspace, options, stream,
                                  _aligned16(x, residual, gamma, y, sum_out))
    _check(lib().norm_rms_fwd_add(_ptr(x), _ptr(residual), _ptr(gamma), _ptr(y), _ptr(sum_out),
                                  _ptr(rstd), M, N, float(eps), dt, _ptr(ws), ws_bytes,
                                  _stream(dev, stream), _opt(options)), "norm_rms_fwd_add")
    return y, sum_out


def norm_ln_fwd_add(x, residual, gamma, beta, y, sum_out, mean=None, rstd=None,
                    eps: float = 1e-5, workspace=None, stream=None, options=None):
    """sum_out = x + residual (rounded to x's type); y = LayerNorm(sum_out)."""
    torch = _torch()
    M, N, dev = _shape(x)
    for t, n in ((x, "x"), (residual, "residual"), (y, "y"), (sum_out, "sum_out")):
        _need(t, n, M * N, x.dtype, dev)
    _need(gamma, "gamma", N, _pdtype(x, gamma), dev)
    _need(beta, "beta", N, _pdtype(x, gamma), dev)
    _need(mean, "mean", M, torch.float32, dev)
    _need(rstd, "rstd", M, torch.float32, dev)
    dt = _types(x, gamma)
    ws, ws_bytes = _fwd_workspace(M, N, True, dt, dev, workspace, options, stream,
                                  _aligned16(x, residual, gamma, beta, y, sum_out))
    _check(lib().norm_ln_fwd_add(_ptr(x), _ptr(residual), _ptr(gamma), _ptr(beta), _ptr(y),
                                 _ptr(sum_out), _ptr(mean), _ptr(rstd), M, N, float(eps), dt,
                                 _ptr(ws), ws_bytes, _stream(dev, stream), _opt(options)),
           "norm_ln_fwd_add")
    return y, sum_out


def norm_rms_bwd_add(dy, sum_in, gamma, rstd, dsum, dx, dgamma, workspace=None, stream=None,
                     options=None):
    """dx = RMSNorm backward at sum_in (+ dsum, the gradient arriving at the sum, if given);
    dgamma overwritten."""
    torch = _torch()
    M, N, dev = _shape(sum_in)
    for t, n in ((dy, "dy"), (sum_in, "sum_in"), (dsum, "dsum"), (dx, "dx")):
        _need(t, n, M * N, sum_in.dtype, dev)
    _need(gamma, "gamma", N, _pdtype(sum_in, gamma), dev)
    _need(rstd, "rstd", M, torch.float32, dev)
    _need(dgamma, "dgamma", N, torch.float32, dev)
    dt = _types(sum_in, gamma)
    ws, ws_bytes = _workspace(M, N, False, dt, dev, workspace, options, stream)
    _check(lib().norm_rms_bwd_add(_ptr(dy), _ptr(sum_in), _ptr(gamma), _ptr(rstd), _ptr(dsum),
                                  _ptr(dx), _ptr(dgamma), M, N, dt, _ptr(ws), ws_bytes,
                                  _stream(dev, stream), _opt(options)),
           "norm_rms_bwd_add")
    return dx, dgamma


def norm_ln_bwd_add(dy, sum_in, gamma, mean, rstd, dsum, dx, dgamma, dbeta, workspace=None,
                    stream=None, options=None):
    """dx = LayerNorm backward at sum_in (+ dsum if given); dgamma, dbeta overwritten."""
    torch = _torch()
    M, N, dev = _shape(sum_in)
    for t, n in ((dy, "dy"), (sum_in, "sum_in"), (dsum, "dsum"), (dx, "dx")):
        _need(t, n, M * N, sum_in.dtype, dev)
    _need(gamma, "gamma", N, _pdtype(sum_in, gamma), dev)
    for t, n, k in ((mean, "mean", M), (rstd, "rstd", M), (dgamma, "dgamma", N),
                    (dbeta, "dbeta", N)):
        _need(t, n, k, torch.float32, dev)
    dt = _types(sum_in, gamma)
    ws, ws_bytes = _workspace(M, N, True, dt, dev, workspace, options, stream)
    _check(lib().norm_ln_bwd_add(_ptr(dy), _ptr(sum_in), _ptr(gamma), _ptr(mean), _ptr(rstd),
                                 _ptr(dsum), _ptr(dx), _ptr(dgamma), _ptr(dbeta), M, N, dt,
                                 _ptr(ws), ws_bytes, _stream(dev, stream),
                                 _opt(options)), "norm_ln_bwd_add")
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
