"""Fused LayerNorm / RMSNorm for AMD MI355X (gfx950): Python binding.

Thin ctypes layer over ``libnormfuse.so`` (the C ABI of ``include/normfuse.h``).
It only marshals arguments: torch supplies device memory (``data_ptr``) and
the stream (``torch.cuda.current_stream()``); every step of the computation
runs in the library's HIP kernels.  There is no fallback: without the built
library, importing works but every call raises ``NormLibraryMissing``.

Operations (definitions in ``include/normfuse.h``):
  ln_fwd / rms_fwd   fused (bias +) residual + LayerNorm / RMSNorm forward
                     with optional residual_out, mean / rstd and amax
  ln_fwd_fp8 / rms_fwd_fp8
                     the same forward with y as FP8 E4M3 codes of y * scale
  ln_bwd / rms_bwd   backward: dx plus dgamma / dbeta (and optionally dbias)
                     from one read of dy, x
  softmax_fwd        row softmax in one read of x
Option keywords: ``zero_centered_gamma`` (forward and backward) and
``dparam_mean`` (backward).
"""
import ctypes
import os

import torch

from .build import LIB as _LIB_PATH
from .build import TUNING_LIB as _TUNING_LIB_PATH

__all__ = ["ln_fwd", "rms_fwd", "ln_fwd_fp8", "rms_fwd_fp8", "ln_bwd", "rms_bwd", "softmax_fwd",
           "ln_bwd_noalloc", "bwd_workspace_size", "describe", "amax_workspace", "NormError",
           "NormLibraryMissing", "library", "load", "TUNING_LIB", "F32", "BF16", "N_MAX",
           "ZERO_CENTERED_GAMMA", "DPARAM_MEAN", "STATIC_SCRATCH_BYTES", "AMAX_WS_BYTES"]

F32 = 0
BF16 = 1
N_MAX = 16384
STATUS = {0: "NORM_OK", 1: "NORM_ERR_NULL", 2: "NORM_ERR_SHAPE", 3: "NORM_ERR_ARG",
          4: "NORM_ERR_DTYPE", 5: "NORM_ERR_ALIGN", 6: "NORM_ERR_WORKSPACE", 7: "NORM_ERR_LAUNCH",
          8: "NORM_ERR_DEVICE"}
ZERO_CENTERED_GAMMA = 1  # option bits of include/normfuse.h
DPARAM_MEAN = 2

EXPORTS = ("ln_fwd", "rms_fwd", "ln_fwd_fp8", "rms_fwd_fp8", "ln_bwd", "rms_bwd",
           "softmax_fwd", "norm_bwd_workspace_size", "norm_status_string", "norm_describe",
           "ln_bwd_noalloc")
STATIC_SCRATCH_BYTES = 32 << 20  # NORM_STATIC_SCRATCH_BYTES
# operation codes and option bits of norm_describe
OPS = {"ln_fwd": 0, "rms_fwd": 1, "ln_bwd": 2, "rms_bwd": 3, "softmax_fwd": 4}
DESCRIBE_AMAX, DESCRIBE_FP8, DESCRIBE_DBIAS, DESCRIBE_AMAX_WS = 1, 2, 4, 8
AMAX_WS_BYTES = 4160  # NORM_AMAX_WS_BYTES


class NormLibraryMissing(RuntimeError):
    pass


class NormError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({text})")
        self.status = status


_lib = None
_product_lib = None  # the product build, once loaded


def library():
    """The loaded ``libnormfuse.so`` (ctypes), with argument types set."""
    global _lib, _product_lib
    if _lib is None:
        _lib = _product_lib = load(_LIB_PATH)
    return _lib


def load(path):
    """Load a build of the library at ``path`` (ctypes) and set its argument
    types.  The package's functions use :func:`library`; the test build
    ``libnormfuse_tuning.so`` (same kernels, host code that also reads the
    ``NORMFUSE_*`` tuning overrides) is loaded with ``load(TUNING_LIB)``."""
    if not os.path.exists(path):
        raise NormLibraryMissing(
            f"{path} is not built; run normalization_ln_fwd_amd/build.py "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    vp, i64, i32, f32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                             ctypes.c_float, ctypes.c_size_t)
    u32 = ctypes.c_uint32
    fwd = [vp, vp, vp, vp, vp, f32, i64, i64, i32, vp, vp, vp, vp, vp, vp, u32, vp]
    lib.ln_fwd.argtypes = fwd
    lib.rms_fwd.argtypes = fwd
    fwd8 = [vp, vp, vp, vp, vp, f32, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, u32, vp]
    lib.ln_fwd_fp8.argtypes = fwd8
    lib.rms_fwd_fp8.argtypes = fwd8
    lib.ln_bwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, vp, vp, vp, vp, i32, vp, sz,
                           u32, vp]
    lib.rms_bwd.argtypes = [vp, vp, vp, vp, f32, i64, i64, i32, vp, vp, vp, vp, i32, vp, sz,
                            u32, vp]
    lib.softmax_fwd.argtypes = [vp, i64, i64, i32, vp, u32, vp]
    lib.norm_bwd_workspace_size.argtypes = [i64, i64, i32, ctypes.POINTER(sz)]
    lib.norm_status_string.argtypes = [i32]
    lib.norm_status_string.restype = ctypes.c_char_p
    lib.norm_describe.argtypes = [i32, i64, i64, i32, u32, ctypes.c_char_p, sz]
    lib.ln_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, vp, vp, vp, vp, i32, u32,
                                   vp]
    for name in ("ln_fwd", "rms_fwd", "ln_fwd_fp8", "rms_fwd_fp8", "ln_bwd", "rms_bwd",
                 "softmax_fwd", "norm_bwd_workspace_size", "norm_describe", "ln_bwd_noalloc"):
        getattr(lib, name).restype = i32
    return lib


TUNING_LIB = _TUNING_LIB_PATH


def _check(fn, st):
    if st != 0:
        raise NormError(fn, st, library().norm_status_string(st).decode())


def _dtype_code(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _ptr(t, name, dtype=None, numel=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")
    return t.data_ptr()


def _fresh_views(device, *sizes, dtype=torch.float32):
    """Fresh tensors of the given sizes (None for 0), carved from one
    allocation: per call, one allocator round trip instead of several."""
    total = sum(sizes)
    if total == 0:
        return [None] * len(sizes)
    buf = torch.empty(total, dtype=dtype, device=device)
    views, at = [], 0
    for n in sizes:
        views.append(buf[at:at + n] if n else None)
        at += n
    return views


# The raw handle of the current stream without building a Stream object
# (a few microseconds per call otherwise).
_current_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, device):
    """The raw stream handle: ``stream``'s, else the current stream of the
    tensors' device (kernels run on the stream's device, so that the
    tensors need not be on the current device)."""
    if stream is not None:
        return stream.cuda_stream
    if _current_raw_stream is not None:
        return _current_raw_stream(device.index if device.index is not None
                                   else torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


def amax_workspace(device=None):
    """A zero-filled amax workspace (NORM_AMAX_WS_BYTES) for the forwards'
    ``amax_workspace``: allocate once and pass it to every call on one
    stream; each call leaves it zero-filled again."""
    return torch.zeros(AMAX_WS_BYTES, dtype=torch.uint8,
                       device=device if device is not None else "cuda")


def _fwd(fn, x, bias, residual, gamma, beta, eps, want_residual_out, want_mean, want_rstd,
         want_amax, stream, out, y_scale=None, zero_centered_gamma=False, amax_workspace=None):
    lib = library()
    N = x.shape[-1]
    M = x.numel() // N if N else 0
    dt = x.dtype
    fp8 = fn.endswith("_fp8")
    out = out or {}
    # outputs not given are allocated here (and need no checks); mean, rstd
    # and amax share one allocation
    y = out.get("y")
    if y is None:
        y = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=x.device) if fp8 \
            else torch.empty_like(x)
        y_p = y.data_ptr()
    else:
        if fp8 and y.dtype not in (torch.float8_e4m3fn, torch.uint8):
            raise TypeError(f"y: expected float8_e4m3fn or uint8, got {y.dtype}")
        y_p = _ptr(y, "y", y.dtype if fp8 else dt, M * N)
    res_out = out.get("residual_out")
    if res_out is None and want_residual_out:
        res_out = torch.empty_like(x)
        res_p = res_out.data_ptr()
    else:
        res_p = _ptr(res_out, "residual_out", dt, M * N)
    mean, rstd, amax = out.get("mean"), out.get("rstd"), out.get("amax")
    new_mean, new_rstd, new_amax = _fresh_views(
        x.device, M if mean is None and want_mean else 0, M if rstd is None and want_rstd else 0,
        1 if amax is None and want_amax else 0)
    stat_shape = x.shape[:-1]
    mean_p = _ptr(mean, "mean", torch.float32, M)
    if new_mean is not None:
        mean, mean_p = new_mean.view(stat_shape), new_mean.data_ptr()
    rstd_p = _ptr(rstd, "rstd", torch.float32, M)
    if new_rstd is not None:
        rstd, rstd_p = new_rstd.view(stat_shape), new_rstd.data_ptr()
    amax_p = _ptr(amax, "amax", torch.float32, 1)
    if new_amax is not None:
        amax, amax_p = new_amax, new_amax.data_ptr()
    head = [_ptr(x, "x"), _ptr(bias, "bias", dt, N), _ptr(residual, "residual", dt, M * N),
            _ptr(gamma, "gamma", dt, N), _ptr(beta, "beta", dt, N), float(eps), M, N,
            _dtype_code(x)]
    if fp8:
        head.append(_ptr(y_scale, "y_scale", torch.float32, 1))
    st = getattr(lib, fn)(
        *head, y_p, res_p, mean_p, rstd_p, amax_p, _ws_ptr(amax_workspace),
        ZERO_CENTERED_GAMMA if zero_centered_gamma else 0, _stream(stream, x.device))
    _check(fn, st)
    return {"y": y, "residual_out": res_out, "mean": mean, "rstd": rstd, "amax": amax}


def _ws_ptr(ws):
    if ws is None:
        return None
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("amax_workspace must be a contiguous GPU tensor")
    if ws.numel() * ws.element_size() < AMAX_WS_BYTES:
        raise ValueError(f"amax_workspace must hold at least {AMAX_WS_BYTES} bytes")
    return ws.data_ptr()


def ln_fwd(x, bias=None, residual=None, gamma=None, beta=None, eps=1e-5, *,
           want_residual_out=None, want_stats=True, want_amax=False, zero_centered_gamma=False,
           amax_workspace=None, stream=None, out=None):
    """Fused (bias +) residual + LayerNorm over the last dimension of ``x``.

    Returns a dict with ``y``, ``residual_out`` (when bias or residual is given,
    unless disabled), ``mean`` / ``rstd`` (fp32, when ``want_stats``) and
    ``amax`` (1-element fp32, when ``want_amax``).  ``out`` may supply any of
    these tensors preallocated.  ``zero_centered_gamma``: the weight is
    1 + gamma.  ``amax_workspace`` (see :func:`amax_workspace`): amax in one
    kernel launch instead of a reset kernel and the forward.
    """
    if want_residual_out is None:
        want_residual_out = bias is not None or residual is not None
    return _fwd("ln_fwd", x, bias, residual, gamma, beta, eps, want_residual_out, want_stats,
                want_stats, want_amax, stream, out, zero_centered_gamma=zero_centered_gamma,
                amax_workspace=amax_workspace)


def rms_fwd(x, bias=None, residual=None, gamma=None, beta=None, eps=1e-6, *,
            want_residual_out=None, want_stats=True, want_amax=False, zero_centered_gamma=False,
            amax_workspace=None, stream=None, out=None):
    """Fused (bias +) residual + RMSNorm; as :func:`ln_fwd` without ``mean``."""
    if want_residual_out is None:
        want_residual_out = bias is not None or residual is not None
    return _fwd("rms_fwd", x, bias, residual, gamma, beta, eps, want_residual_out, False,
                want_stats, want_amax, stream, out, zero_centered_gamma=zero_centered_gamma,
                amax_workspace=amax_workspace)


def ln_fwd_fp8(x, y_scale, bias=None, residual=None, gamma=None, beta=None, eps=1e-5, *,
               want_residual_out=None, want_stats=True, want_amax=False,
               zero_centered_gamma=False, amax_workspace=None, stream=None, out=None):
    """:func:`ln_fwd` with ``y`` as OCP FP8 E4M3 codes of y * y_scale
    (``y_scale``: a 1-element fp32 tensor on the GPU); ``y`` is returned as a
    ``float8_e4m3fn`` tensor (``out`` may supply one, or a ``uint8`` one)."""
    if want_residual_out is None:
        want_residual_out = bias is not None or residual is not None
    return _fwd("ln_fwd_fp8", x, bias, residual, gamma, beta, eps, want_residual_out,
                want_stats, want_stats, want_amax, stream, out, y_scale, zero_centered_gamma,
                amax_workspace)


def rms_fwd_fp8(x, y_scale, bias=None, residual=None, gamma=None, beta=None, eps=1e-6, *,
                want_residual_out=None, want_stats=True, want_amax=False,
                zero_centered_gamma=False, amax_workspace=None, stream=None, out=None):
    """:func:`rms_fwd` with ``y`` as OCP FP8 E4M3 codes of y * y_scale."""
    if want_residual_out is None:
        want_residual_out = bias is not None or residual is not None
    return _fwd("rms_fwd_fp8", x, bias, residual, gamma, beta, eps, want_residual_out, False,
                want_stats, want_amax, stream, out, y_scale, zero_centered_gamma, amax_workspace)


def softmax_fwd(x, *, stream=None, out=None):
    """Row softmax over the last dimension of ``x`` (bf16 or fp32), one read
    of x: returns y of x's shape and dtype (``out`` may supply it)."""
    lib = library()
    N = x.shape[-1]
    M = x.numel() // N if N else 0
    y = out if out is not None else torch.empty_like(x)
    _check("softmax_fwd", lib.softmax_fwd(_ptr(x, "x"), M, N, _dtype_code(x),
                                          _ptr(y, "y", x.dtype, M * N), 0,
                                          _stream(stream, x.device)))
    return y


_DTYPE_NAMES = {"f32": F32, "fp32": F32, "float32": F32, "bf16": BF16, "bfloat16": BF16}


def _code_of(dtype):
    """The library's dtype code of ``dtype``: a code, a torch dtype or a name."""
    if isinstance(dtype, int) and dtype in (F32, BF16):
        return dtype
    if dtype == torch.float32:
        return F32
    if dtype == torch.bfloat16:
        return BF16
    if isinstance(dtype, str) and dtype in _DTYPE_NAMES:
        return _DTYPE_NAMES[dtype]
    raise TypeError(f"unsupported dtype {dtype!r}; use float32 or bfloat16")


def describe(op, M, N, dtype, *, amax=False, fp8=False, dbias=False, amax_ws=False):
    """Text naming the kernels, grid and walk a call of ``op`` ("ln_fwd",
    "rms_fwd", "ln_bwd", "rms_bwd", "softmax_fwd"; the _fp8 forwards with
    ``fp8=True``) on an [M, N] problem would launch, for 16-byte aligned
    tensors.  Touches no device."""
    lib = library()
    code = _code_of(dtype)
    opts = (DESCRIBE_AMAX if amax else 0) | (DESCRIBE_FP8 if fp8 else 0) | \
        (DESCRIBE_DBIAS if dbias else 0) | (DESCRIBE_AMAX_WS if amax_ws else 0)
    buf = ctypes.create_string_buffer(512)
    _check("norm_describe", lib.norm_describe(OPS[op], M, N, code, opts, buf, len(buf)))
    return buf.value.decode()


def bwd_workspace_size(M, N, dtype):
    """Workspace bytes ln_bwd / rms_bwd need for an [M, N] problem."""
    lib = library()
    n = ctypes.c_size_t(0)
    code = _code_of(dtype)
    _check("norm_bwd_workspace_size", lib.norm_bwd_workspace_size(M, N, code, ctypes.byref(n)))
    return n.value


# Workspace sizes the product library gave, by (M, N, dtype): a pure
# function of them there (the test build's depends on its overrides too,
# and is asked every time).
_ws_bytes = {}


def _workspace_bytes(lib, M, N, dtype):
    if lib is not _product_lib:
        return bwd_workspace_size(M, N, dtype)
    key = (M, N, dtype)
    n = _ws_bytes.get(key)
    if n is None:
        if len(_ws_bytes) >= 1024:
            _ws_bytes.clear()
        n = _ws_bytes[key] = bwd_workspace_size(M, N, dtype)
    return n


def _bwd(fn, dy, x, gamma, mean, rstd, eps, dparam_dtype, want_dgamma, want_dbeta, want_dbias,
         workspace, stream, out, flags=0):
    dt = x.dtype
    pdt = dt if dparam_dtype is None else dparam_dtype
    if pdt not in (torch.float32, torch.bfloat16):
        raise TypeError(f"dparam_dtype {pdt} unsupported; use torch.float32 or torch.bfloat16")
    lib = library()
    N = x.shape[-1]
    M = x.numel() // N if N else 0
    out = out or {}
    dx = out.get("dx")
    if dx is None:
        dx = torch.empty_like(x)
    # the parameter gradients not given share one allocation
    dgamma, dbeta, dbias = out.get("dgamma"), out.get("dbeta"), out.get("dbias")
    new = _fresh_views(x.device, N if dgamma is None and want_dgamma else 0,
                     N if dbeta is None and want_dbeta else 0,
                     N if dbias is None and want_dbias else 0, dtype=pdt)
    dgamma = dgamma if new[0] is None else new[0]
    dbeta = dbeta if new[1] is None else new[1]
    dbias = dbias if new[2] is None else new[2]
    noalloc = fn == "ln_bwd_noalloc"
    if workspace is None and not noalloc:
        need = _workspace_bytes(lib, M, N, dt)
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=x.device)
    pcode = F32 if pdt == torch.float32 else BF16
    args = [_ptr(dy, "dy", dt, M * N), _ptr(x, "x"), _ptr(gamma, "gamma", dt, N)]
    if fn != "rms_bwd":
        args += [_ptr(mean, "mean", torch.float32, M), _ptr(rstd, "rstd", torch.float32, M)]
    else:
        args += [_ptr(rstd, "rstd", torch.float32, M), float(eps)]
    args += [M, N, _dtype_code(x), _ptr(dx, "dx", dt, M * N),
             _ptr(dgamma, "dgamma", pdt, N), _ptr(dbeta, "dbeta", pdt, N),
             _ptr(dbias, "dbias", pdt, N), pcode]
    if not noalloc:
        args += [_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size()]
    args += [flags, _stream(stream, x.device)]
    if noalloc and x.device.index is not None and x.device.index != torch.cuda.current_device():
        # the static scratch is the current device's: make x's device current
        with torch.cuda.device(x.device):
            _check(fn, getattr(lib, fn)(*args))
    else:
        _check(fn, getattr(lib, fn)(*args))
    return {"dx": dx, "dgamma": dgamma, "dbeta": dbeta, "dbias": dbias}


def _bwd_flags(zero_centered_gamma, dparam_mean):
    return (ZERO_CENTERED_GAMMA if zero_centered_gamma else 0) | (DPARAM_MEAN if dparam_mean
                                                                  else 0)


def ln_bwd(dy, x, gamma, mean, rstd, *, dparam_dtype=None, want_dgamma=True, want_dbeta=True,
           want_dbias=False, zero_centered_gamma=False, dparam_mean=False, workspace=None,
           stream=None, out=None):
    """LayerNorm backward (dx, dgamma, dbeta) from one read of dy and x.
    ``dparam_dtype`` (default: x's dtype) is the type of dgamma / dbeta.
    ``want_dbias`` also returns the gradient of the forward's bias (the
    column sums of dx), for a forward that fused (x + bias) + residual.
    ``zero_centered_gamma``: the forward's weight was 1 + gamma;
    ``dparam_mean``: the column results are means over the rows."""
    return _bwd("ln_bwd", dy, x, gamma, mean, rstd, 0.0, dparam_dtype, want_dgamma, want_dbeta,
                want_dbias, workspace, stream, out, _bwd_flags(zero_centered_gamma, dparam_mean))


def ln_bwd_noalloc(dy, x, gamma, mean, rstd, *, dparam_dtype=None, want_dgamma=True,
                   want_dbeta=True, want_dbias=False, zero_centered_gamma=False,
                   dparam_mean=False, stream=None, out=None):
    """:func:`ln_bwd` on the library's static device scratch instead of a
    workspace (for callers that cannot allocate; pass every output in
    ``out`` to allocate nothing here either).  Calls that overlap on one GPU
    race; problems needing more than STATIC_SCRATCH_BYTES are refused."""
    return _bwd("ln_bwd_noalloc", dy, x, gamma, mean, rstd, 0.0, dparam_dtype, want_dgamma,
                want_dbeta, want_dbias, None, stream, out,
                _bwd_flags(zero_centered_gamma, dparam_mean))


def rms_bwd(dy, x, gamma, rstd=None, eps=1e-6, *, dparam_dtype=None, want_dgamma=True,
            want_dbeta=False, want_dbias=False, zero_centered_gamma=False, dparam_mean=False,
            workspace=None, stream=None, out=None):
    """RMSNorm backward; ``rstd=None`` recomputes it from ``x`` and ``eps``."""
    return _bwd("rms_bwd", dy, x, gamma, None, rstd, eps, dparam_dtype, want_dgamma, want_dbeta,
                want_dbias, workspace, stream, out, _bwd_flags(zero_centered_gamma, dparam_mean))
