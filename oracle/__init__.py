"""Double-precision CPU oracle for fused LayerNorm / RMSNorm (forward with
bias + residual + amax, backward with dx / dgamma / dbeta).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only callers.  The GPU library never
imports or links it and shares no code with it.

Parity status of each function (what pins it, in ``tests/test_oracle.py``):
  norm_fwd (LayerNorm)  -- pinned: closed-form worked example, mean/variance
                           invariants, special cases, torch's float64
                           ``layer_norm`` (the call the nvFuser layernorm + amax
                           comment makes), brute-force amax.
  norm_fwd (RMSNorm)    -- pinned: closed-form worked example, mean-square
                           invariant, torch's float64 ``rms_norm``.
  norm_bwd (both)       -- pinned: central finite differences of the forward,
                           the closed-form row invariants of dx, special cases,
                           float64 autograd, brute-force column sums.
  norm_bwd dbias        -- pinned: central finite differences of the forward
                           with respect to bias, float64 autograd through
                           (x + bias) + residual, and (LayerNorm) the closed
                           form sum_j dbias_j = 0.
  round_to_dtype        -- pinned: exhaustive checks against exactly
                           representable neighbours and ties.
  zero_centered_gamma   -- pinned: torch's float64 layer_norm / rms_norm with
                           the weight `1 + gamma` formed by torch in the I/O
                           dtype (the expression the nvFuser comment uses), and
                           float64 autograd of dx / dgamma through w = 1 + gamma.
  dparam_mean           -- pinned: the closed form of dbeta's row mean with a
                           row-constant dy, and the sums over M rows / M.
  softmax_fwd           -- pinned: torch's float64 softmax, rows summing to 1,
                           shift invariance, the two-element closed form, a
                           constant row (1/N) and a large row offset.
  quantize_e4m3         -- pinned: torch's float8_e4m3fn cast on every code,
                           every midpoint and its neighbours and random
                           in-range values; the format's fixed codes
                           (1.0, 448, 2^-6, 2^-9); saturation and NaN.

This module is a thin ctypes shim over ``liboracle.so`` (built from
``oracle.c`` by ``oracle/build.py``); arrays are numpy.  bf16 tensors are
passed as ``uint16`` arrays of bf16 bit patterns, fp32 tensors as float32.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32 = 0
BF16 = 1

_lib = None


def _load():
    global _lib
    if _lib is None:
        # A test may point this at a deliberately altered build of oracle.c
        # to check that the pins catch the alteration.
        path = os.environ.get("NORMFUSE_ORACLE_LIB")
        if path is None:
            path = _build.LIB
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
                _build.build()
        lib = ctypes.CDLL(path)
        vp, i64, dbl, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double, ctypes.c_int
        lib.oracle_norm_fwd.argtypes = [ci, vp, vp, vp, vp, vp, dbl, i64, i64, ci, ci,
                                        vp, vp, vp, vp, vp, ci]
        lib.oracle_norm_fwd.restype = ci
        lib.oracle_norm_bwd.argtypes = [ci, vp, vp, vp, vp, vp, dbl, i64, i64, ci, ci,
                                        vp, vp, vp, vp, vp, vp, vp, vp, ci, ci]
        lib.oracle_norm_bwd.restype = ci
        lib.oracle_round_to_dtype.argtypes = [vp, i64, ci, vp]
        lib.oracle_round_to_dtype.restype = ci
        lib.oracle_quantize_e4m3.argtypes = [vp, i64, ctypes.c_float, vp]
        lib.oracle_quantize_e4m3.restype = ci
        lib.oracle_softmax_fwd.argtypes = [vp, i64, i64, ci, ci, vp]
        lib.oracle_softmax_fwd.restype = ci
        _lib = lib
    return _lib


def _io_dtype(dtype):
    return np.float32 if dtype == F32 else np.uint16


def _ptr(a):
    return None if a is None else a.ctypes.data


def _in(a, dtype, shape=None, name="array"):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype != _io_dtype(dtype):
        raise TypeError(f"{name}: expected {_io_dtype(dtype).__name__}, got {a.dtype}")
    if shape is not None and a.shape != shape:
        raise ValueError(f"{name}: expected shape {shape}, got {a.shape}")
    return a


def default_threads():
    return max(1, len(os.sched_getaffinity(0)))


def norm_fwd(x, bias=None, residual=None, gamma=None, beta=None, eps=1e-5, *,
             rms=False, dtype=BF16, nthreads=None, want_u=True, want_y=True,
             zero_centered_gamma=False):
    """Forward of the fused op on an (M, N) matrix.

    Returns a dict: ``u`` (residual_out, I/O dtype), ``y`` (float64, exact,
    unrounded), ``mean`` / ``rstd`` (float64 [M]; mean is 0 for RMSNorm) and
    ``amax`` (float64 scalar, max |y| after rounding y to the I/O dtype).
    ``zero_centered_gamma``: the weight is 1 + gamma, formed in the I/O dtype.
    """
    lib = _load()
    x = _in(x, dtype, name="x")
    M, N = x.shape
    bias = _in(bias, dtype, (N,), "bias")
    residual = _in(residual, dtype, (M, N), "residual")
    gamma = _in(gamma, dtype, (N,), "gamma")
    beta = _in(beta, dtype, (N,), "beta")
    u = np.empty((M, N), _io_dtype(dtype)) if want_u else None
    y = np.empty((M, N), np.float64) if want_y else None
    mean = np.empty(M, np.float64)
    rstd = np.empty(M, np.float64)
    amax = np.zeros(1, np.float64)
    rc = lib.oracle_norm_fwd(int(rms), _ptr(x), _ptr(bias), _ptr(residual), _ptr(gamma),
                             _ptr(beta), float(eps), M, N, dtype,
                             nthreads or default_threads(), _ptr(u), _ptr(y), _ptr(mean),
                             _ptr(rstd), _ptr(amax), int(bool(zero_centered_gamma)))
    if rc != 0:
        raise ValueError("oracle_norm_fwd rejected its arguments")
    return {"u": u, "y": y, "mean": mean, "rstd": rstd, "amax": float(amax[0])}


def norm_bwd(dy, x, gamma=None, mean=None, rstd=None, eps=1e-5, *, rms=False,
             dtype=BF16, nthreads=None, want_dx=True, want_params=True, want_dbias=False,
             zero_centered_gamma=False, dparam_mean=False):
    """Backward on an (M, N) matrix.

    ``mean`` / ``rstd`` are per-row arrays (any float dtype, widened exactly
    to float64); RMSNorm takes ``rstd=None`` to recompute it from ``x``.
    Returns a dict of float64 arrays: ``dx`` (M, N), ``dgamma``, ``dbeta``,
    ``dgamma_l2``, ``dbeta_l2`` (N,), all unrounded, and ``rstd`` (M,), the
    rstd the gradients used; with ``want_dbias`` also ``dbias`` (N,), the
    gradient of the forward's bias (column sums of dx), and ``dbias_l2``.
    ``zero_centered_gamma``: the forward's weight was 1 + gamma.
    ``dparam_mean``: the column results (and their 2-norms) are divided by M.
    """
    lib = _load()
    dy = _in(dy, dtype, name="dy")
    M, N = dy.shape
    x = _in(x, dtype, (M, N), "x")
    gamma = _in(gamma, dtype, (N,), "gamma")
    mean = None if mean is None else np.ascontiguousarray(mean, np.float64).reshape(M)
    rstd = None if rstd is None else np.ascontiguousarray(rstd, np.float64).reshape(M)
    dx = np.empty((M, N), np.float64) if want_dx else None
    out = {k: (np.empty(N, np.float64) if want_params else None)
           for k in ("dgamma", "dbeta", "dgamma_l2", "dbeta_l2")}
    for k in ("dbias", "dbias_l2"):
        out[k] = np.empty(N, np.float64) if want_dbias else None
    rstd_used = np.empty(M, np.float64)
    rc = lib.oracle_norm_bwd(int(rms), _ptr(dy), _ptr(x), _ptr(gamma), _ptr(mean), _ptr(rstd),
                             float(eps), M, N, dtype, nthreads or default_threads(), _ptr(dx),
                             _ptr(out["dgamma"]), _ptr(out["dbeta"]), _ptr(out["dgamma_l2"]),
                             _ptr(out["dbeta_l2"]), _ptr(rstd_used), _ptr(out["dbias"]),
                             _ptr(out["dbias_l2"]), int(bool(zero_centered_gamma)),
                             int(bool(dparam_mean)))
    if rc != 0:
        raise ValueError("oracle_norm_bwd rejected its arguments")
    out["dx"] = dx
    out["rstd"] = rstd_used
    return out


def round_to_dtype(v, dtype=BF16):
    """Round float64 values to the I/O dtype (ties to even); returns the
    dtype's storage array (uint16 bf16 patterns or float32)."""
    lib = _load()
    v = np.ascontiguousarray(v, np.float64)
    out = np.empty(v.shape, _io_dtype(dtype))
    if lib.oracle_round_to_dtype(_ptr(v), v.size, dtype, _ptr(out)) != 0:
        raise ValueError("oracle_round_to_dtype rejected its arguments")
    return out


def quantize_e4m3(v, scale):
    """OCP FP8 E4M3 codes (uint8) of the fp32 products ``v * scale``: round to
    nearest, ties to even, magnitudes beyond 448 saturate.  ``v`` is taken as
    float32 values (bf16 patterns must be widened by the caller)."""
    lib = _load()
    v = np.ascontiguousarray(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    if lib.oracle_quantize_e4m3(_ptr(v), v.size, float(np.float32(scale)), _ptr(out)) != 0:
        raise ValueError("oracle_quantize_e4m3 rejected its arguments")
    return out


def softmax_fwd(x, *, dtype=BF16, nthreads=None):
    """Row softmax of an (M, N) matrix in the I/O dtype: float64 (M, N),
    unrounded."""
    lib = _load()
    x = _in(x, dtype, name="x")
    M, N = x.shape
    y = np.empty((M, N), np.float64)
    if lib.oracle_softmax_fwd(_ptr(x), M, N, dtype, nthreads or default_threads(), _ptr(y)) != 0:
        raise ValueError("oracle_softmax_fwd rejected its arguments")
    return y


def bf16_bits_to_f64(a):
    """Exact value of bf16 bit patterns (uint16) as float64."""
    a = np.asarray(a, np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
