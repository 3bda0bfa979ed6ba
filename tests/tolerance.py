"""Parity tolerances (test infrastructure).

  * fp32 outputs (y, dx): |got - ref| <= 1e-5 * s_i, with s_i the row scale
    max_j |ref_ij| (1 where the row is all zero); for dx the row scale is at
    least the scale of the terms dx is formed from, rstd_i * max_j |dy_ij
    gamma_j| (dx = rstd * (g - ...) cancels to far below its terms when, e.g.,
    N = 1);
  * residual_out (the fused add, computed in fp32 as (x + bias) + residual and
    rounded once to the I/O dtype, against the exact sum rounded once): one
    ulp of the I/O dtype plus the two fp32 additions' rounding bound
    2^-23 * (|x| + |bias| + |residual|);
  * bf16 outputs (y, dx, residual_out): |got - ref| <= max(ulp_bf16(ref),
    1e-5 * s_i), ulp_bf16(v) = 2^(floor(log2 |v|) - 7) -- one bf16 ulp, with
    an absolute floor where cancellation makes an element tiny next to its row;
  * column sums (dgamma, dbeta, dbias): |got - ref| <= rel * max(|ref|,
    ||terms||_2), ||terms||_2 being the 2-norm of the summed terms (the scale a
    zero-mean sum is compared against); for dbias, whose terms are dx, at least
    the 2-norm of dx's own terms rstd * |dy * gamma| (dbias_term_l2); bf16
    outputs additionally may be one bf16 ulp off.
The reference ``ref`` is the oracle's exact (double) value.
"""
import numpy as np

F32, BF16 = 0, 1


def ulp_bf16(ref):
    a = np.abs(np.asarray(ref, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126.0)
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


def ulp_io(ref, dtype):
    if dtype == BF16:
        return ulp_bf16(ref)
    return np.spacing(np.abs(np.asarray(ref, np.float32))).astype(np.float64)


def row_scale(ref):
    s = np.max(np.abs(ref), axis=-1, keepdims=True) if ref.shape[-1] else np.ones(ref.shape[:-1] + (1,))
    return np.where(s > 0, s, 1.0)


def _report(name, got, ref, err, tol, bad):
    idx = np.argwhere(bad)[:5]
    lines = [f"{name}: {int(bad.sum())} of {bad.size} elements out of tolerance"]
    for ij in idx:
        t = tuple(ij)
        lines.append(f"  at {t}: got {got[t]!r} ref {ref[t]!r} err {err[t]:.3e} tol {tol[t]:.3e}")
    return "\n".join(lines)


def dx_term_scale(dy, gamma, rstd, dtype):
    """Per-row scale of the terms of dx: rstd_i * max_j |dy_ij * gamma_j|."""
    dy = to_f64(dy, dtype)
    g = dy if gamma is None else dy * to_f64(gamma, dtype)[None, :]
    return np.asarray(rstd, np.float64).reshape(-1) * np.max(np.abs(g), axis=1)


def dbias_term_l2(dy, gamma, rstd, dtype):
    """Per-column 2-norm over the rows of rstd_i * |dy_ij * gamma_j|, the
    scale of the terms each dx_ij is formed from.  dbias_j sums dx_ij; where
    dx cancels to almost nothing (e.g. N = 1) its rounding error is relative
    to these terms, not to dx."""
    dy = to_f64(dy, dtype)
    g = dy if gamma is None else dy * to_f64(gamma, dtype)[None, :]
    r = np.asarray(rstd, np.float64).reshape(-1, 1)
    return np.sqrt(np.sum((r * g) ** 2, axis=0))


def to_f64(a, dtype):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def assert_rows_close(got, ref, dtype, name, rel_floor=1e-5, ulps=1.0, scale=None):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    s = row_scale(ref)
    if scale is not None:
        s = np.maximum(s, np.asarray(scale, np.float64).reshape(-1, 1))
    err = np.abs(got - ref)
    tol = rel_floor * s * np.ones_like(ref)
    if dtype == BF16:
        tol = np.maximum(ulps * ulp_bf16(ref), tol)
    bad = ~(err <= tol)
    assert not bad.any(), _report(name, got, ref, err, tol, bad)
    return float(np.max(err / tol))


def assert_within_ulps(got, ref, dtype, name, ulps=1.0):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    tol = ulps * ulp_io(ref, dtype) + np.where(ref == 0, 2.0 ** -133, 0.0)
    bad = ~(err <= tol)
    assert not bad.any(), _report(name, got, ref, err, tol, bad)


def assert_fused_add_close(u_got, u_ref, inp, dtype, name):
    """residual_out against the oracle's rounded exact sum (storage arrays)."""
    got, ref = to_f64(u_got, dtype), to_f64(u_ref, dtype)
    terms = np.abs(to_f64(inp["x"], dtype))
    if inp.get("bias") is not None:
        terms = terms + np.abs(to_f64(inp["bias"], dtype))[None, :]
    if inp.get("residual") is not None:
        terms = terms + np.abs(to_f64(inp["residual"], dtype))
    err = np.abs(got - ref)
    tol = ulp_io(ref, dtype) + 2.0 ** -23 * terms
    bad = ~(err <= tol)
    assert not bad.any(), _report(name, got, ref, err, tol, bad)


def assert_colsums_close(got, ref, l2, rel, name, dtype=F32):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.maximum(np.abs(ref), l2)
    scale = np.where(scale > 0, scale, 1.0)
    err = np.abs(got - ref)
    tol = rel * scale
    if dtype == BF16:
        tol = np.maximum(tol, ulp_bf16(ref))
    bad = ~(err <= tol)
    assert not bad.any(), _report(name, got, ref, err, tol, bad)
    return float(np.max(err / scale))
