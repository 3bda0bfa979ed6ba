"""Seeded synthetic inputs for the fused LayerNorm / RMSNorm workloads.

Shared by the tests and the benchmark; holds none of the normalisation
arithmetic.  The pages' workloads (a miniLM encoder in IREE issue #9139 and
"some internal model" at (1152 * 500, 384) in PyTorch PR #165370) are not
available, so Gaussian tensors of those shapes stand in for them.

Recipe (every config):
  * each tensor has its own numpy PCG64 stream, seeded from (seed, tensor id),
    so a tensor never depends on which other tensors a config draws, and the
    first R rows of an M-row tensor are the same for every M >= R;
  * values are ``standard_normal`` float32 draws, row-major;
    x, residual, dy ~ N(0, 1); bias, beta ~ N(0, 0.1) (std 0.1);
    gamma ~ 1 + N(0, 0.1);
  * optional outlier stress: an independent Bernoulli(p) mask per element of
    x / residual / dy scales the element by ``outlier_scale`` (in float32);
  * bf16 tensors are the float32 values rounded to nearest, ties to even, by
    bit manipulation, returned as uint16 bit patterns.
"""
import numpy as np

F32 = 0
BF16 = 1

# Stable ids, one per tensor role, mixed into the seed.
_TENSOR_IDS = {"x": 1, "residual": 2, "bias": 3, "gamma": 4, "beta": 5, "dy": 6,
               "x_mask": 11, "residual_mask": 12, "dy_mask": 16}
_CHUNK_ROWS = 4096


def _rng(seed, name):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _TENSOR_IDS[name]])))


def f32_to_bf16_bits(a):
    """Round float32 values to bf16 (nearest, ties to even); uint16 patterns.
    Inputs here are finite; NaN is not produced by the generators."""
    a = np.ascontiguousarray(a, np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    b = np.ascontiguousarray(b, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _normal(seed, name, rows, cols):
    """float32 N(0,1) [rows, cols], drawn row-major in 4096-row chunks."""
    g = _rng(seed, name)
    out = np.empty((rows, cols), np.float32)
    for r0 in range(0, rows, _CHUNK_ROWS):
        r1 = min(rows, r0 + _CHUNK_ROWS)
        out[r0:r1] = g.standard_normal((r1 - r0, cols), dtype=np.float32)
    return out


def _with_outliers(a, seed, name, p, scale):
    if p <= 0.0:
        return a
    g = _rng(seed, name + "_mask")
    for r0 in range(0, a.shape[0], _CHUNK_ROWS):
        r1 = min(a.shape[0], r0 + _CHUNK_ROWS)
        m = g.random((r1 - r0, a.shape[1]), dtype=np.float32) < np.float32(p)
        a[r0:r1][m] *= np.float32(scale)
    return a


def _cast(a, dtype):
    return f32_to_bf16_bits(a) if dtype == BF16 else np.ascontiguousarray(a, np.float32)


def make_inputs(M, N, *, dtype=BF16, seed=0, names=("x", "residual", "bias", "gamma", "beta"),
                outlier_p=0.0, outlier_scale=100.0):
    """Dict of host arrays (uint16 bf16 patterns or float32) for the given
    tensor roles.  [M, N] roles: x, residual, dy; [N] roles: bias, gamma, beta."""
    out = {}
    for name in names:
        if name in ("x", "residual", "dy"):
            a = _normal(seed, name, M, N)
            a = _with_outliers(a, seed, name, outlier_p, outlier_scale)
        elif name in ("bias", "beta"):
            a = np.float32(0.1) * _normal(seed, name, 1, N)[0]
        elif name == "gamma":
            a = np.float32(1.0) + np.float32(0.1) * _normal(seed, name, 1, N)[0]
        else:
            raise KeyError(name)
        out[name] = _cast(a, dtype)
    return out


def to_f64(a, dtype):
    """Exact float64 value of a generator array."""
    return (bf16_bits_to_f32(a) if dtype == BF16 else np.asarray(a, np.float32)).astype(np.float64)
