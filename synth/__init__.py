"""Seeded synthetic inputs for the fused LayerNorm / RMSNorm workloads.

Shared by the tests and the benchmark; holds none of the normalisation
arithmetic.  The pages' workloads (a miniLM encoder in IREE issue #9139 and
"some internal model" at (1152 * 500, 384) in PyTorch PR #165370) are not
available, so Gaussian tensors of those shapes stand in for them.

Recipe (every config):
  * every tensor is drawn in 4096-row chunks; chunk c of a tensor has its own
    numpy PCG64 stream seeded from (seed, tensor id, c), so a tensor never
    depends on which other tensors a config draws, and the first R rows of an
    M-row tensor are the same for every M >= R;
  * values are ``standard_normal`` float32 draws, row-major;
    x, residual, dy ~ N(0, 1); bias, beta ~ N(0, 0.1) (std 0.1);
    gamma ~ 1 + N(0, 0.1);
  * optional outlier stress: an independent Bernoulli(p) mask per element of
    x / residual / dy scales the element by ``outlier_scale`` (in float32);
  * bf16 tensors are the float32 values rounded to nearest, ties to even, by
    bit manipulation, returned as uint16 bit patterns.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

F32 = 0
BF16 = 1

# Stable ids, one per tensor role, mixed into the seed.
_TENSOR_IDS = {"x": 1, "residual": 2, "bias": 3, "gamma": 4, "beta": 5, "dy": 6,
               "x_mask": 11, "residual_mask": 12, "dy_mask": 16}
_CHUNK_ROWS = 4096


def _rng(seed, name, chunk=0):
    ss = np.random.SeedSequence([seed, _TENSOR_IDS[name], chunk])
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(a):
    """Round float32 values to bf16 (nearest, ties to even); uint16 patterns.
    Inputs here are finite, so the 32-bit sum below cannot wrap."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF)
    r += (u >> np.uint32(16)) & np.uint32(1)
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    b = np.ascontiguousarray(b, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _cast(a, dtype):
    return f32_to_bf16_bits(a) if dtype == BF16 else np.ascontiguousarray(a, np.float32)


def _matrix(seed, name, rows, cols, dtype, outlier_p, outlier_scale):
    """[rows, cols] N(0,1) draws, row-major; rows come in 4096-row chunks,
    chunk c drawn from its own stream (seed, tensor, c), then the optional
    outliers, then the cast to the I/O dtype.  Chunks fill in parallel."""
    out = np.empty((rows, cols), np.uint16 if dtype == BF16 else np.float32)

    def fill(c):
        r0 = c * _CHUNK_ROWS
        r1 = min(rows, r0 + _CHUNK_ROWS)
        a = _rng(seed, name, c).standard_normal((r1 - r0, cols), dtype=np.float32)
        if outlier_p > 0.0:
            u = _rng(seed, name + "_mask", c).random((r1 - r0, cols), dtype=np.float32)
            a[u < np.float32(outlier_p)] *= np.float32(outlier_scale)
        out[r0:r1] = _cast(a, dtype)

    n_chunks = (rows + _CHUNK_ROWS - 1) // _CHUNK_ROWS
    workers = max(1, min(16, len(os.sched_getaffinity(0)), n_chunks))
    if workers == 1:
        for c in range(n_chunks):
            fill(c)
    else:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out


def _vector(seed, name, cols):
    return _rng(seed, name).standard_normal((1, cols), dtype=np.float32)[0]


def make_inputs(M, N, *, dtype=BF16, seed=0, names=("x", "residual", "bias", "gamma", "beta"),
                outlier_p=0.0, outlier_scale=100.0):
    """Dict of host arrays (uint16 bf16 patterns or float32) for the given
    tensor roles.  [M, N] roles: x, residual, dy; [N] roles: bias, gamma, beta."""
    out = {}
    for name in names:
        if name in ("x", "residual", "dy"):
            out[name] = _matrix(seed, name, M, N, dtype, outlier_p, outlier_scale)
        elif name in ("bias", "beta"):
            out[name] = _cast(np.float32(0.1) * _vector(seed, name, N), dtype)
        elif name == "gamma":
            out[name] = _cast(np.float32(1.0) + np.float32(0.1) * _vector(seed, name, N), dtype)
        else:
            raise KeyError(name)
    return out


def to_f64(a, dtype):
    """Exact float64 value of a generator array."""
    return (bf16_bits_to_f32(a) if dtype == BF16 else np.asarray(a, np.float32)).astype(np.float64)
