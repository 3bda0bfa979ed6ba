"""GPU parity of the row softmax (softmax_fwd) against the oracle: sizes
spanning several workgroups with ragged tails, both dtypes, the 16-byte and
element-wise kernels, and rows the definition fixes (constant rows, large
offsets, one dominant element)."""
import numpy as np
import pytest
import torch

import normalization_ln_fwd_amd as nf
import oracle
import synth
from gpu_util import BF16, F32, f64, require_gpu, to_dev
from tolerance import assert_rows_close

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1), (3, 7), (37, 8), (130, 64), (257, 100), (300, 384), (77, 520), (64, 1000),
          (33, 1024), (17, 1536), (9, 2000), (43, 4096), (5, 5000), (3, 16384), (2, 16383),
          (5000, 384), (21, 2560), (13, 1200), (45, 1002), (19, 4100),
          (5, 2), (6, 4), (7, 6), (6, 8192), (4, 6152), (1000, 3072), (700, 2304), (900, 1280)]


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("M,N", SHAPES)
@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("misalign", [False, True], ids=["vec", "elem"])
def test_softmax_matches_oracle(M, N, dtype, misalign):
    x = synth.make_inputs(M, N, dtype=dtype, seed=M * 3 + N, names=("x",))["x"]
    y = nf.softmax_fwd(to_dev(x, dtype, misalign))
    torch.cuda.synchronize()
    ref = oracle.softmax_fwd(x, dtype=dtype)
    assert_rows_close(f64(y), ref, dtype, "softmax")
    if M * N:
        rs = f64(y).sum(1)
        assert np.all(np.abs(rs - 1.0) <= N * (2.0**-8 if dtype == BF16 else 2.0**-22))


@pytest.mark.parametrize("M,N,dtype", [(100003, 384, BF16), (40001, 384, F32)])
def test_softmax_512_thread_workgroups_match_oracle(M, N, dtype):
    """Row counts that take the 512-thread variant of the narrow shape (the
    instantiation the benchmark's 576000-row softmax runs), ragged tail."""
    x = synth.make_inputs(M, N, dtype=dtype, seed=M + 1, names=("x",))["x"]
    y = nf.softmax_fwd(to_dev(x, dtype))
    torch.cuda.synchronize()
    assert_rows_close(f64(y), oracle.softmax_fwd(x, dtype=dtype), dtype, "softmax")


def test_softmax_special_rows():
    N = 384
    x = np.zeros((4, N), np.float32)
    x[0] = -7.25                                   # constant: 1/N
    x[1] = 1000.0 + np.linspace(-3, 3, N)          # large offset
    x[2] = -1000.0 + np.linspace(-3, 3, N)
    x[3] = 0.0
    x[3, 17] = 80.0                                # one dominant element
    y = nf.softmax_fwd(to_dev(x, F32))
    torch.cuda.synchronize()
    ref = oracle.softmax_fwd(x, dtype=F32)
    assert_rows_close(f64(y), ref, F32, "softmax special rows")
    assert np.all(np.isfinite(f64(y)))


def test_softmax_empty_and_rejects():
    y = nf.softmax_fwd(torch.empty((0, 384), dtype=torch.bfloat16, device="cuda"))
    assert y.shape == (0, 384)
    with pytest.raises(nf.NormError) as e:
        nf.softmax_fwd(torch.empty((4, 16385), dtype=torch.bfloat16, device="cuda"))
    assert e.value.status == 2
