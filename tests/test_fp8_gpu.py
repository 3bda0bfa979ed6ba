"""GPU parity of the FP8 output (ln_fwd_fp8 / rms_fwd_fp8).

Staged like the forward tests.  The normalised y of the FP8 call is the one
ln_fwd / rms_fwd stores; those tests check it against the oracle, and here it
is also checked end to end.  The FP8 codes must then be exactly the oracle's
E4M3 quantisation of that stored y times the scale: the quantisation's
rounding decisions are taken on the same fp32 products on both sides.
residual_out, mean, rstd and amax must be bit-identical to the plain call's
when both take the same kernels (pointers in the same alignment class).
"""
import numpy as np
import pytest
import torch

import normalization_ln_fwd_amd as nf
import oracle
import synth
from gpu_util import BF16, F32, f64, require_gpu, to_dev
from tolerance import assert_rows_close

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1), (3, 7), (37, 8), (130, 64), (257, 100), (300, 384), (77, 520), (33, 1024),
          (17, 1536), (40, 4096), (43, 4096), (5, 5000), (3, 16384), (2, 16383), (21, 2560),
          (13, 1200), (45, 1002), (19, 4100),
          (5, 2), (6, 4), (7, 6),
          # teams of 640 and 768 lanes holding two vectors
          (7, 9216), (129, 10240), (5, 12288), (200, 6144),
          # one wave per row holding five vectors (taken from 2048 row groups on)
          (8198, 2312),
          # 1024-thread workgroups with the parameters staged in LDS
          (600, 16383), (300, 16382), (700, 8191)]


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def codes(t):
    return t.view(torch.uint8).cpu().numpy()


def run_pair(rms, inp, dtype, eps, scale, misalign=False, y8=None, plain_y=None):
    dev = {k: to_dev(inp[k], dtype, misalign and k == "x")
           for k in ("x", "bias", "residual", "gamma", "beta")}
    plain_fn, fp8_fn = (nf.rms_fwd, nf.rms_fwd_fp8) if rms else (nf.ln_fwd, nf.ln_fwd_fp8)
    sc = torch.tensor([scale], dtype=torch.float32, device="cuda")
    plain = plain_fn(dev["x"], dev["bias"], dev["residual"], dev["gamma"], dev["beta"], eps,
                     want_residual_out=True, want_amax=True,
                     out=None if plain_y is None else {"y": plain_y})
    out = None if y8 is None else {"y": y8}
    q = fp8_fn(dev["x"], sc, dev["bias"], dev["residual"], dev["gamma"], dev["beta"], eps,
               want_residual_out=True, want_amax=True, out=out)
    torch.cuda.synchronize()
    return plain, q


def check_pair(plain, q, scale, dtype, exact_y=None):
    for k in ("residual_out", "rstd", "amax") + (("mean",) if plain["mean"] is not None else ()):
        assert torch.equal(plain[k], q[k]), k
    y32 = plain["y"].float().cpu().numpy()
    ref = oracle.quantize_e4m3(y32, scale)
    got = codes(q["y"])
    bad = np.argwhere(got != ref)
    assert bad.size == 0, (f"{len(bad)} FP8 codes differ, first at {tuple(bad[0])}: "
                           f"got {got[tuple(bad[0])]:#04x} want {ref[tuple(bad[0])]:#04x}")
    if exact_y is not None:
        assert_rows_close(f64(plain["y"]), exact_y, dtype, "y (end to end)", ulps=2.0)


@pytest.mark.parametrize("M,N", SHAPES)
@pytest.mark.parametrize("rms", [False, True], ids=["ln", "rms"])
@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("misalign", [False, True], ids=["vec", "elem"])
def test_fp8_codes_are_the_quantised_stored_y(M, N, rms, dtype, misalign):
    inp = synth.make_inputs(M, N, dtype=dtype, seed=M * 101 + N)
    eps = 1e-6 if rms else 1e-5
    ref = oracle.norm_fwd(inp["x"], inp["bias"], inp["residual"], inp["gamma"], inp["beta"], eps,
                          rms=rms, dtype=dtype)
    scale = float(np.float32(448.0 / max(ref["amax"], 1e-30)))
    plain, q = run_pair(rms, inp, dtype, eps, scale, misalign)
    check_pair(plain, q, scale, dtype, exact_y=ref["y"])


@pytest.mark.parametrize("scale", [1.0, 0.03125, 37.0, 1e4])
def test_fp8_scales_and_saturation(scale):
    """Any scale; large ones saturate at +-448 (code 0x7E / 0xFE) instead of
    producing NaN."""
    inp = synth.make_inputs(500, 384, dtype=BF16, seed=3)
    plain, q = run_pair(False, inp, BF16, 1e-5, scale)
    check_pair(plain, q, scale, BF16)
    if scale >= 1e4:
        got = codes(q["y"])
        assert np.count_nonzero((got & 0x7F) == 0x7E) > got.size // 2
        assert np.count_nonzero((got & 0x7F) == 0x7F) == 0


def test_fp8_unaligned_output_takes_the_element_path():
    """An FP8 output off an 8-byte boundary leaves the vectorised kernels;
    compared with a plain call whose y is misaligned too (the same path)."""
    M, N = 64, 384
    inp = synth.make_inputs(M, N, dtype=BF16, seed=4)
    buf = torch.empty(M * N + 16, dtype=torch.uint8, device="cuda")
    y8 = buf[3:3 + M * N].view(M, N)
    ybuf = torch.empty(M * N + 8, dtype=torch.bfloat16, device="cuda")
    plain, q = run_pair(False, inp, BF16, 1e-5, 2.0, y8=y8,
                        plain_y=ybuf[1:1 + M * N].view(M, N))
    check_pair(plain, q, 2.0, BF16)


def test_fp8_empty_rows():
    x = torch.empty((0, 384), dtype=torch.bfloat16, device="cuda")
    amax = torch.full((1,), 5.0, device="cuda")
    out = nf.ln_fwd_fp8(x, None, want_amax=True, out={"amax": amax})
    torch.cuda.synchronize()
    assert out["amax"].item() == 0.0 and out["y"].shape == (0, 384)


def test_fp8_full_size_576000x384():
    """The benchmark shape: every code against the stored y's quantisation
    (torch's float8_e4m3fn cast of the clamped fp32 products, a library
    routine the oracle's quantiser is pinned to), sampled rows against the
    oracle's."""
    M, N = 576000, 384
    inp = synth.make_inputs(M, N, dtype=BF16, seed=0)
    dev = {k: to_dev(inp[k], BF16) for k in ("x", "bias", "residual", "gamma", "beta")}
    plain = nf.ln_fwd(dev["x"], dev["bias"], dev["residual"], dev["gamma"], dev["beta"], 1e-5,
                      want_amax=True)
    sc = (448.0 / plain["amax"]).to(torch.float32)
    q = nf.ln_fwd_fp8(dev["x"], sc, dev["bias"], dev["residual"], dev["gamma"], dev["beta"],
                      1e-5, want_amax=True)
    torch.cuda.synchronize()
    assert torch.equal(plain["amax"], q["amax"]) and torch.equal(plain["rstd"], q["rstd"])
    prod = (plain["y"].float() * sc).clamp(-448.0, 448.0)
    assert torch.equal(q["y"].view(torch.uint8), prod.to(torch.float8_e4m3fn).view(torch.uint8))
    rows = np.random.default_rng(5).choice(M, 512, replace=False)
    y32 = plain["y"][torch.from_numpy(rows).cuda()].float().cpu().numpy()
    ref = oracle.quantize_e4m3(y32, float(sc.item()))
    assert np.array_equal(codes(q["y"][torch.from_numpy(rows).cuda()]), ref)
