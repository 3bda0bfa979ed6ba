"""GPU parity of the variants: zero-centred gamma (forward and backward) and
the mean epilogue of the backward's column reductions.

Each variant is checked against the oracle run with the same option, and
against the plain entry point in the form the option is defined by: a
zero-centred gamma behaves exactly as the weight 1 + gamma rounded to the I/O
dtype passed as an ordinary gamma, and the mean is the fp32 column sum
divided by M.
"""
import numpy as np
import pytest
import torch

import normalization_ln_fwd_amd as nf
import oracle
import synth
from gpu_util import BF16, F32, TORCH_DT, f64, from_dev, require_gpu, to_dev
from tolerance import (assert_colsums_close, assert_fused_add_close, assert_rows_close,
                       dbias_term_l2, dx_term_scale)

pytestmark = pytest.mark.gpu

SHAPES = [(3, 7), (130, 64), (300, 384), (77, 520), (33, 1024), (17, 1536), (43, 4096),
          (5, 5000), (3, 16384), (45, 1002), (19, 4100), (21, 2560)]
# the forward's 512-thread workgroups (bf16 rows of 384 from 65505 rows on,
# fp32 from 32753)
FWD_SHAPES = SHAPES + [(100003, 384)]


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def zc_gamma(N, dtype, seed):
    """A zero-centred weight, ~ 0.1 * N(0, 1), and the ordinary weight
    1 + gamma it stands for, rounded to the I/O dtype."""
    g = synth.make_inputs(1, N, dtype=dtype, seed=seed, names=("beta",))["beta"]
    w = (to_dev(g, dtype).float() + 1.0).to(TORCH_DT[dtype])
    return g, w


@pytest.mark.parametrize("M,N", FWD_SHAPES)
@pytest.mark.parametrize("rms", [False, True], ids=["ln", "rms"])
@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("misalign", [False, True], ids=["vec", "elem"])
def test_zero_centered_gamma_forward(M, N, rms, dtype, misalign):
    inp = synth.make_inputs(M, N, dtype=dtype, seed=M * 13 + N)
    g, w = zc_gamma(N, dtype, seed=N)
    eps = 1e-6 if rms else 1e-5
    dev = {k: to_dev(inp[k], dtype, misalign and k == "x")
           for k in ("x", "bias", "residual", "beta")}
    fn = nf.rms_fwd if rms else nf.ln_fwd
    out = fn(dev["x"], dev["bias"], dev["residual"], to_dev(g, dtype), dev["beta"], eps,
             want_amax=True, zero_centered_gamma=True)
    plain = fn(dev["x"], dev["bias"], dev["residual"], w, dev["beta"], eps, want_amax=True)
    torch.cuda.synchronize()
    for k in ("y", "residual_out", "rstd", "amax") + (() if rms else ("mean",)):
        assert torch.equal(out[k], plain[k]), k
    ref = oracle.norm_fwd(inp["x"], inp["bias"], inp["residual"], g, inp["beta"], eps, rms=rms,
                          dtype=dtype, zero_centered_gamma=True)
    u_gpu = from_dev(out["residual_out"], dtype)
    assert_fused_add_close(u_gpu, ref["u"], inp, dtype, "residual_out")
    st = oracle.norm_fwd(u_gpu, None, None, g, inp["beta"], eps, rms=rms, dtype=dtype,
                         zero_centered_gamma=True)
    assert_rows_close(f64(out["y"]), st["y"], dtype, "y (staged)")


@pytest.mark.parametrize("M,N", SHAPES)
@pytest.mark.parametrize("rms", [False, True], ids=["ln", "rms"])
@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "f32"])
def test_zero_centered_gamma_backward(M, N, rms, dtype):
    inp = synth.make_inputs(M, N, dtype=dtype, seed=M * 17 + N, names=("x", "dy"))
    g, w = zc_gamma(N, dtype, seed=N + 1)
    eps = 1e-6 if rms else 1e-5
    f = oracle.norm_fwd(inp["x"], gamma=g, eps=eps, rms=rms, dtype=dtype, want_u=False,
                        want_y=False, zero_centered_gamma=True)
    mean = torch.from_numpy(f["mean"].astype(np.float32)).cuda()
    rstd = torch.from_numpy(f["rstd"].astype(np.float32)).cuda()
    dy, x, gd = to_dev(inp["dy"], dtype), to_dev(inp["x"], dtype), to_dev(g, dtype)
    if rms:
        out = nf.rms_bwd(dy, x, gd, rstd, eps, dparam_dtype=torch.float32, want_dbias=True,
                         zero_centered_gamma=True)
        plain = nf.rms_bwd(dy, x, w, rstd, eps, dparam_dtype=torch.float32, want_dbias=True)
    else:
        out = nf.ln_bwd(dy, x, gd, mean, rstd, dparam_dtype=torch.float32, want_dbias=True,
                        zero_centered_gamma=True)
        plain = nf.ln_bwd(dy, x, w, mean, rstd, dparam_dtype=torch.float32, want_dbias=True)
    torch.cuda.synchronize()
    for k in ("dx", "dgamma", "dbias") + (() if rms else ("dbeta",)):
        assert torch.equal(out[k], plain[k]), k
    ref = oracle.norm_bwd(inp["dy"], inp["x"], g, None if rms else f["mean"].astype(np.float32),
                          f["rstd"].astype(np.float32), eps, rms=rms, dtype=dtype,
                          want_dbias=True, zero_centered_gamma=True)
    wh = from_dev(w, dtype)
    assert_rows_close(f64(out["dx"]), ref["dx"], dtype, "dx",
                      scale=dx_term_scale(inp["dy"], wh, ref["rstd"], dtype))
    assert_colsums_close(f64(out["dgamma"]), ref["dgamma"], ref["dgamma_l2"], 1e-5, "dgamma")
    l2 = np.maximum(ref["dbias_l2"], dbias_term_l2(inp["dy"], wh, ref["rstd"], dtype))
    assert_colsums_close(f64(out["dbias"]), ref["dbias"], l2, 1e-5, "dbias")


@pytest.mark.parametrize("M,N", [(1, 8), (300, 384), (20000, 384), (301, 4096)])
@pytest.mark.parametrize("pdt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_dparam_mean_is_the_sum_over_m(M, N, pdt):
    inp = synth.make_inputs(M, N, dtype=BF16, seed=M + N, names=("x", "dy", "gamma"))
    f = oracle.norm_fwd(inp["x"], eps=1e-5, dtype=BF16, want_u=False, want_y=False)
    mean = torch.from_numpy(f["mean"].astype(np.float32)).cuda()
    rstd = torch.from_numpy(f["rstd"].astype(np.float32)).cuda()
    dy, x, g = to_dev(inp["dy"], BF16), to_dev(inp["x"], BF16), to_dev(inp["gamma"], BF16)
    m = nf.ln_bwd(dy, x, g, mean, rstd, dparam_dtype=pdt, want_dbias=True, dparam_mean=True)
    s = nf.ln_bwd(dy, x, g, mean, rstd, dparam_dtype=torch.float32, want_dbias=True)
    torch.cuda.synchronize()
    assert torch.equal(m["dx"], s["dx"])
    for k in ("dgamma", "dbeta", "dbias"):
        # correctly rounded fp32 division (numpy), then the down-cast
        want = torch.from_numpy(s[k].cpu().numpy() / np.float32(M)).to(pdt)
        assert torch.equal(m[k].cpu(), want), k
    if pdt == torch.float32:
        ref = oracle.norm_bwd(inp["dy"], inp["x"], inp["gamma"], f["mean"].astype(np.float32),
                              f["rstd"].astype(np.float32), 1e-5, want_dbias=True,
                              dparam_mean=True)
        for k in ("dgamma", "dbeta"):
            assert_colsums_close(f64(m[k]), ref[k], ref[k + "_l2"], 1e-5, k)


def test_dparam_mean_with_no_rows_is_zero():
    x = torch.empty((0, 384), dtype=torch.bfloat16, device="cuda")
    st = torch.empty((0,), dtype=torch.float32, device="cuda")
    out = nf.ln_bwd(x, x, None, st, st, dparam_dtype=torch.float32, dparam_mean=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out["dgamma"]) == 0 and torch.count_nonzero(out["dbeta"]) == 0
    assert not torch.isnan(out["dgamma"]).any()
