"""The largest sizes: tensors past 4 GiB (64-bit addressing of row groups)
and the longest rows (N = NORM_N_MAX), against the oracle.

M = 6,000,000 rows of 384 bf16 elements is 4.6 GB per tensor; the forward
runs on it end to end (y and residual_out on sampled rows, amax over all of
y) and the backward's column sums over every row are compared with the
oracle's, at the 1e-3 bar of the 576000-row workloads."""
import numpy as np
import pytest
import torch

import normalization_ln_fwd_amd as nf
import oracle
import synth
from gpu_util import BF16, f64, from_dev, require_gpu
from tolerance import assert_colsums_close, assert_fused_add_close, assert_rows_close

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def dev_randn(shape, seed, scale=1.0, shift=0.0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return (torch.randn(shape, device="cuda", generator=g) * scale + shift).to(torch.bfloat16)


def bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def test_forward_and_backward_past_4gib():
    M, N = 6_000_000, 384
    x, res, dy = dev_randn((M, N), 1), dev_randn((M, N), 2), dev_randn((M, N), 3)
    bias, beta = dev_randn((N,), 4, 0.1), dev_randn((N,), 5, 0.1)
    gamma = dev_randn((N,), 6, 0.1, 1.0)
    assert x.numel() * x.element_size() > 4 << 30
    out = nf.ln_fwd(x, bias, res, gamma, beta, 1e-5, want_amax=True)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 2**21 + 5, M // 2, 5_592_405, M - 2, M - 1])
    ridx = torch.from_numpy(rows).cuda()
    sub = {"x": bits(x[ridx]), "residual": bits(res[ridx]), "bias": bits(bias),
           "gamma": bits(gamma), "beta": bits(beta)}
    ref = oracle.norm_fwd(sub["x"], sub["bias"], sub["residual"], sub["gamma"], sub["beta"], 1e-5)
    u_gpu = from_dev(out["residual_out"][ridx], BF16)
    assert_fused_add_close(u_gpu, ref["u"], sub, BF16, "residual_out (sampled)")
    st = oracle.norm_fwd(u_gpu, None, None, sub["gamma"], sub["beta"], 1e-5)
    assert_rows_close(f64(out["y"][ridx]), st["y"], BF16, "y (sampled)")
    assert float(out["amax"].item()) == float(out["y"].abs().max().float().item())

    del res
    b = nf.ln_bwd(dy, out["residual_out"], gamma, out["mean"], out["rstd"],
                  dparam_dtype=torch.float32, want_dbias=True)
    torch.cuda.synchronize()
    ref_b = oracle.norm_bwd(bits(dy[ridx]), u_gpu, sub["gamma"],
                            out["mean"][ridx].cpu().numpy(), out["rstd"][ridx].cpu().numpy(),
                            1e-5, want_params=False)
    assert_rows_close(f64(b["dx"][ridx]), ref_b["dx"], BF16, "dx (sampled)", ulps=1.0,
                      scale=ref_b["rstd"] * np.max(np.abs(synth.to_f64(bits(dy[ridx]), BF16)
                                                          * synth.to_f64(sub["gamma"], BF16)),
                                                   axis=1))
    # column sums over every row against the oracle (its column sums only),
    # on the same dy, residual_out, gamma and the GPU forward's fp32 mean / rstd
    dy_h = bits(dy)
    del dy
    u_h = bits(out["residual_out"])
    mean_h, rstd_h = out["mean"].cpu().numpy(), out["rstd"].cpu().numpy()
    ref_c = oracle.norm_bwd(dy_h, u_h, sub["gamma"], mean_h, rstd_h, 1e-5, want_dx=False)
    del dy_h, u_h
    for k in ("dgamma", "dbeta"):
        e = assert_colsums_close(f64(b[k]), ref_c[k], ref_c[k + "_l2"], 1e-3, k + " (all rows)")
        print(f"{k} over {M} rows: max |err| / max(|ref|, l2) = {e:.3e}")


@pytest.mark.parametrize("rms", [False, True], ids=["ln", "rms"])
def test_longest_rows(rms):
    M, N = 700, nf.N_MAX
    inp = synth.make_inputs(M, N, dtype=BF16, seed=9, names=("x", "residual", "gamma", "beta",
                                                             "dy"))
    d = {k: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda() for k, v in inp.items()}
    fn = nf.rms_fwd if rms else nf.ln_fwd
    out = fn(d["x"], None, d["residual"], d["gamma"], d["beta"], 1e-5, want_amax=True)
    torch.cuda.synchronize()
    ref = oracle.norm_fwd(inp["x"], None, inp["residual"], inp["gamma"], inp["beta"], 1e-5,
                          rms=rms)
    assert_rows_close(f64(out["y"]), ref["y"], BF16, "y", ulps=2.0)
    bwd = nf.rms_bwd if rms else nf.ln_bwd
    args = (d["dy"], out["residual_out"], d["gamma"]) + \
        ((out["rstd"], 1e-5) if rms else (out["mean"], out["rstd"]))
    b = bwd(*args, dparam_dtype=torch.float32)
    torch.cuda.synchronize()
    u = from_dev(out["residual_out"], BF16)
    rb = oracle.norm_bwd(inp["dy"], u, inp["gamma"], None if rms else out["mean"].cpu().numpy(),
                         out["rstd"].cpu().numpy(), 1e-5, rms=rms)
    assert_colsums_close(f64(b["dgamma"]), rb["dgamma"], rb["dgamma_l2"], 1e-5, "dgamma")
