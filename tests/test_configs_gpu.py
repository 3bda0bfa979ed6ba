"""Five workloads at their full sizes, plus the fused forward at the
(576000, 384) benchmark shape, on the GPU against the oracle:

  - LayerNorm fwd, fp32, 64 x 384, bias + residual + gamma + beta, eps 1e-5
  - fused bias + residual + LayerNorm fwd, bf16, 4096 x 384, residual_out, amax
  - RMSNorm bwd, bf16, 576000 x 384, rstd recomputed (eps 1e-6), dgamma cast to bf16
  - LayerNorm bwd, bf16, 576000 x 384, fp32 saved mean / rstd, dgamma, dbeta
  - residual + LayerNorm fwd then bwd, bf16, 8192 x 4096, 1% of x / residual /
     dy elements scaled by 100
At 576000 rows dx is compared on sampled rows (the oracle computes those
rows one by one); the column sums and amax are compared in full.  The kernel
configuration is the one the benchmark times.
"""
import numpy as np
import pytest
import torch

import normalization_ln_fwd_amd as nf
import oracle
import synth
from gpu_util import BF16, F32, f64, from_dev, require_gpu, to_dev
from test_fwd_gpu import check_fwd, run_fwd
from tolerance import (assert_colsums_close, assert_fused_add_close, assert_rows_close,
                       dx_term_scale)

pytestmark = pytest.mark.gpu

BIG_M = 1152 * 500
# bound for the column sums at M = 576000 (relative error 1e-3), relative
# to max(|sum|, ||terms||_2); the observed error is printed
COLSUM_REL_BIG = 1e-3


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def sample_rows(M, seed=0, n_random=4096, edge=2048):
    rng = np.random.default_rng(seed)
    rows = np.concatenate([np.arange(min(edge, M)), np.arange(max(0, M - edge), M),
                           rng.integers(0, M, n_random)])
    return np.unique(rows)


def test_ln_fwd_fp32_64x384():
    M, N = 64, 384
    inp = synth.make_inputs(M, N, dtype=F32, seed=0)
    out = run_fwd(False, inp, F32, 1e-5, want_amax=False)
    check_fwd(False, inp, F32, 1e-5, out)


def test_fused_ln_fwd_bf16_amax_4096x384():
    M, N = 4096, 384
    inp = synth.make_inputs(M, N, dtype=BF16, seed=0)
    out = run_fwd(False, inp, BF16, 1e-5, want_amax=True)
    check_fwd(False, inp, BF16, 1e-5, out)


def _big_bwd(rms):
    M, N = BIG_M, 384
    names = ("x", "dy", "gamma")
    inp = synth.make_inputs(M, N, dtype=BF16, seed=0, names=names)
    eps = 1e-6 if rms else 1e-5
    mean = rstd = None
    if not rms:
        f = oracle.norm_fwd(inp["x"], eps=eps, dtype=BF16, want_u=False, want_y=False)
        mean, rstd = f["mean"].astype(np.float32), f["rstd"].astype(np.float32)
    dy, x, g = (to_dev(inp[k], BF16) for k in ("dy", "x", "gamma"))
    outs = {}
    for pdt in (torch.float32, torch.bfloat16):
        if rms:
            outs[pdt] = nf.rms_bwd(dy, x, g, None, eps, dparam_dtype=pdt, want_dbias=True)
        else:
            outs[pdt] = nf.ln_bwd(dy, x, g, torch.from_numpy(mean).cuda(),
                                  torch.from_numpy(rstd).cuda(), dparam_dtype=pdt,
                                  want_dbias=True)
    torch.cuda.synchronize()
    # column sums over every row (dbias: the backward of a fused bias add,
    # asked for alongside)
    ref = oracle.norm_bwd(inp["dy"], inp["x"], inp["gamma"], mean, rstd if not rms else None,
                          eps, rms=rms, dtype=BF16, want_dx=False, want_dbias=True)
    keys = ("dgamma", "dbias") if rms else ("dgamma", "dbeta", "dbias")
    for k in keys:
        e32 = assert_colsums_close(f64(outs[torch.float32][k]), ref[k], ref[k + "_l2"],
                                   COLSUM_REL_BIG, k)
        print(f"{k}: max err / max(|ref|, l2) = {e32:.3e}")
        assert_colsums_close(f64(outs[torch.bfloat16][k]), ref[k], ref[k + "_l2"],
                             COLSUM_REL_BIG, k + " (bf16)", dtype=BF16)
        assert torch.equal(outs[torch.bfloat16][k], outs[torch.float32][k].to(torch.bfloat16))
    # dx on sampled rows
    rows = sample_rows(M)
    rs = oracle.norm_bwd(inp["dy"][rows], inp["x"][rows], inp["gamma"],
                         None if rms else mean[rows], None if rms else rstd[rows], eps,
                         rms=rms, dtype=BF16, want_params=False)
    dx = outs[torch.float32]["dx"][torch.from_numpy(rows).cuda()]
    assert_rows_close(f64(dx), rs["dx"], BF16, "dx (sampled rows)",
                      scale=dx_term_scale(inp["dy"][rows], inp["gamma"], rs["rstd"], BF16))
    # the row invariant of LayerNorm's dx holds at every row: sum_j dx_j ~ 0
    if not rms:
        dxall = outs[torch.float32]["dx"].float()
        rowsum = dxall.sum(dim=1).abs()
        rowscale = dxall.abs().amax(dim=1).clamp_min(1e-30)
        assert float((rowsum / rowscale).max()) < 384 * 2.0 ** -8


def test_rms_bwd_recompute_576000x384():
    _big_bwd(rms=True)


def test_ln_bwd_576000x384():
    _big_bwd(rms=False)


def test_fused_ln_fwd_576k_amax():
    """The forward at the benchmark shape: sampled rows against the oracle,
    amax against the brute-force max over all of y."""
    M, N = BIG_M, 384
    inp = synth.make_inputs(M, N, dtype=BF16, seed=0)
    out = run_fwd(False, inp, BF16, 1e-5, want_amax=True)
    y = out["y"]
    brute = float(y.float().abs().max().item())
    assert float(out["amax"].item()) == brute
    rows = sample_rows(M, seed=1)
    sub = {k: (inp[k][rows] if k in ("x", "residual") else inp[k]) for k in inp}
    ref = oracle.norm_fwd(sub["x"], sub["bias"], sub["residual"], sub["gamma"], sub["beta"], 1e-5)
    ridx = torch.from_numpy(rows).cuda()
    u_gpu = from_dev(out["residual_out"][ridx], BF16)
    assert_fused_add_close(u_gpu, ref["u"], sub, BF16, "residual_out (sampled)")
    st = oracle.norm_fwd(u_gpu, None, None, sub["gamma"], sub["beta"], 1e-5)
    assert_rows_close(f64(y[ridx]), st["y"], BF16, "y (sampled rows)")
    rel = np.abs(f64(out["rstd"][ridx]) - st["rstd"]) / st["rstd"]
    assert rel.max() <= 1e-5


def test_ln_fwd_then_bwd_outliers_8192x4096():
    M, N = 8192, 4096
    inp = synth.make_inputs(M, N, dtype=BF16, seed=0, outlier_p=0.01,
                            names=("x", "residual", "gamma", "beta", "dy"))
    parts = ("x", "residual", "gamma", "beta")
    out = run_fwd(False, inp, BF16, 1e-5, want_amax=True, parts=parts)
    check_fwd(False, inp, BF16, 1e-5, out, parts=parts)
    # backward of the GPU forward: x = residual_out, the GPU's mean / rstd
    x_gpu = out["residual_out"]
    dy = to_dev(inp["dy"], BF16)
    g = to_dev(inp["gamma"], BF16)
    b = nf.ln_bwd(dy, x_gpu, g, out["mean"], out["rstd"], dparam_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.norm_bwd(inp["dy"], from_dev(x_gpu, BF16), inp["gamma"],
                          f64(out["mean"]), f64(out["rstd"]), 1e-5, dtype=BF16)
    assert_rows_close(f64(b["dx"]), ref["dx"], BF16, "dx",
                      scale=dx_term_scale(inp["dy"], inp["gamma"], ref["rstd"], BF16))
    for k in ("dgamma", "dbeta"):
        e = assert_colsums_close(f64(b[k]), ref[k], ref[k + "_l2"], 1e-5, k)
        print(f"{k}: max err / max(|ref|, l2) = {e:.3e}")
