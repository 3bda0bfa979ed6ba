"""Five workloads at their full sizes, plus the fused forward at the
(576000, 384) benchmark shape, on the GPU against the oracle:

  - LayerNorm fwd, fp32, 64 x 384, bias + residual + gamma + beta, eps 1e-5
  - fused bias + residual + LayerNorm fwd, bf16, 4096 x 384, residual_out, amax
  - RMSNorm bwd, bf16, 576000 x 384, rstd recomputed (eps 1e-6), dgamma cast to bf16
  - LayerNorm bwd, bf16, 576000 x 384, fp32 saved mean / rstd, dgamma, dbeta
  - residual + LayerNorm fwd then bwd, bf16, 8192 x 4096, 1% of x / residual /
     dy elements scaled by 100
Every row is compared at every size (dx, y, residual_out at 576000 rows in
chunks of rows, against the oracle run on the same chunk); the column sums
and amax in full.  The kernel configurations are the ones the benchmark
times: the backward at 576000 x 384 runs both with dbias (one instantiation)
and without (the one the benchmark's configs 3 and 4 take).
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


CHUNK = 65536  # rows per comparison chunk (bounds host memory)


def colsum_report(name, got, ref, l2):
    """The scaled error the bar is set on, and the plain per-element relative
    error |got - ref| / |ref| next to it (ill-posed where a zero-mean column
    sum lands near 0, hence not the bar)."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    scaled = np.abs(got - ref) / np.maximum(np.maximum(np.abs(ref), l2), 1e-300)
    plain = np.abs(got - ref) / np.maximum(np.abs(ref), 1e-300)
    print(f"{name}: max |err| / max(|ref|, l2) = {scaled.max():.3e}; plain relative error "
          f"max {plain.max():.3e}, median {np.median(plain):.3e}")


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
    # fp32 parameter gradients with dbias (the backward of a fused bias add,
    # asked for alongside: one kernel instantiation); bf16 ones without
    # dbias (the instantiation the configs as specified take)
    outs = {}
    for pdt, db in ((torch.float32, True), (torch.bfloat16, False)):
        if rms:
            outs[pdt] = nf.rms_bwd(dy, x, g, None, eps, dparam_dtype=pdt, want_dbias=db)
        else:
            outs[pdt] = nf.ln_bwd(dy, x, g, torch.from_numpy(mean).cuda(),
                                  torch.from_numpy(rstd).cuda(), dparam_dtype=pdt,
                                  want_dbias=db)
    torch.cuda.synchronize()
    assert outs[torch.bfloat16]["dbias"] is None
    # column sums over every row
    ref = oracle.norm_bwd(inp["dy"], inp["x"], inp["gamma"], mean, rstd if not rms else None,
                          eps, rms=rms, dtype=BF16, want_dx=False, want_dbias=True)
    keys = ("dgamma",) if rms else ("dgamma", "dbeta")
    for k in keys + ("dbias",):
        assert_colsums_close(f64(outs[torch.float32][k]), ref[k], ref[k + "_l2"],
                             COLSUM_REL_BIG, k)
        colsum_report(k, f64(outs[torch.float32][k]), ref[k], ref[k + "_l2"])
    for k in keys:
        assert_colsums_close(f64(outs[torch.bfloat16][k]), ref[k], ref[k + "_l2"],
                             COLSUM_REL_BIG, k + " (bf16)", dtype=BF16)
        # with or without dbias the dgamma / dbeta sums are the same: the bf16
        # result is the fp32 one rounded to nearest even
        assert torch.equal(outs[torch.bfloat16][k], outs[torch.float32][k].to(torch.bfloat16))
    # dx of every row, in chunks, for both instantiations
    worst = 0.0
    for r0 in range(0, M, CHUNK):
        r1 = min(M, r0 + CHUNK)
        rs = oracle.norm_bwd(inp["dy"][r0:r1], inp["x"][r0:r1], inp["gamma"],
                             None if rms else mean[r0:r1], None if rms else rstd[r0:r1], eps,
                             rms=rms, dtype=BF16, want_params=False)
        scale = dx_term_scale(inp["dy"][r0:r1], inp["gamma"], rs["rstd"], BF16)
        for pdt in outs:
            e = assert_rows_close(f64(outs[pdt]["dx"][r0:r1]), rs["dx"], BF16,
                                  f"dx rows {r0}..{r1} ({pdt})", scale=scale)
            worst = max(worst, e)
    print(f"dx: all {M} rows within tolerance (max err / tol = {worst:.3f})")


def test_rms_bwd_recompute_576000x384():
    _big_bwd(rms=True)


def test_ln_bwd_576000x384():
    _big_bwd(rms=False)


def check_big_fwd(rms, inp, out, eps):
    """Every row of a large forward against the oracle, in chunks, staged as
    in the small sweeps: residual_out against the exact sum, y / mean / rstd
    against the oracle run on the GPU's residual_out; amax bit-exact against
    the brute-force max over all of y."""
    M = inp["x"].shape[0]
    y = out["y"]
    brute = float(y.float().abs().max().item())
    assert float(out["amax"].item()) == brute
    for r0 in range(0, M, CHUNK):
        r1 = min(M, r0 + CHUNK)
        sub = {k: (inp[k][r0:r1] if k in ("x", "residual") else inp[k]) for k in inp}
        ref = oracle.norm_fwd(sub["x"], sub["bias"], sub["residual"], sub["gamma"],
                              sub["beta"], eps, rms=rms)
        u_gpu = from_dev(out["residual_out"][r0:r1], BF16)
        assert_fused_add_close(u_gpu, ref["u"], sub, BF16, f"residual_out rows {r0}..{r1}")
        st = oracle.norm_fwd(u_gpu, None, None, sub["gamma"], sub["beta"], eps, rms=rms)
        assert_rows_close(f64(y[r0:r1]), st["y"], BF16, f"y rows {r0}..{r1}")
        rel = np.abs(f64(out["rstd"][r0:r1]) - st["rstd"]) / st["rstd"]
        assert rel.max() <= 1e-5, f"rstd rows {r0}..{r1}: {rel.max():.3e}"
        if not rms:
            s = np.maximum(np.max(np.abs(synth.to_f64(u_gpu, BF16)), axis=1), 1e-30)
            assert np.all(np.abs(f64(out["mean"][r0:r1]) - st["mean"]) <= 1e-5 * s), "mean"


def test_fused_ln_fwd_576k_amax():
    """The forward at the benchmark shape (its 512-thread instantiation),
    every row against the oracle."""
    M, N = BIG_M, 384
    inp = synth.make_inputs(M, N, dtype=BF16, seed=0)
    out = run_fwd(False, inp, BF16, 1e-5, want_amax=True)
    check_big_fwd(False, inp, out, 1e-5)


def test_fused_rms_fwd_576k_amax():
    """RMSNorm forward at the benchmark shape, as the benchmark runs it (no
    beta), every row against the oracle."""
    M, N = BIG_M, 384
    inp = synth.make_inputs(M, N, dtype=BF16, seed=2)
    inp["beta"] = None
    out = run_fwd(True, inp, BF16, 1e-6, want_amax=True, parts=("x", "bias", "residual", "gamma"))
    check_big_fwd(True, inp, out, 1e-6)


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
