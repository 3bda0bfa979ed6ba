"""GPU parity of the mix-order backward (ln_bwd / rms_bwd) against the oracle.

Both sides consume the same inputs: dy, x, gamma, and for LayerNorm the
fp32 mean / rstd that the oracle forward produced (rounded to fp32), so the
comparison isolates the backward.  dx is checked row by row (one bf16 ulp or
1e-5 of the row scale), dgamma / dbeta against the oracle's exact column
sums relative to max(|sum|, ||terms||_2).
"""
import ctypes

import numpy as np
import pytest
import torch

import normalization_ln_fwd_amd as nf
import oracle
import synth
from gpu_util import BF16, F32, f64, from_dev, require_gpu, to_dev
from tolerance import assert_colsums_close, assert_rows_close, dbias_term_l2, dx_term_scale

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1), (3, 7), (37, 8), (130, 64), (257, 100), (300, 384), (77, 520), (64, 1000),
          (33, 1024), (17, 1536), (9, 2000), (40, 4096), (5, 5000), (3, 16384), (2, 16383),
          (2500, 384), (1100, 1024), (301, 4096), (93, 3000), (21, 2560), (11, 2304), (13, 1200),
          (9, 6000), (35, 4608),
          (45, 1002), (19, 4100), (7, 6002), (6, 12004), (301, 4100), (23, 6140), (70, 5004),
          (5, 2), (6, 4), (7, 6), (9, 12),
          # teams of 640 and 768 lanes holding two vectors
          (7, 9216), (5, 12288), (129, 10240), (200, 6144),
          # two teams of 320 lanes holding two vectors, several groups each
          (700, 4800),
          # the widest rows in 1024-thread workgroups (gamma and the dbias
          # sums in LDS), walking several row groups per workgroup
          (600, 16383), (300, 16380),
          # bf16 pairs on teams of 640 and 768 lanes
          (5, 10002), (4, 12002)]
# column sums over at most a few thousand rows in fp32: far inside 1e-5 of
# the terms' 2-norm
COLSUM_REL_SMALL = 1e-5


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def make_case(M, N, dtype, rms, seed, outlier_p=0.0, eps=None):
    inp = synth.make_inputs(M, N, dtype=dtype, seed=seed, names=("x", "dy", "gamma"),
                            outlier_p=outlier_p)
    eps = (1e-6 if rms else 1e-5) if eps is None else eps
    f = oracle.norm_fwd(inp["x"], eps=eps, rms=rms, dtype=dtype, want_u=False, want_y=False)
    inp["mean"] = f["mean"].astype(np.float32)
    inp["rstd"] = f["rstd"].astype(np.float32)
    return inp, eps


def run_bwd(rms, inp, dtype, eps, misalign=False, recompute=False, dparam_dtype=None,
            want_dbeta=True, want_dbias=False):
    dy = to_dev(inp["dy"], dtype, misalign)
    x = to_dev(inp["x"], dtype)
    g = to_dev(inp["gamma"], dtype)
    rstd = None if recompute else torch.from_numpy(inp["rstd"]).cuda()
    if rms:
        out = nf.rms_bwd(dy, x, g, rstd, eps, dparam_dtype=dparam_dtype, want_dbeta=want_dbeta,
                         want_dbias=want_dbias)
    else:
        mean = torch.from_numpy(inp["mean"]).cuda()
        out = nf.ln_bwd(dy, x, g, mean, rstd, dparam_dtype=dparam_dtype, want_dbeta=want_dbeta,
                        want_dbias=want_dbias)
    torch.cuda.synchronize()
    return out


def oracle_bwd(rms, inp, dtype, eps, recompute=False, rows=None, want_dbias=False):
    sl = slice(None) if rows is None else rows
    return oracle.norm_bwd(inp["dy"][sl], inp["x"][sl], inp["gamma"],
                           None if rms else inp["mean"][sl],
                           None if recompute else inp["rstd"][sl], eps, rms=rms, dtype=dtype,
                           want_dbias=want_dbias)


@pytest.mark.parametrize("M,N", SHAPES)
@pytest.mark.parametrize("rms", [False, True], ids=["ln", "rms"])
@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("misalign", [False, True], ids=["vec", "elem"])
def test_bwd_matches_oracle(M, N, rms, dtype, misalign):
    inp, eps = make_case(M, N, dtype, rms, seed=M * 31 + N)
    out = run_bwd(rms, inp, dtype, eps, misalign, dparam_dtype=torch.float32)
    ref = oracle_bwd(rms, inp, dtype, eps)
    assert_rows_close(f64(out["dx"]), ref["dx"], dtype, "dx",
                      scale=dx_term_scale(inp["dy"], inp["gamma"], ref["rstd"], dtype))
    assert_colsums_close(f64(out["dgamma"]), ref["dgamma"], ref["dgamma_l2"], COLSUM_REL_SMALL,
                         "dgamma")
    assert_colsums_close(f64(out["dbeta"]), ref["dbeta"], ref["dbeta_l2"], COLSUM_REL_SMALL,
                         "dbeta")


@pytest.mark.parametrize("M,N", SHAPES)
@pytest.mark.parametrize("rms", [False, True], ids=["ln", "rms"])
@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("misalign", [False, True], ids=["vec", "elem"])
def test_bwd_dbias_matches_oracle(M, N, rms, dtype, misalign):
    """The gradient of the forward's bias (column sums of dx) from the same
    pass; dx, dgamma and dbeta are bit-identical to a call without it."""
    inp, eps = make_case(M, N, dtype, rms, seed=M * 37 + N)
    out = run_bwd(rms, inp, dtype, eps, misalign, dparam_dtype=torch.float32, want_dbias=True)
    ref = oracle_bwd(rms, inp, dtype, eps, want_dbias=True)
    l2 = np.maximum(ref["dbias_l2"], dbias_term_l2(inp["dy"], inp["gamma"], ref["rstd"], dtype))
    assert_colsums_close(f64(out["dbias"]), ref["dbias"], l2, COLSUM_REL_SMALL, "dbias")
    plain = run_bwd(rms, inp, dtype, eps, misalign, dparam_dtype=torch.float32)
    for k in ("dx", "dgamma", "dbeta"):
        assert torch.equal(out[k], plain[k]), k


@pytest.mark.parametrize("rms", [False, True], ids=["ln", "rms"])
def test_bwd_dbias_bf16_is_rounded_sum(rms):
    M, N = 3000, 384
    inp, eps = make_case(M, N, BF16, rms, seed=77)
    o32 = run_bwd(rms, inp, BF16, eps, dparam_dtype=torch.float32, want_dbias=True)
    o16 = run_bwd(rms, inp, BF16, eps, dparam_dtype=torch.bfloat16, want_dbias=True)
    assert torch.equal(o16["dbias"], o32["dbias"].to(torch.bfloat16))
    ref = oracle_bwd(rms, inp, BF16, eps, want_dbias=True)
    l2 = np.maximum(ref["dbias_l2"], dbias_term_l2(inp["dy"], inp["gamma"], ref["rstd"], BF16))
    assert_colsums_close(f64(o16["dbias"]), ref["dbias"], l2, COLSUM_REL_SMALL,
                         "dbias (bf16)", dtype=BF16)


@pytest.mark.parametrize("N", [7, 384, 4096])
def test_rms_bwd_recomputes_rstd(N):
    M = 300
    inp, eps = make_case(M, N, BF16, True, seed=N)
    out = run_bwd(True, inp, BF16, eps, recompute=True, dparam_dtype=torch.float32)
    ref = oracle_bwd(True, inp, BF16, eps, recompute=True)
    assert_rows_close(f64(out["dx"]), ref["dx"], BF16, "dx",
                      scale=dx_term_scale(inp["dy"], inp["gamma"], ref["rstd"], BF16))
    assert_colsums_close(f64(out["dgamma"]), ref["dgamma"], ref["dgamma_l2"], COLSUM_REL_SMALL,
                         "dgamma")


@pytest.mark.parametrize("rms", [False, True], ids=["ln", "rms"])
def test_bwd_bf16_params_are_rounded_sums(rms):
    """dgamma / dbeta requested in bf16: the fp32 column sums rounded to
    nearest-even, i.e. within one bf16 ulp of the exact sums."""
    inp, eps = make_case(2000, 384, BF16, rms, seed=77)
    out = run_bwd(rms, inp, BF16, eps, dparam_dtype=torch.bfloat16)
    out32 = run_bwd(rms, inp, BF16, eps, dparam_dtype=torch.float32)
    ref = oracle_bwd(rms, inp, BF16, eps)
    for k in ("dgamma", "dbeta"):
        assert out[k].dtype == torch.bfloat16
        assert torch.equal(out[k], out32[k].to(torch.bfloat16)), k
        assert_colsums_close(f64(out[k]), ref[k], ref[k + "_l2"], COLSUM_REL_SMALL, k, dtype=BF16)


def test_bwd_gamma_absent_means_one():
    inp, eps = make_case(200, 256, BF16, False, seed=4)
    x, dy = to_dev(inp["x"], BF16), to_dev(inp["dy"], BF16)
    mean, rstd = torch.from_numpy(inp["mean"]).cuda(), torch.from_numpy(inp["rstd"]).cuda()
    out = nf.ln_bwd(dy, x, None, mean, rstd, dparam_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.norm_bwd(inp["dy"], inp["x"], None, inp["mean"], inp["rstd"], eps)
    assert_rows_close(f64(out["dx"]), ref["dx"], BF16, "dx",
                      scale=dx_term_scale(inp["dy"], None, ref["rstd"], BF16))
    assert_colsums_close(f64(out["dgamma"]), ref["dgamma"], ref["dgamma_l2"], COLSUM_REL_SMALL,
                         "dgamma")


def test_bwd_outliers_wide_rows():
    inp, eps = make_case(256, 4096, BF16, False, seed=5, outlier_p=0.01)
    out = run_bwd(False, inp, BF16, eps, dparam_dtype=torch.float32)
    ref = oracle_bwd(False, inp, BF16, eps)
    assert_rows_close(f64(out["dx"]), ref["dx"], BF16, "dx",
                      scale=dx_term_scale(inp["dy"], inp["gamma"], ref["rstd"], BF16))
    assert_colsums_close(f64(out["dgamma"]), ref["dgamma"], ref["dgamma_l2"], COLSUM_REL_SMALL,
                         "dgamma")


def test_bwd_empty_rows_zero_params():
    x = torch.empty((0, 384), dtype=torch.bfloat16, device="cuda")
    st = torch.empty((0,), dtype=torch.float32, device="cuda")
    dg = torch.full((384,), 7.0, device="cuda")
    db = torch.full((384,), 7.0, device="cuda")
    dbias = torch.full((384,), 7.0, device="cuda")
    out = nf.ln_bwd(x, x, None, st, st, dparam_dtype=torch.float32,
                    out={"dgamma": dg, "dbeta": db, "dbias": dbias})
    torch.cuda.synchronize()
    assert torch.count_nonzero(out["dgamma"]) == 0 and torch.count_nonzero(out["dbeta"]) == 0
    assert torch.count_nonzero(out["dbias"]) == 0


def test_bwd_rejects_small_workspace():
    M, N = 1000, 384
    need = nf.bwd_workspace_size(M, N, torch.bfloat16)
    assert need > 0
    x = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    st = torch.ones((M,), dtype=torch.float32, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(nf.NormError) as e:
        nf.ln_bwd(x, x, None, st, st, workspace=ws)
    assert e.value.status == 6


# Shapes whose split of the column reduction over the rows (row groups per
# workgroup) lands between its bounds, with ragged last workgroups: wide rows
# at one workgroup per CU, narrow rows at about two per CU.
SPLIT_SHAPES = [(1024, 16384), (601, 8192), (4097, 4096), (65537, 384), (16385, 2048)]


@pytest.mark.parametrize("M,N", SPLIT_SHAPES)
@pytest.mark.parametrize("rms,dtype", [(False, BF16), (True, F32)], ids=["ln-bf16", "rms-f32"])
def test_bwd_row_splits_match_oracle(M, N, rms, dtype):
    inp, eps = make_case(M, N, dtype, rms, seed=M + 7 * N)
    out = run_bwd(rms, inp, dtype, eps, dparam_dtype=torch.float32, want_dbias=True)
    ref = oracle_bwd(rms, inp, dtype, eps, want_dbias=True)
    assert_rows_close(f64(out["dx"]), ref["dx"], dtype, "dx",
                      scale=dx_term_scale(inp["dy"], inp["gamma"], ref["rstd"], dtype))
    for k in ("dgamma", "dbeta"):
        assert_colsums_close(f64(out[k]), ref[k], ref[k + "_l2"], COLSUM_REL_SMALL, k)
    l2 = np.maximum(ref["dbias_l2"], dbias_term_l2(inp["dy"], inp["gamma"], ref["rstd"], dtype))
    assert_colsums_close(f64(out["dbias"]), ref["dbias"], l2, COLSUM_REL_SMALL, "dbias")


# Few rows of many columns: the rows are split along N into column chunks
# (two passes: chunk row sums, then dx).  Each shape runs with the split
# forced on and off; ragged M (not a multiple of the four rows of a group),
# a ragged last chunk, one row, and a forced split at larger M (several
# groups per row block).
SPLIT_N_SHAPES = [(1, 4096), (3, 16384), (16, 16384), (64, 16384), (255, 8192), (7, 3000),
                  (130, 2056), (1030, 4096)]


@pytest.mark.parametrize("M,N", SPLIT_N_SHAPES)
@pytest.mark.parametrize("case", ["ln-bf16", "rms-f32", "rms-bf16-recompute", "ln-f32"])
@pytest.mark.parametrize("split", ["1", "0"], ids=["split", "whole"])
def test_bwd_split_along_n_matches_oracle(M, N, case, split, tuning):
    rms = case.startswith("rms")
    dtype = F32 if "f32" in case else BF16
    recompute = case.endswith("recompute")
    tuning.setenv("NORMFUSE_BWD_SPLIT", split)
    inp, eps = make_case(M, N, dtype, rms, seed=M * 5 + N)
    out = run_bwd(rms, inp, dtype, eps, recompute=recompute, dparam_dtype=torch.float32,
                  want_dbias=True)
    ref = oracle_bwd(rms, inp, dtype, eps, recompute=recompute, want_dbias=True)
    assert_rows_close(f64(out["dx"]), ref["dx"], dtype, "dx",
                      scale=dx_term_scale(inp["dy"], inp["gamma"], ref["rstd"], dtype))
    for k in ("dgamma",) + (() if rms else ("dbeta",)):
        assert_colsums_close(f64(out[k]), ref[k], ref[k + "_l2"], COLSUM_REL_SMALL, k)
    l2 = np.maximum(ref["dbias_l2"], dbias_term_l2(inp["dy"], inp["gamma"], ref["rstd"], dtype))
    assert_colsums_close(f64(out["dbias"]), ref["dbias"], l2, COLSUM_REL_SMALL, "dbias")


@pytest.mark.parametrize("M,N", [(64, 16384), (13, 4096)])
@pytest.mark.parametrize("rms", [False, True], ids=["ln", "rms"])
def test_bwd_split_along_n_options(M, N, rms, tuning):
    """Zero-centred gamma and the mean epilogue on the split path: against
    the oracle run with the same options."""
    tuning.setenv("NORMFUSE_BWD_SPLIT", "1")
    inp, eps = make_case(M, N, BF16, rms, seed=M + 3 * N)
    dy, x, g = (to_dev(inp[k], BF16) for k in ("dy", "x", "gamma"))
    rstd = torch.from_numpy(inp["rstd"]).cuda()
    kw = dict(dparam_dtype=torch.float32, want_dbias=True, zero_centered_gamma=True,
              dparam_mean=True)
    if rms:
        out = nf.rms_bwd(dy, x, g, rstd, eps, **kw)
    else:
        out = nf.ln_bwd(dy, x, g, torch.from_numpy(inp["mean"]).cuda(), rstd, **kw)
    torch.cuda.synchronize()
    ref = oracle.norm_bwd(inp["dy"], inp["x"], inp["gamma"], None if rms else inp["mean"],
                          inp["rstd"], eps, rms=rms, dtype=BF16, want_dbias=True,
                          zero_centered_gamma=True, dparam_mean=True)
    w = (to_dev(inp["gamma"], BF16).float() + 1.0).to(torch.bfloat16)
    wh = from_dev(w, BF16)
    assert_rows_close(f64(out["dx"]), ref["dx"], BF16, "dx",
                      scale=dx_term_scale(inp["dy"], wh, ref["rstd"], BF16))
    for k in ("dgamma",) + (() if rms else ("dbeta",)):
        assert_colsums_close(f64(out[k]), ref[k], ref[k + "_l2"], COLSUM_REL_SMALL, k)
    l2 = np.maximum(ref["dbias_l2"], dbias_term_l2(inp["dy"], wh, ref["rstd"], BF16) / M)
    assert_colsums_close(f64(out["dbias"]), ref["dbias"], l2, COLSUM_REL_SMALL, "dbias")


def test_bwd_split_along_n_is_deterministic(tuning):
    tuning.setenv("NORMFUSE_BWD_SPLIT", "1")
    inp, eps = make_case(200, 16384, BF16, False, seed=3)
    a = run_bwd(False, inp, BF16, eps, dparam_dtype=torch.float32, want_dbias=True)
    b = run_bwd(False, inp, BF16, eps, dparam_dtype=torch.float32, want_dbias=True)
    for k in ("dx", "dgamma", "dbeta", "dbias"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("M,N,dtype", [(20000, 384, BF16), (9000, 1000, F32), (3000, 4096, BF16)])
def test_bwd_many_partial_rows_two_level_sums(M, N, dtype, tuning):
    """One row group per workgroup (forced) leaves more than 512 partial
    rows, which the column sums add in two launches."""
    tuning.setenv("NORMFUSE_BWD_GROUPS_PER_WG", "1")
    inp, eps = make_case(M, N, dtype, False, seed=M + N)
    out = run_bwd(False, inp, dtype, eps, dparam_dtype=torch.float32, want_dbias=True)
    ref = oracle_bwd(False, inp, dtype, eps, want_dbias=True)
    assert_rows_close(f64(out["dx"]), ref["dx"], dtype, "dx",
                      scale=dx_term_scale(inp["dy"], inp["gamma"], ref["rstd"], dtype))
    for k in ("dgamma", "dbeta"):
        assert_colsums_close(f64(out[k]), ref[k], ref[k + "_l2"], COLSUM_REL_SMALL, k)
    l2 = np.maximum(ref["dbias_l2"], dbias_term_l2(inp["dy"], inp["gamma"], ref["rstd"], dtype))
    assert_colsums_close(f64(out["dbias"]), ref["dbias"], l2, COLSUM_REL_SMALL, "dbias")


def test_bwd_is_deterministic():
    inp, eps = make_case(20000, 384, BF16, False, seed=8)
    a = run_bwd(False, inp, BF16, eps, dparam_dtype=torch.float32)
    b = run_bwd(False, inp, BF16, eps, dparam_dtype=torch.float32)
    for k in ("dx", "dgamma", "dbeta"):
        assert torch.equal(a[k], b[k]), k


def test_product_library_ignores_tuning_environment(tuning):
    """The product build takes its choices from the call's arguments alone:
    a tuning override changes the test build's workspace size, not the
    product's."""
    M, N = 20000, 384
    base = nf.bwd_workspace_size(M, N, torch.bfloat16)  # the test build, no overrides
    tuning.setenv("NORMFUSE_BWD_GROUPS_PER_WG", "1")
    forced = nf.bwd_workspace_size(M, N, torch.bfloat16)
    assert forced > base
    product = nf.load(nf.build.LIB)
    n = ctypes.c_size_t(0)
    assert product.norm_bwd_workspace_size(M, N, nf.BF16, ctypes.byref(n)) == 0
    assert n.value == base
