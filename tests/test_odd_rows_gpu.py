"""GPU parity of the odd-row kernels: rows whose length is an odd multiple
of a unit U (U = 1: odd N; U = 2: N = 2 mod 4; U = 4: bf16 N = 4 mod 8)
and whose [M, N] tensors are aligned to 2U elements, each row read in
aligned vectors of 2U from its first such element plus its one leftover
unit (forward, FP8 forward, softmax, and the backward, whose teams each
keep one row parity).

Every shape the odd-row tables hold (bf16 rows up to 16383 columns, fp32
forward rows up to 8193), N = 1, row counts of both parities and around the
row-group size, several row groups per workgroup (the columns a lane holds
change with each row's parity), and every optional input.  Checked against
the oracle (the staged checks of the plain forward), against the
single-element kernels on the test build with the odd-row kernels turned
off (residual_out bit-identical: the same fused-add rounding), and for
writes outside the outputs (guard elements around each output stay
untouched).
"""
import re

import numpy as np
import pytest
import torch

import normalization_ln_fwd_amd as nf
import oracle
import synth
from gpu_util import BF16, F32, TORCH_DT, f64, require_gpu, to_dev
from test_fp8_gpu import check_pair as check_fp8, run_pair as run_fp8
from test_fwd_gpu import check_fwd, run_fwd
from tolerance import assert_rows_close

pytestmark = pytest.mark.gpu

# (M, N): each table entry at the longest row it holds (pairs' capacity
# 128, 256, 384, 512, 768, 1024, 1536, 2048, 3072, 4096, 5120, 6144, 8192,
# 10240, 12288, 16384 elements, plus the leftover), N = 1 and 3, odd and
# even row counts, a few thousand rows (many workgroups, several row groups
# each); fp32 8195 leaves the forward's table (its softmax goes on).
SHAPES_BF16 = [(1, 1), (2, 1), (5, 1), (3, 3), (3, 7), (8, 7), (37, 129), (17, 257), (12, 385),
               (40, 513), (9, 769), (33, 1025), (10, 1537), (31, 2049), (7, 3073), (20, 4097),
               (7, 5121), (11, 6145), (9, 8193), (6, 8191), (5, 10241), (4, 12289), (3, 16383),
               (2001, 385), (1025, 4097), (65, 1001)]
SHAPES_F32 = [(1, 1), (2, 1), (3, 7), (8, 7), (37, 129), (17, 257), (12, 385), (40, 513),
              (9, 769), (33, 1025), (10, 1537), (31, 2049), (7, 3073), (20, 4097), (7, 5121),
              (11, 6145), (7, 8193), (2001, 385), (5, 8195), (3, 16383), (3, 10243)]
# units 2 and 4: each table's narrow and wide entries, the longest rows,
# rows of a single leftover unit (N = 2, 4) and the same row parities
SHAPES_BF16_U2 = [(3, 2), (5, 6), (8, 10), (37, 130), (17, 258), (12, 386), (40, 514), (33, 1026),
                  (10, 1538), (31, 2050), (7, 3074), (20, 4098), (7, 5122), (11, 6146),
                  (9, 8194), (5, 10242), (4, 12290), (3, 16382), (2001, 386), (1025, 4098),
                  (9, 38), (5, 134), (7, 518), (6, 1030)]
SHAPES_BF16_U4 = [(3, 4), (5, 12), (8, 20), (37, 132), (17, 260), (12, 388), (40, 516), (33, 1028),
                  (10, 1540), (31, 2052), (7, 3076), (20, 4100), (7, 5124), (11, 6148),
                  (9, 8196), (5, 10244), (4, 12292), (3, 16380), (2001, 388), (1025, 4100),
                  (7, 524), (6, 2060)]
SHAPES_F32_U2 = [(3, 2), (5, 6), (8, 10), (37, 130), (17, 258), (40, 514), (33, 1026),
                 (31, 2050), (20, 4098), (7, 8194), (5, 8198), (3, 16382), (2001, 386),
                 (9, 38), (5, 134), (7, 518), (6, 1030), (5, 1286), (4, 4102), (3, 5126),
                 (3, 10246)]
CASES = ([(M, N, BF16) for M, N in SHAPES_BF16 + SHAPES_BF16_U2 + SHAPES_BF16_U4] +
         [(M, N, F32) for M, N in SHAPES_F32 + SHAPES_F32_U2])


def _id(c):
    M, N, dt = c
    return f"{'bf16' if dt == BF16 else 'f32'}-{M}x{N}"


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _unit(op, M, N, dtype):
    """The odd-row unit a call would take (0: another kernel)."""
    m = re.search(r"odd_kernel<\w+, unit (\d+),", nf.describe(op, M, N, dtype))
    return int(m.group(1)) if m else 0


@pytest.mark.parametrize("c", CASES, ids=_id)
@pytest.mark.parametrize("rms", [False, True], ids=["ln", "rms"])
def test_odd_forward_matches_oracle(c, rms):
    M, N, dtype = c
    inp = synth.make_inputs(M, N, dtype=dtype, seed=M * 7 + N)
    eps = 1e-6 if rms else 1e-5
    out = run_fwd(rms, inp, dtype, eps)
    check_fwd(rms, inp, dtype, eps, out)


PARTS = [("x",), ("x", "gamma"), ("x", "residual", "gamma", "beta"),
         ("x", "bias", "gamma", "beta")]


@pytest.mark.parametrize("parts", PARTS, ids=lambda p: "+".join(p))
@pytest.mark.parametrize("M,N,dtype", [(9, 255, BF16), (33, 1023, F32), (7, 5119, BF16)])
def test_odd_forward_optional_inputs(parts, M, N, dtype):
    inp = synth.make_inputs(M, N, dtype=dtype, seed=N)
    for rms in (False, True):
        out = run_fwd(rms, inp, dtype, 1e-5, parts=parts)
        _check_parts(rms, inp, dtype, out, parts)


def _check_parts(rms, inp, dtype, out, parts):
    g = {k: (inp[k] if k in parts else None) for k in ("x", "bias", "residual", "gamma", "beta")}
    ref = oracle.norm_fwd(g["x"], g["bias"], g["residual"], g["gamma"], g["beta"], 1e-5,
                          rms=rms, dtype=dtype)
    assert_rows_close(f64(out["y"]), ref["y"], dtype, "y", ulps=2.0)
    rel = np.abs(f64(out["rstd"]) - ref["rstd"]) / ref["rstd"]
    assert np.all(rel <= 1e-5), rel.max()


@pytest.mark.parametrize("c", [(3, 7, BF16), (9, 8193, BF16), (2001, 385, BF16), (3, 16383, BF16),
                               (31, 2049, F32), (2001, 385, F32)], ids=_id)
@pytest.mark.parametrize("rms", [False, True], ids=["ln", "rms"])
def test_odd_forward_matches_single_element_kernels(c, rms, tuning):
    """The same call on the test build with the odd-row kernels turned off:
    residual_out bit-identical (the fused add rounds the same values), y
    within one ulp, rstd within its summation-order bounds."""
    M, N, dtype = c
    inp = synth.make_inputs(M, N, dtype=dtype, seed=M + N)
    eps = 1e-6 if rms else 1e-5
    a = run_fwd(rms, inp, dtype, eps)
    tuning.setenv("NORMFUSE_PAIRS", "0")
    assert not _unit("rms_fwd" if rms else "ln_fwd", M, N, dtype)
    b = run_fwd(rms, inp, dtype, eps)
    assert torch.equal(a["residual_out"], b["residual_out"])
    assert_rows_close(f64(a["y"]), f64(b["y"]), dtype, "y pairs vs elements", ulps=1.0)
    rel = np.abs(f64(a["rstd"]) - f64(b["rstd"])) / f64(b["rstd"])
    assert np.all(rel <= 2e-6), rel.max()


@pytest.mark.parametrize("groups", [1, 2, 3, 8])
@pytest.mark.parametrize("M", [1, 7, 8, 9, 63, 64, 65, 257])
def test_odd_forward_walks_and_row_parities(M, groups, tuning):
    """Row groups per workgroup forced, row counts around the group size (4
    rows for the 64-lane teams), so that a workgroup's groups start on even
    and odd rows alike."""
    tuning.setenv("NORMFUSE_FWD_GROUPS_PER_WG", str(groups))
    tuning.setenv("NORMFUSE_FWD_INTERLEAVE", "3")
    N = 255
    inp = synth.make_inputs(M, N, dtype=BF16, seed=M * 31 + groups)
    out = run_fwd(False, inp, BF16, 1e-5)
    check_fwd(False, inp, BF16, 1e-5, out)


@pytest.mark.parametrize("M,N,dtype", [(3, 7, BF16), (5, 1, F32), (9, 8193, BF16),
                                       (65, 1001, F32), (7, 5121, BF16), (3, 16383, BF16)])
def test_odd_outputs_stay_in_bounds(M, N, dtype):
    """Outputs placed two elements into guard buffers (still aligned to two
    elements): the guard elements before and after every [M, N] output, the
    FP8 codes' and the statistics' keep their fill."""
    tdt = TORCH_DT[dtype]
    inp = synth.make_inputs(M, N, dtype=dtype, seed=M + 3 * N)
    dev = {k: to_dev(inp[k], dtype) for k in ("x", "bias", "residual", "gamma", "beta")}
    G = 32

    def guarded(n, dt, fill):
        buf = torch.full((n + 2 + G,), fill, dtype=dt, device="cuda")
        return buf, buf[2:2 + n]

    yb, y = guarded(M * N, tdt, 7.0)
    rb, r = guarded(M * N, tdt, 7.0)
    mb, mean = guarded(M, torch.float32, 7.0)
    sb, rstd = guarded(M, torch.float32, 7.0)
    qb, q = guarded(M * N, torch.uint8, 0x5A)
    out = nf.ln_fwd(dev["x"], dev["bias"], dev["residual"], dev["gamma"], dev["beta"],
                    want_amax=True, out={"y": y.view(M, N), "residual_out": r.view(M, N),
                                         "mean": mean, "rstd": rstd})
    sc = torch.ones(1, dtype=torch.float32, device="cuda")
    nf.ln_fwd_fp8(dev["x"], sc, dev["bias"], dev["residual"], dev["gamma"], dev["beta"],
                  out={"y": q.view(M, N)})
    sm = torch.full((M * N + 2 + G,), 7.0, dtype=tdt, device="cuda")
    nf.softmax_fwd(dev["x"], out=sm[2:2 + M * N].view(M, N))
    torch.cuda.synchronize()
    for name, buf, n, fill in (("y", yb, M * N, 7.0), ("residual_out", rb, M * N, 7.0),
                               ("mean", mb, M, 7.0), ("rstd", sb, M, 7.0),
                               ("softmax", sm, M * N, 7.0)):
        assert torch.all(buf[:2] == fill) and torch.all(buf[2 + n:] == fill), name
    assert torch.all(qb[:2] == 0x5A) and torch.all(qb[2 + M * N:] == 0x5A), "fp8 y"
    check_fwd(False, inp, dtype, 1e-5, out)


@pytest.mark.parametrize("c", [(3, 7, BF16), (40, 513, BF16), (9, 8193, BF16), (2001, 385, BF16),
                               (17, 257, F32), (20, 4097, F32), (3, 16383, BF16)], ids=_id)
@pytest.mark.parametrize("rms", [False, True], ids=["ln", "rms"])
def test_odd_fp8_codes_are_the_quantised_stored_y(c, rms):
    M, N, dtype = c
    inp = synth.make_inputs(M, N, dtype=dtype, seed=M * 5 + N)
    eps = 1e-6 if rms else 1e-5
    ref = oracle.norm_fwd(inp["x"], inp["bias"], inp["residual"], inp["gamma"], inp["beta"], eps,
                          rms=rms, dtype=dtype)
    scale = float(np.float32(448.0 / max(ref["amax"], 1e-30)))
    plain, q = run_fp8(rms, inp, dtype, eps, scale)
    check_fp8(plain, q, scale, dtype, exact_y=ref["y"])


@pytest.mark.parametrize("c", [(3, 7, BF16), (2001, 385, BF16), (65, 1001, F32), (1, 1, F32)],
                         ids=_id)
@pytest.mark.parametrize("rms", [False, True], ids=["ln", "rms"])
def test_odd_amax_workspace(c, rms):
    """amax combined in the workspace equals the reset path's and max |y|."""
    M, N, dtype = c
    inp = synth.make_inputs(M, N, dtype=dtype, seed=M + 11 * N)
    dev = {k: to_dev(inp[k], dtype) for k in ("x", "bias", "residual", "gamma", "beta")}
    fn = nf.rms_fwd if rms else nf.ln_fwd
    ws = nf.amax_workspace()
    a = fn(dev["x"], dev["bias"], dev["residual"], dev["gamma"], dev["beta"], want_amax=True)
    b = fn(dev["x"], dev["bias"], dev["residual"], dev["gamma"], dev["beta"], want_amax=True,
           amax_workspace=ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(ws).item() == 0
    assert float(b["amax"].item()) == float(a["amax"].item()) == \
        float(b["y"].float().abs().max().item())


@pytest.mark.parametrize("rms", [False, True], ids=["ln", "rms"])
def test_odd_zero_centred_gamma(rms):
    M, N = 33, 1023
    inp = synth.make_inputs(M, N, dtype=BF16, seed=12)
    dev = {k: to_dev(inp[k], BF16) for k in ("x", "gamma", "beta")}
    fn = nf.rms_fwd if rms else nf.ln_fwd
    out = fn(dev["x"], None, None, dev["gamma"], dev["beta"], 1e-5, zero_centered_gamma=True)
    torch.cuda.synchronize()
    ref = oracle.norm_fwd(inp["x"], None, None, inp["gamma"], inp["beta"], 1e-5, rms=rms,
                          dtype=BF16, zero_centered_gamma=True)
    assert_rows_close(f64(out["y"]), ref["y"], BF16, "y", ulps=2.0)


@pytest.mark.parametrize("c", CASES, ids=_id)
def test_odd_softmax_matches_oracle(c):
    M, N, dtype = c
    x = synth.make_inputs(M, N, dtype=dtype, seed=M * 3 + N, names=("x",))["x"]
    y = nf.softmax_fwd(to_dev(x, dtype))
    torch.cuda.synchronize()
    assert_rows_close(f64(y), oracle.softmax_fwd(x, dtype=dtype), dtype, "softmax")


# ---------------------------------------------------------------- backward
from test_bwd_gpu import COLSUM_REL_SMALL, make_case, oracle_bwd, run_bwd  # noqa: E402
from tolerance import assert_colsums_close, dbias_term_l2, dx_term_scale  # noqa: E402

# each backward table entry at its longest row (two or four teams per
# workgroup, each keeping one row parity), row counts of both parities and
# around the group sizes (2 and 4 rows), a few thousand rows; 8195 leaves
# the table
BWD_SHAPES = [(1, 1), (2, 1), (3, 3), (5, 7), (8, 7), (37, 129), (17, 257), (12, 385), (40, 513),
              (9, 769), (33, 1025), (10, 1537), (31, 2049), (7, 3073), (20, 4097), (7, 5121),
              (11, 6145), (9, 8193), (6, 8191), (2001, 385), (1025, 4097), (5, 8195)]
BWD_SHAPES_U2 = [(3, 2), (5, 6), (8, 10), (37, 130), (12, 386), (33, 1026), (31, 2050),
                 (20, 4098), (11, 6146), (9, 8194), (2001, 386), (1025, 4098), (5, 8198),
                 (9, 38), (5, 134), (7, 198), (6, 390), (7, 518), (6, 1030), (5, 1286),
                 (4, 4102)]
BWD_SHAPES_U4 = [(3, 4), (5, 12), (8, 20), (37, 132), (12, 388), (33, 1028), (31, 2052),
                 (20, 4100), (11, 6148), (9, 8196), (2001, 388), (1025, 4100), (5, 8204),
                 (9, 140), (7, 396), (7, 524), (6, 1036), (6, 2060), (5, 2572), (4, 4108)]
BWD_CASES = ([(M, N, BF16) for M, N in BWD_SHAPES + BWD_SHAPES_U2 + BWD_SHAPES_U4] +
             [(M, N, F32) for M, N in BWD_SHAPES + BWD_SHAPES_U2])


def _check_bwd(inp, out, ref, dtype, dbias):
    assert_rows_close(f64(out["dx"]), ref["dx"], dtype, "dx",
                      scale=dx_term_scale(inp["dy"], inp["gamma"], ref["rstd"], dtype))
    assert_colsums_close(f64(out["dgamma"]), ref["dgamma"], ref["dgamma_l2"], COLSUM_REL_SMALL,
                         "dgamma")
    assert_colsums_close(f64(out["dbeta"]), ref["dbeta"], ref["dbeta_l2"], COLSUM_REL_SMALL,
                         "dbeta")
    if dbias:
        l2 = np.maximum(ref["dbias_l2"], dbias_term_l2(inp["dy"], inp["gamma"], ref["rstd"], dtype))
        assert_colsums_close(f64(out["dbias"]), ref["dbias"], l2, COLSUM_REL_SMALL, "dbias")


@pytest.mark.parametrize("c", BWD_CASES, ids=_id)
@pytest.mark.parametrize("rms", [False, True], ids=["ln", "rms"])
def test_odd_backward_matches_oracle(c, rms):
    """dx row by row, dgamma / dbeta / dbias against the oracle's column
    sums; dx, dgamma and dbeta identical without dbias."""
    M, N, dtype = c
    inp, eps = make_case(M, N, dtype, rms, seed=M * 41 + N)
    out = run_bwd(rms, inp, dtype, eps, dparam_dtype=torch.float32, want_dbias=True)
    _check_bwd(inp, out, oracle_bwd(rms, inp, dtype, eps, want_dbias=True), dtype, True)
    plain = run_bwd(rms, inp, dtype, eps, dparam_dtype=torch.float32)
    for k in ("dx", "dgamma", "dbeta"):
        assert torch.equal(out[k], plain[k]), k


@pytest.mark.parametrize("c", [(3, 7, BF16), (2001, 385, F32), (9, 8193, BF16), (10, 1537, F32)],
                         ids=_id)
def test_odd_backward_rms_recomputes_rstd(c):
    M, N, dtype = c
    inp, eps = make_case(M, N, dtype, True, seed=M + 5 * N)
    out = run_bwd(True, inp, dtype, eps, recompute=True, dparam_dtype=torch.float32)
    _check_bwd(inp, out, oracle_bwd(True, inp, dtype, eps, recompute=True), dtype, False)


@pytest.mark.parametrize("c", [(3, 7, BF16), (9, 8193, BF16), (2001, 385, BF16), (1025, 4097, F32),
                               (31, 2049, F32)], ids=_id)
@pytest.mark.parametrize("rms", [False, True], ids=["ln", "rms"])
def test_odd_backward_matches_single_element_kernels(c, rms, tuning):
    """The same call with the odd-row kernels turned off: both within the
    oracle's bar, and dx within one ulp (or its row scale) of each other."""
    M, N, dtype = c
    inp, eps = make_case(M, N, dtype, rms, seed=M + 9 * N)
    a = run_bwd(rms, inp, dtype, eps, dparam_dtype=torch.float32, want_dbias=True)
    tuning.setenv("NORMFUSE_PAIRS", "0")
    assert not _unit("rms_bwd" if rms else "ln_bwd", M, N, dtype)
    b = run_bwd(rms, inp, dtype, eps, dparam_dtype=torch.float32, want_dbias=True)
    ref = oracle_bwd(rms, inp, dtype, eps, want_dbias=True)
    _check_bwd(inp, a, ref, dtype, True)
    _check_bwd(inp, b, ref, dtype, True)
    assert_rows_close(f64(a["dx"]), f64(b["dx"]), dtype, "dx pairs vs elements",
                      scale=dx_term_scale(inp["dy"], inp["gamma"], ref["rstd"], dtype))


@pytest.mark.parametrize("groups", [1, 2, 3, 7])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 63, 64, 65, 257])
def test_odd_backward_walks(M, groups, tuning):
    """Row groups per workgroup and interleave blocks forced (more or fewer
    partial rows), row counts around the group size of four."""
    tuning.setenv("NORMFUSE_BWD_GROUPS_PER_WG", str(groups))
    tuning.setenv("NORMFUSE_BWD_INTERLEAVE", "3")
    N = 1001
    inp, eps = make_case(M, N, BF16, False, seed=M * 13 + groups)
    out = run_bwd(False, inp, BF16, eps, dparam_dtype=torch.float32, want_dbias=True)
    _check_bwd(inp, out, oracle_bwd(False, inp, BF16, eps, want_dbias=True), BF16, True)


@pytest.mark.parametrize("M,N,dtype", [(3, 7, BF16), (5, 1, F32), (9, 8193, BF16),
                                       (65, 1001, F32)])
def test_odd_backward_dx_stays_in_bounds(M, N, dtype):
    inp, eps = make_case(M, N, dtype, False, seed=M + 7 * N)
    tdt = TORCH_DT[dtype]
    buf = torch.full((M * N + 2 + 32,), 7.0, dtype=tdt, device="cuda")
    dx = buf[2:2 + M * N].view(M, N)
    nf.ln_bwd(to_dev(inp["dy"], dtype), to_dev(inp["x"], dtype), to_dev(inp["gamma"], dtype),
              torch.from_numpy(inp["mean"]).cuda(), torch.from_numpy(inp["rstd"]).cuda(),
              dparam_dtype=torch.float32, out={"dx": dx})
    torch.cuda.synchronize()
    assert torch.all(buf[:2] == 7.0) and torch.all(buf[2 + M * N:] == 7.0)
    ref = oracle_bwd(False, inp, dtype, eps)
    assert_rows_close(f64(dx), ref["dx"], dtype, "dx",
                      scale=dx_term_scale(inp["dy"], inp["gamma"], ref["rstd"], dtype))
