"""ln_bwd_noalloc, the backward on the library's static device scratch (for
callers that cannot allocate), through the C ABI: its outputs equal those of
ln_bwd with a caller workspace bit for bit (same kernels, same summation
order) and meet the oracle's bar; two calls in a row, the second with fewer
rows, reuse the scratch; a problem whose workspace exceeds the scratch is
refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import normalization_ln_fwd_amd as nf
import oracle
import synth
from gpu_util import BF16, f64, require_gpu, to_dev
from tolerance import assert_colsums_close, assert_rows_close, dx_term_scale

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _case(M, N, seed):
    inp = synth.make_inputs(M, N, dtype=BF16, seed=seed, names=("x", "dy", "gamma"))
    f = oracle.norm_fwd(inp["x"], eps=1e-5, dtype=BF16, want_u=False, want_y=False)
    inp["mean"], inp["rstd"] = f["mean"].astype(np.float32), f["rstd"].astype(np.float32)
    return inp


def _noalloc_abi(d, M, N, dbias):
    """ln_bwd_noalloc called through ctypes with every output preallocated."""
    out = {"dx": torch.empty_like(d["x"]),
           "dgamma": torch.empty(N, dtype=torch.float32, device="cuda"),
           "dbeta": torch.empty(N, dtype=torch.float32, device="cuda"),
           "dbias": torch.empty(N, dtype=torch.float32, device="cuda") if dbias else None}
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    st = nf.library().ln_bwd_noalloc(
        ptr(d["dy"]), ptr(d["x"]), ptr(d["gamma"]), ptr(d["mean"]), ptr(d["rstd"]), M, N,
        nf.BF16, ptr(out["dx"]), ptr(out["dgamma"]), ptr(out["dbeta"]), ptr(out["dbias"]),
        nf.F32, 0, torch.cuda.current_stream().cuda_stream)
    assert st == 0, nf.library().norm_status_string(st)
    return out


@pytest.mark.parametrize("shapes", [((8192, 4096), (3000, 4096)), ((20000, 384), (5000, 384)),
                                    ((301, 1024), (7, 1024)), ((2001, 1001), (7, 1001)),
                                    ((1025, 4100), (9, 4100)), ((2001, 386), (5, 386))],
                         ids=["8192x4096-then-3000", "20000x384-then-5000", "301x1024-then-7",
                              "2001x1001-then-7", "1025x4100-then-9", "2001x386-then-5"])
def test_noalloc_matches_workspace_entry_point(shapes):
    for i, ((M, N), dbias) in enumerate(zip(shapes, (True, False))):
        inp = _case(M, N, seed=M + i)
        d = {k: to_dev(inp[k], BF16) for k in ("x", "dy", "gamma")}
        d["mean"], d["rstd"] = (torch.from_numpy(inp[k]).cuda() for k in ("mean", "rstd"))
        got = _noalloc_abi(d, M, N, dbias)
        ref = nf.ln_bwd(d["dy"], d["x"], d["gamma"], d["mean"], d["rstd"],
                        dparam_dtype=torch.float32, want_dbias=dbias)
        torch.cuda.synchronize()
        for k in ("dx", "dgamma", "dbeta") + (("dbias",) if dbias else ()):
            assert torch.equal(got[k], ref[k]), (M, N, k)
        o = oracle.norm_bwd(inp["dy"], inp["x"], inp["gamma"], inp["mean"], inp["rstd"], 1e-5,
                            dtype=BF16)
        assert_rows_close(f64(got["dx"]), o["dx"], BF16, "dx",
                          scale=dx_term_scale(inp["dy"], inp["gamma"], o["rstd"], BF16))
        for k in ("dgamma", "dbeta"):
            assert_colsums_close(f64(got[k]), o[k], o[k + "_l2"], 1e-5, k)


def test_noalloc_binding_and_refusal():
    M, N = 2000, 384
    inp = _case(M, N, seed=5)
    d = {k: to_dev(inp[k], BF16) for k in ("x", "dy", "gamma")}
    mean, rstd = (torch.from_numpy(inp[k]).cuda() for k in ("mean", "rstd"))
    a = nf.ln_bwd_noalloc(d["dy"], d["x"], d["gamma"], mean, rstd, dparam_dtype=torch.bfloat16)
    b = nf.ln_bwd(d["dy"], d["x"], d["gamma"], mean, rstd, dparam_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for k in ("dx", "dgamma", "dbeta"):
        assert torch.equal(a[k], b[k]), k
    # 512 rows of 16384 columns with dbias need a 50 MB workspace: refused
    # (real buffers of that size, so nothing could be read past them)
    M, N = 512, 16384
    assert nf.bwd_workspace_size(M, N, torch.bfloat16) > nf.STATIC_SCRATCH_BYTES
    t = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    st = torch.ones(M, device="cuda")
    with pytest.raises(nf.NormError) as e:
        nf.ln_bwd_noalloc(t, t, None, st, st, dparam_dtype=torch.float32, want_dbias=True)
    assert e.value.status == 6
