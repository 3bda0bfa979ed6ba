"""In-place calls: an [M, N] output passed as the very tensor of an [M, N]
input of the same call (y over x or residual, residual_out over x or
residual, dx over dy or x, softmax's y over x).  Every workgroup loads a row
group before it stores that group's outputs, and no other workgroup reads
those rows, so the results must equal the out-of-place call's bit for bit.
The shapes reach each kind of kernel: narrow rows in 256- and 512-thread
workgroups, wide rows with the next group's loads in flight (forward) or the
pipelined walk (backward), 8-byte vectors, single elements, fp32, and the
backward's split of few wide rows along N."""
import pytest
import torch

import normalization_ln_fwd_amd as nf
import synth
from gpu_util import BF16, F32, require_gpu, to_dev

pytestmark = pytest.mark.gpu

FWD_SHAPES = [(BF16, 5000, 384), (BF16, 70000, 384), (BF16, 300, 4096), (BF16, 64, 8192),
              (BF16, 301, 4100), (BF16, 77, 1001), (F32, 300, 384), (F32, 33, 4096)]
BWD_SHAPES = [(BF16, 5000, 384), (BF16, 1024, 4096), (BF16, 64, 16384), (BF16, 301, 4100),
              (BF16, 77, 1001), (F32, 300, 384), (F32, 33, 4096)]
IDS = lambda c: f"{'bf16' if c[0] == BF16 else 'f32'}-{c[1]}x{c[2]}"


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _inputs(dtype, M, N, seed):
    inp = synth.make_inputs(M, N, dtype=dtype, seed=seed,
                            names=("x", "residual", "bias", "gamma", "beta", "dy"))
    return {k: to_dev(v, dtype) for k, v in inp.items()}


@pytest.mark.parametrize("case", FWD_SHAPES, ids=IDS)
@pytest.mark.parametrize("rms", [False, True], ids=["ln", "rms"])
@pytest.mark.parametrize("alias", ["y=x,res_out=res", "y=res,res_out=x"])
def test_forward_in_place(case, rms, alias):
    dtype, M, N = case
    d = _inputs(dtype, M, N, seed=M + N)
    fn = nf.rms_fwd if rms else nf.ln_fwd
    eps = 1e-6 if rms else 1e-5
    ref = fn(d["x"], d["bias"], d["residual"], d["gamma"], d["beta"], eps, want_amax=True)
    x, res = d["x"].clone(), d["residual"].clone()
    out = {"y": x, "residual_out": res} if alias == "y=x,res_out=res" else \
        {"y": res, "residual_out": x}
    got = fn(x, d["bias"], res, d["gamma"], d["beta"], eps, want_amax=True, out=out)
    torch.cuda.synchronize()
    for k in ("y", "residual_out", "rstd", "amax") + (() if rms else ("mean",)):
        assert torch.equal(got[k], ref[k]), k


@pytest.mark.parametrize("case", [c for c in FWD_SHAPES if c[0] == BF16], ids=IDS)
def test_fp8_forward_residual_out_in_place(case):
    dtype, M, N = case
    d = _inputs(dtype, M, N, seed=3 * M + N)
    scale = torch.full((1,), 2.0, device="cuda")
    ref = nf.ln_fwd_fp8(d["x"], scale, d["bias"], d["residual"], d["gamma"], d["beta"],
                        want_amax=True)
    x = d["x"].clone()
    got = nf.ln_fwd_fp8(x, scale, d["bias"], d["residual"], d["gamma"], d["beta"],
                        want_amax=True, out={"residual_out": x})
    torch.cuda.synchronize()
    assert torch.equal(got["y"].view(torch.uint8), ref["y"].view(torch.uint8))
    for k in ("residual_out", "mean", "rstd", "amax"):
        assert torch.equal(got[k], ref[k]), k


@pytest.mark.parametrize("case", BWD_SHAPES, ids=IDS)
@pytest.mark.parametrize("op", ["ln", "rms", "rms-recompute"])
@pytest.mark.parametrize("alias", ["dx=dy", "dx=x"])
def test_backward_in_place(case, op, alias):
    dtype, M, N = case
    d = _inputs(dtype, M, N, seed=5 * M + N)
    f = (nf.rms_fwd if op != "ln" else nf.ln_fwd)(d["x"], None, None, d["gamma"], None, 1e-5)
    pdt = torch.float32

    def run(dy, x, out=None):
        if op == "ln":
            return nf.ln_bwd(dy, x, d["gamma"], f["mean"], f["rstd"], dparam_dtype=pdt,
                             want_dbias=True, out=out)
        rstd = None if op == "rms-recompute" else f["rstd"]
        return nf.rms_bwd(dy, x, d["gamma"], rstd, 1e-5, dparam_dtype=pdt, want_dbeta=True,
                          want_dbias=True, out=out)

    ref = run(d["dy"], d["x"])
    dy, x = d["dy"].clone(), d["x"].clone()
    got = run(dy, x, out={"dx": dy if alias == "dx=dy" else x})
    torch.cuda.synchronize()
    for k in ("dx", "dgamma", "dbeta", "dbias"):
        assert torch.equal(got[k], ref[k]), k


@pytest.mark.parametrize("case", [(BF16, 5000, 384), (BF16, 70000, 384), (BF16, 300, 4096),
                                  (BF16, 77, 1001), (F32, 33, 4096)], ids=IDS)
def test_softmax_in_place(case):
    dtype, M, N = case
    x = _inputs(dtype, M, N, seed=M)["x"]
    ref = nf.softmax_fwd(x)
    y = x.clone()
    got = nf.softmax_fwd(y, out=y)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
