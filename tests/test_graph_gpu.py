"""The path under HIP graph capture: a forward + backward step (amax reset
kernel or the amax workspace, forward, backward stage 1, column sums)
captured once with torch.cuda.graph on a side stream and replayed several
times, with eager work and synchronisations between the replays; every
replay must equal the eager result bit for bit, and the amax workspace must
be zero-filled after each."""
import numpy as np
import pytest
import torch

import normalization_ln_fwd_amd as nf
import synth
from gpu_util import BF16, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("M,N,amax_ws", [(20000, 384, False), (512, 4096, False),
                                         (20000, 384, True), (512, 4096, True)],
                         ids=["20000x384", "512x4096", "20000x384-amax-ws", "512x4096-amax-ws"])
def test_captured_step_replays_match_eager(M, N, amax_ws):
    inp = synth.make_inputs(M, N, dtype=BF16, seed=31,
                            names=("x", "residual", "bias", "gamma", "beta", "dy"))
    d = {k: to_dev(v, BF16) for k, v in inp.items()}
    ws = torch.empty(max(16, nf.bwd_workspace_size(M, N, torch.bfloat16)), dtype=torch.uint8,
                     device="cuda")
    fo = {"y": torch.empty_like(d["x"]), "residual_out": torch.empty_like(d["x"]),
          "mean": torch.empty(M, device="cuda"), "rstd": torch.empty(M, device="cuda"),
          "amax": torch.empty(1, device="cuda")}
    bo = {"dx": torch.empty_like(d["x"]),
          "dgamma": torch.empty(N, dtype=torch.bfloat16, device="cuda"),
          "dbeta": torch.empty(N, dtype=torch.bfloat16, device="cuda"),
          "dbias": torch.empty(N, dtype=torch.bfloat16, device="cuda")}

    aws = nf.amax_workspace() if amax_ws else None

    def step():
        nf.ln_fwd(d["x"], d["bias"], d["residual"], d["gamma"], d["beta"], 1e-5, want_amax=True,
                  amax_workspace=aws, out=fo)
        nf.ln_bwd(d["dy"], fo["residual_out"], d["gamma"], fo["mean"], fo["rstd"],
                  dparam_dtype=torch.bfloat16, want_dbias=True, workspace=ws, out=bo)

    step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in {**fo, **bo}.items()}

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for rep in range(4):
        for t in list(fo.values()) + list(bo.values()):
            t.fill_(7)  # eager work between replays; outputs must be rewritten
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in {**fo, **bo}.items():
            assert torch.equal(v, eager[k]), (rep, k)
        if aws is not None:
            assert torch.count_nonzero(aws).item() == 0, rep
