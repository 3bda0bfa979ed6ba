"""GPU parity on randomly drawn configurations (a fixed, seeded list): shape,
dtype, alignment, which optional inputs are present, the options, the amax
path and in-place outputs, for the forward, the FP8 forward, the backward and
softmax.  Each case is compared with the oracle run on the same inputs and
options, with the tolerances of the dedicated tests.  The draw spans 1 to
16384 columns (half of them multiples of 8) and 1 to a few thousand rows, and
so every kind of kernel and walk."""
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

SPECIAL_N = (1, 2, 3, 7, 384, 1001, 4100, 6002, 8191, 12004, 16383, 16384)


def _shape(rng):
    r = rng.random()
    if r < 0.5:
        N = 8 * int(np.exp(rng.uniform(0.0, np.log(2048.0))))
    elif r < 0.8:
        N = int(np.exp(rng.uniform(0.0, np.log(16384.0))))
    else:
        N = int(rng.choice(SPECIAL_N))
    N = max(1, min(N, 16384))
    # at most about 3 million elements, so that the oracle stays quick
    m_max = max(1, min(5000, 3_000_000 // N))
    M = int(np.exp(rng.uniform(0.0, np.log(m_max + 1.0))))
    return max(1, M), N


def _fwd_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M, N = _shape(rng)
        out.append(dict(i=i, M=M, N=N, dtype=BF16 if rng.random() < 0.7 else F32,
                        rms=bool(rng.random() < 0.5), misalign=bool(rng.random() < 0.2),
                        parts=tuple(k for k in ("bias", "residual", "gamma", "beta")
                                    if rng.random() < 0.75),
                        zc=bool(rng.random() < 0.25), amax_ws=bool(rng.random() < 0.5),
                        in_place=bool(rng.random() < 0.25), seed=int(rng.integers(1 << 30))))
    return out


def _bwd_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M, N = _shape(rng)
        rms = bool(rng.random() < 0.5)
        out.append(dict(i=i, M=M, N=N, dtype=BF16 if rng.random() < 0.7 else F32, rms=rms,
                        recompute=rms and bool(rng.random() < 0.5),
                        misalign=bool(rng.random() < 0.2), gamma=bool(rng.random() < 0.85),
                        zc=bool(rng.random() < 0.25), mean=bool(rng.random() < 0.2),
                        dbias=bool(rng.random() < 0.4),
                        pdt=BF16 if rng.random() < 0.5 else F32,
                        in_place=bool(rng.random() < 0.25), seed=int(rng.integers(1 << 30))))
    return out


def _id(c):
    dt = "bf16" if c["dtype"] == BF16 else "f32"
    return f"{c['i']:02d}-{'rms' if c['rms'] else 'ln'}-{dt}-{c['M']}x{c['N']}"


FWD_CASES = _fwd_cases(150, seed=20241)
BWD_CASES = _bwd_cases(150, seed=20242)
FP8_CASES = _fwd_cases(60, seed=20243)
SOFTMAX_CASES = _fwd_cases(60, seed=20244)


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("c", FWD_CASES, ids=_id)
def test_random_forward(c):
    _check_forward(c)


@pytest.mark.parametrize("c", BWD_CASES, ids=_id)
def test_random_backward(c):
    _check_backward(c)


def _walk_knobs(rng, direction):
    """Forced row groups per workgroup, interleave block and write-through
    bytes for the test build (and, backward, the split along N on or off)."""
    env = {f"NORMFUSE_{direction}_GROUPS_PER_WG": str(int(rng.integers(1, 9))),
           f"NORMFUSE_{direction}_INTERLEAVE": str(int(rng.choice([1, 3, 7, 64, 256, 1000]))),
           f"NORMFUSE_{direction}_WT_BYTES": str(int(rng.choice([0, 4096, 1 << 20, 1 << 30])))}
    if direction == "BWD" and rng.random() < 0.5:
        env["NORMFUSE_BWD_SPLIT"] = str(int(rng.integers(0, 2)))
    return env


def _walk_cases(cases, direction, seed):
    rng = np.random.default_rng(seed)
    return [dict(c, env=_walk_knobs(rng, direction)) for c in cases]


FWD_WALK_CASES = _walk_cases(_fwd_cases(60, seed=20245), "FWD", 20246)
BWD_WALK_CASES = _walk_cases(_bwd_cases(60, seed=20247), "BWD", 20248)


@pytest.mark.parametrize("c", FWD_WALK_CASES, ids=_id)
def test_random_forward_walks(c, tuning):
    """The same checks on the test build with the walk forced: row groups per
    workgroup, interleave blocks that need not divide the grid, and where the
    write-through tail starts."""
    for k, v in c["env"].items():
        tuning.setenv(k, v)
    _check_forward(c)


@pytest.mark.parametrize("c", BWD_WALK_CASES, ids=_id)
def test_random_backward_walks(c, tuning):
    """As above for the backward (more or fewer partial rows, the two-level
    column sums, the split along N forced on or off where it applies)."""
    for k, v in c["env"].items():
        tuning.setenv(k, v)
    _check_backward(c)


def _check_forward(c):
    M, N, dtype, rms = c["M"], c["N"], c["dtype"], c["rms"]
    eps = 1e-6 if rms else 1e-5
    inp = synth.make_inputs(M, N, dtype=dtype, seed=c["seed"])
    g = {k: (inp[k] if k == "x" or k in c["parts"] else None)
         for k in ("x", "bias", "residual", "gamma", "beta")}
    dev = {k: to_dev(v, dtype, c["misalign"] and k == "x") if v is not None else None
           for k, v in g.items()}
    fn = nf.rms_fwd if rms else nf.ln_fwd
    ws = nf.amax_workspace() if c["amax_ws"] else None
    out = {}
    if c["in_place"]:
        out["y"] = dev["x"]  # y over x: the call reads each row before writing it
    res = fn(dev["x"], dev["bias"], dev["residual"], dev["gamma"], dev["beta"], eps,
             want_residual_out=True, want_amax=True, zero_centered_gamma=c["zc"],
             amax_workspace=ws, out=out)
    torch.cuda.synchronize()
    ref = oracle.norm_fwd(g["x"], g["bias"], g["residual"], g["gamma"], g["beta"], eps, rms=rms,
                          dtype=dtype, zero_centered_gamma=c["zc"])
    u_gpu = from_dev(res["residual_out"], dtype)
    assert_fused_add_close(u_gpu, ref["u"], g, dtype, "residual_out")
    st = oracle.norm_fwd(u_gpu, None, None, g["gamma"], g["beta"], eps, rms=rms, dtype=dtype,
                         zero_centered_gamma=c["zc"])
    y_gpu = f64(res["y"])
    assert_rows_close(y_gpu, st["y"], dtype, "y (staged)")
    rel = np.abs(f64(res["rstd"]) - st["rstd"]) / st["rstd"]
    assert np.all(rel <= 1e-5), f"rstd: max rel err {rel.max():.3e}"
    if not rms:
        s = np.maximum(np.max(np.abs(synth.to_f64(u_gpu, dtype)), axis=1), 1e-30)
        assert np.all(np.abs(f64(res["mean"]) - st["mean"]) <= 1e-5 * s), "mean"
    brute = float(np.max(np.abs(y_gpu)))
    assert float(res["amax"].item()) == brute, (res["amax"].item(), brute)
    if ws is not None:
        assert torch.count_nonzero(ws).item() == 0, "amax workspace not left zero-filled"


def _check_backward(c):
    M, N, dtype, rms = c["M"], c["N"], c["dtype"], c["rms"]
    eps = 1e-6 if rms else 1e-5
    inp = synth.make_inputs(M, N, dtype=dtype, seed=c["seed"], names=("x", "dy", "gamma"))
    gamma = inp["gamma"] if c["gamma"] else None
    f = oracle.norm_fwd(inp["x"], gamma=gamma, eps=eps, rms=rms, dtype=dtype, want_u=False,
                        want_y=False, zero_centered_gamma=c["zc"])
    mean = None if rms else f["mean"].astype(np.float32)
    rstd = None if c["recompute"] else f["rstd"].astype(np.float32)
    dy = to_dev(inp["dy"], dtype, c["misalign"])
    x = to_dev(inp["x"], dtype)
    g = to_dev(gamma, dtype) if gamma is not None else None
    pdt = TORCH_DT[c["pdt"]]
    out = {"dx": dy} if c["in_place"] else None  # dx over dy
    kw = dict(dparam_dtype=pdt, want_dbias=c["dbias"], zero_centered_gamma=c["zc"],
              dparam_mean=c["mean"], out=out)
    if rms:
        res = nf.rms_bwd(dy, x, g, None if rstd is None else torch.from_numpy(rstd).cuda(), eps,
                         want_dbeta=True, **kw)
    else:
        res = nf.ln_bwd(dy, x, g, torch.from_numpy(mean).cuda(), torch.from_numpy(rstd).cuda(),
                        **kw)
    torch.cuda.synchronize()
    ref = oracle.norm_bwd(inp["dy"], inp["x"], gamma, mean, rstd, eps, rms=rms, dtype=dtype,
                          want_dbias=c["dbias"], zero_centered_gamma=c["zc"],
                          dparam_mean=c["mean"])
    # the weight dx is formed with: gamma, 1 + gamma in the I/O dtype when
    # zero-centred, or 1 when absent
    if gamma is None:
        gam = None
    elif c["zc"]:
        gam = from_dev((g.float() + 1.0).to(TORCH_DT[dtype]), dtype)
    else:
        gam = gamma
    assert_rows_close(f64(res["dx"]), ref["dx"], dtype, "dx",
                      scale=dx_term_scale(inp["dy"], gam, ref["rstd"], dtype))
    for k in ("dgamma", "dbeta"):
        assert_colsums_close(f64(res[k]), ref[k], ref[k + "_l2"], 1e-5, k, dtype=c["pdt"])
    if c["dbias"]:
        l2 = np.maximum(ref["dbias_l2"], dbias_term_l2(inp["dy"], gam, ref["rstd"], dtype)
                        / (M if c["mean"] else 1))
        assert_colsums_close(f64(res["dbias"]), ref["dbias"], l2, 1e-5, "dbias", dtype=c["pdt"])


@pytest.mark.parametrize("c", FP8_CASES, ids=_id)
def test_random_fp8_forward(c):
    """FP8 codes are the E4M3 quantisation of the y the plain forward stores,
    and every other output is that call's, bit for bit."""
    M, N, dtype, rms = c["M"], c["N"], c["dtype"], c["rms"]
    eps = 1e-6 if rms else 1e-5
    inp = synth.make_inputs(M, N, dtype=dtype, seed=c["seed"])
    dev = {k: to_dev(inp[k], dtype, c["misalign"] and k == "x") if k == "x" or k in c["parts"]
           else None for k in ("x", "bias", "residual", "gamma", "beta")}
    plain_fn, fp8_fn = (nf.rms_fwd, nf.rms_fwd_fp8) if rms else (nf.ln_fwd, nf.ln_fwd_fp8)
    plain = plain_fn(dev["x"], dev["bias"], dev["residual"], dev["gamma"], dev["beta"], eps,
                     want_residual_out=True, want_amax=True, zero_centered_gamma=c["zc"])
    torch.cuda.synchronize()
    scale = float(np.float32(448.0 / max(float(plain["amax"].item()), 1e-30)))
    sc = torch.tensor([scale], dtype=torch.float32, device="cuda")
    ws = nf.amax_workspace() if c["amax_ws"] else None
    q = fp8_fn(dev["x"], sc, dev["bias"], dev["residual"], dev["gamma"], dev["beta"], eps,
               want_residual_out=True, want_amax=True, zero_centered_gamma=c["zc"],
               amax_workspace=ws)
    torch.cuda.synchronize()
    for k in ("residual_out", "rstd", "amax") + (() if rms else ("mean",)):
        assert torch.equal(plain[k], q[k]), k
    ref = oracle.quantize_e4m3(plain["y"].float().cpu().numpy(), scale)
    got = q["y"].view(torch.uint8).cpu().numpy()
    assert np.array_equal(got, ref), f"{int(np.sum(got != ref))} FP8 codes differ"


@pytest.mark.parametrize("c", SOFTMAX_CASES, ids=_id)
def test_random_softmax(c):
    M, N, dtype = c["M"], c["N"], c["dtype"]
    x = synth.make_inputs(M, N, dtype=dtype, seed=c["seed"], names=("x",))["x"]
    xd = to_dev(x, dtype, c["misalign"])
    y = nf.softmax_fwd(xd, out=xd if c["in_place"] else None)
    torch.cuda.synchronize()
    assert_rows_close(f64(y), oracle.softmax_fwd(x, dtype=dtype), dtype, "softmax")
