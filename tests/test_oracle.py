"""Pins for the double-precision CPU oracle (runs on the CPU, no GPU).

The pages print no numeric results, so the oracle is pinned by what the
mathematics fixes: closed-form worked examples, exact invariants of the
normalised output and of dx, special cases, central finite differences of
the forward, library routines the pages themselves call (torch's
``layer_norm`` in float64, named in the nvFuser layernorm + amax comment),
brute force, and the distributive identity of nvFuser issue #1660.  Each is
chosen so that a plausible slip in the oracle (a dropped term, a wrong sign,
an N-1 for N, a swapped index) breaks at least one of them; the mutation
test in ``test_oracle_mutants.py`` checks that claim.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F32, BF16 = 0, 1


def f32(a):
    return np.ascontiguousarray(a, np.float32)


def t64(a):
    return torch.from_numpy(np.asarray(a, np.float64).copy())


def dyadic(rng, shape, lo=-512, hi=512, shift=8):
    """Values k * 2^-shift: exact in fp32, and so is v +- 2^-14."""
    return f32(rng.integers(lo, hi + 1, size=shape).astype(np.float64) / 2.0**shift)


# ------------------------------------------------------------ rounding

def test_round_bf16_grid_and_ties(oracle_mod):
    """Every finite bf16 value rounds to itself; a value just above / below a
    midpoint goes to the nearer neighbour; an exact midpoint goes to the
    neighbour whose last bit is 0."""
    bits = np.arange(0, 0x7F80, dtype=np.uint16)           # +0 .. largest finite
    vals = oracle_mod.bf16_bits_to_f64(bits)
    assert np.array_equal(oracle_mod.round_to_dtype(vals, BF16), bits)
    assert np.array_equal(oracle_mod.round_to_dtype(-vals, BF16), bits | np.uint16(0x8000))
    lo, hi = vals[:-1], vals[1:]
    mid = (lo + hi) / 2.0                                   # exact in double
    below = np.nextafter(mid, -np.inf)
    above = np.nextafter(mid, np.inf)
    assert np.array_equal(oracle_mod.round_to_dtype(below, BF16), bits[:-1])
    assert np.array_equal(oracle_mod.round_to_dtype(above, BF16), bits[1:])
    even = np.where(bits[:-1] % 2 == 0, bits[:-1], bits[1:])
    assert np.array_equal(oracle_mod.round_to_dtype(mid, BF16), even)
    # beyond the largest finite value's rounding range -> inf
    assert oracle_mod.round_to_dtype(np.array([2.0**128]), BF16)[0] == 0x7F80


def test_round_bf16_agrees_with_torch_and_generator(oracle_mod):
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.standard_normal(1000) * 1e-39])  # bf16 subnormals too
    v32 = v.astype(np.float32).astype(np.float64)          # fp32 values: no double rounding
    ours = oracle_mod.round_to_dtype(v32, BF16)
    ref = torch.from_numpy(v32.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(ours, ref.view(np.uint16))
    assert np.array_equal(ours, synth.f32_to_bf16_bits(v32.astype(np.float32)))


# ------------------------------------------------------- worked examples

def test_ln_worked_example(oracle_mod):
    """x = [1, 2, 3, 4], eps = 0, gamma = 1, beta = 0: mean 5/2, biased
    variance 5/4, so y = (x - 5/2) / sqrt(5/4) = (2x - 5) / sqrt(5)."""
    x = f32([[1, 2, 3, 4]])
    r = oracle_mod.norm_fwd(x, eps=0.0, dtype=F32)
    s5 = math.sqrt(5.0)
    assert r["mean"][0] == 2.5
    assert abs(r["rstd"][0] - 1.0 / math.sqrt(1.25)) < 1e-15
    np.testing.assert_allclose(r["y"][0], [-3 / s5, -1 / s5, 1 / s5, 3 / s5], rtol=0, atol=1e-15)
    # amax = 3/sqrt(5) = 1.3416..., rounded to fp32
    assert r["amax"] == float(np.float32(3 / s5))


def test_rms_worked_example(oracle_mod):
    """x = [1, 2, 3, 4], eps = 0: mean square 30/4, y = x / sqrt(7.5)."""
    x = f32([[1, 2, 3, 4]])
    r = oracle_mod.norm_fwd(x, eps=0.0, dtype=F32, rms=True)
    assert abs(r["rstd"][0] - 1.0 / math.sqrt(7.5)) < 1e-15
    np.testing.assert_allclose(r["y"][0], np.array([1, 2, 3, 4]) / math.sqrt(7.5), rtol=0,
                               atol=1e-15)


def test_affine_and_fused_add_worked_example(oracle_mod):
    """bias, residual, gamma, beta on a row where everything is exact:
    t = (x + bias) + residual = [1, 3, 5, 7] -> mean 4, var 5, so
    y = (t - 4) / sqrt(5) * gamma + beta."""
    x = f32([[0.5, 1.0, 1.5, 2.0]])
    bias = f32([0.5, 0.5, 0.5, 0.5])
    res = f32([[0.0, 1.5, 3.0, 4.5]])
    gamma = f32([2.0, -1.0, 0.5, 1.0])
    beta = f32([0.25, 0.0, -0.25, 1.0])
    r = oracle_mod.norm_fwd(x, bias, res, gamma, beta, eps=0.0, dtype=F32)
    np.testing.assert_array_equal(r["u"], f32([[1, 3, 5, 7]]))
    s5 = math.sqrt(5.0)
    want = np.array([-3 / s5 * 2 + 0.25, -1 / s5 * -1, 1 / s5 * 0.5 - 0.25, 3 / s5 + 1.0])
    np.testing.assert_allclose(r["y"][0], want, rtol=0, atol=1e-15)


# --------------------------------------------------------- invariants

@pytest.mark.parametrize("eps", [0.0, 1e-5, 0.5])
def test_ln_output_moments(oracle_mod, eps):
    """gamma = 1, beta = 0: every row of y has mean 0 and mean square
    var / (var + eps) (exactly 1 when eps = 0)."""
    rng = np.random.default_rng(1)
    x = f32(rng.standard_normal((37, 129)) * 3 + 1)
    r = oracle_mod.norm_fwd(x, eps=eps, dtype=F32)
    y = r["y"]
    xd = x.astype(np.float64)
    var = xd.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose((y * y).mean(axis=1), var / (var + eps), rtol=1e-12)
    np.testing.assert_allclose(r["mean"], xd.mean(axis=1), rtol=1e-13)


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.5])
def test_rms_output_moments(oracle_mod, eps):
    rng = np.random.default_rng(2)
    x = f32(rng.standard_normal((23, 200)) + 0.5)
    r = oracle_mod.norm_fwd(x, eps=eps, dtype=F32, rms=True)
    ms = (x.astype(np.float64) ** 2).mean(axis=1)
    np.testing.assert_allclose((r["y"] ** 2).mean(axis=1), ms / (ms + eps), rtol=1e-12)
    # y is proportional to x within a row
    np.testing.assert_allclose(r["y"], x * r["rstd"][:, None], rtol=1e-14)


def test_ln_degenerate_rows(oracle_mod):
    """N = 1 and constant rows have zero variance: y = beta, rstd = eps^-1/2."""
    beta1 = f32([0.75])
    r = oracle_mod.norm_fwd(f32([[3.0], [-2.0]]), gamma=f32([5.0]), beta=beta1, eps=0.25,
                            dtype=F32)
    np.testing.assert_array_equal(r["y"], [[0.75], [0.75]])
    np.testing.assert_array_equal(r["rstd"], [2.0, 2.0])
    beta = f32([0.5, -1.0, 2.0])
    r = oracle_mod.norm_fwd(f32([[7.0, 7.0, 7.0]]), gamma=f32([3, 3, 3]), beta=beta, eps=1e-2,
                            dtype=F32)
    np.testing.assert_array_equal(r["y"][0], beta)


def test_empty_matrix(oracle_mod):
    r = oracle_mod.norm_fwd(np.zeros((0, 8), np.uint16), dtype=BF16)
    assert r["amax"] == 0.0 and r["y"].shape == (0, 8)
    b = oracle_mod.norm_bwd(np.zeros((0, 8), np.uint16), np.zeros((0, 8), np.uint16),
                            mean=np.zeros(0), rstd=np.zeros(0), dtype=BF16)
    np.testing.assert_array_equal(b["dgamma"], 0.0)
    np.testing.assert_array_equal(b["dbeta"], 0.0)


# ------------------------------------------- library routine the page calls

@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("rms", [False, True])
def test_forward_matches_torch_float64(oracle_mod, dtype, rms):
    """The nvFuser layernorm + amax comment defines the op as
    out1 = (x + bias) + residual; out2 = layer_norm(out1, w, ln_bias, eps);
    amax = max(abs(out2)).  Reproduce it with torch in float64 (RMSNorm with
    torch's rms_norm), rounding out1 and out2 to the I/O dtype."""
    M, N = 33, 97
    inp = synth.make_inputs(M, N, dtype=dtype, seed=3)
    tdt = torch.float32 if dtype == F32 else torch.bfloat16
    v = {k: t64(synth.to_f64(a, dtype)) for k, a in inp.items()}
    out1 = ((v["x"] + v["bias"]) + v["residual"]).to(tdt).double()
    if rms:
        out2 = F.rms_norm(out1, (N,), v["gamma"], 1e-6) + v["beta"]
    else:
        out2 = F.layer_norm(out1, (N,), v["gamma"], v["beta"], 1e-5)
    amax = torch.amax(torch.abs(out2.to(tdt).double())).item()
    r = oracle_mod.norm_fwd(inp["x"], inp["bias"], inp["residual"], inp["gamma"], inp["beta"],
                            1e-6 if rms else 1e-5, rms=rms, dtype=dtype)
    u = synth.to_f64(r["u"], dtype)
    np.testing.assert_array_equal(u, out1.numpy())
    np.testing.assert_allclose(r["y"], out2.numpy(), rtol=0, atol=1e-12)
    assert r["amax"] == amax
    if not rms:
        _, mean, rstd = torch.ops.aten.native_layer_norm(out1, (N,), None, None, 1e-5)
        np.testing.assert_allclose(r["mean"], mean.view(-1).numpy(), rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(r["rstd"], rstd.view(-1).numpy(), rtol=1e-13)


def test_amax_brute_force(oracle_mod):
    """amax = max over every element of |y rounded to the I/O dtype|."""
    M, N = 64, 50
    inp = synth.make_inputs(M, N, dtype=BF16, seed=4, outlier_p=0.05)
    r = oracle_mod.norm_fwd(inp["x"], inp["bias"], inp["residual"], inp["gamma"], inp["beta"],
                            1e-5, dtype=BF16)
    y_stored = oracle_mod.bf16_bits_to_f64(oracle_mod.round_to_dtype(r["y"], BF16))
    best = 0.0
    for i in range(M):
        for j in range(N):
            best = max(best, abs(float(y_stored[i, j])))
    assert r["amax"] == best


# --------------------------------------------------------------- backward

def _fd_grads(oracle_mod, x, gamma, beta, dy, eps, rms, h):
    """Central differences of L = sum(dy * y(x, gamma, beta)) with step h;
    all perturbed inputs are exactly representable in fp32."""
    def loss(xx, gg, bb):
        r = oracle_mod.norm_fwd(f32(xx), gamma=f32(gg), beta=f32(bb), eps=eps, rms=rms, dtype=F32)
        return float(np.sum(dy * r["y"]))

    def grad(arr, which):
        g = np.zeros(arr.shape)
        for idx in np.ndindex(arr.shape):
            hi = arr.astype(np.float64).copy()
            lo = hi.copy()
            hi[idx] += h
            lo[idx] -= h
            args_hi = [x, gamma, beta]
            args_lo = [x, gamma, beta]
            args_hi[which], args_lo[which] = hi, lo
            g[idx] = (loss(*args_hi) - loss(*args_lo)) / (2 * h)
        return g

    return grad(x, 0), grad(gamma, 1), grad(beta, 2)


@pytest.mark.parametrize("rms", [False, True])
@pytest.mark.parametrize("N", [1, 2, 3, 7, 8, 17])
@pytest.mark.parametrize("eps", [1e-5, 0.05])
def test_backward_finite_differences(oracle_mod, rms, N, eps):
    rng = np.random.default_rng(100 + N)
    M = 3
    x = dyadic(rng, (M, N))
    x[0] += f32(0.5)   # a row off-centre
    gamma = dyadic(rng, (N,), 64, 384)
    beta = dyadic(rng, (N,))
    dy = rng.standard_normal((M, N))
    fwd = oracle_mod.norm_fwd(x, gamma=gamma, beta=beta, eps=eps, rms=rms, dtype=F32)
    # the backward reads dy / x / gamma in the I/O dtype; feed dy as fp32
    dy32 = f32(dy)
    b = oracle_mod.norm_bwd(dy32, x, gamma, None if rms else fwd["mean"], fwd["rstd"], eps,
                            rms=rms, dtype=F32)
    # Richardson extrapolation of two central differences: O(h^4) error
    h1, h2 = 2.0**-10, 2.0**-11
    g1 = _fd_grads(oracle_mod, x, gamma, beta, dy32.astype(np.float64), eps, rms, h1)
    g2 = _fd_grads(oracle_mod, x, gamma, beta, dy32.astype(np.float64), eps, rms, h2)
    fd = [(4 * b2 - b1) / 3 for b1, b2 in zip(g1, g2)]
    scale = max(1.0, float(np.max(np.abs(fwd["rstd"]))))
    np.testing.assert_allclose(b["dx"], fd[0], rtol=0, atol=2e-8 * scale)
    np.testing.assert_allclose(b["dgamma"], fd[1], rtol=0, atol=2e-8 * scale)
    np.testing.assert_allclose(b["dbeta"], fd[2], rtol=0, atol=2e-8)


@pytest.mark.parametrize("rms", [False, True])
def test_backward_matches_autograd_float64(oracle_mod, rms):
    M, N = 19, 77
    rng = np.random.default_rng(7)
    x = f32(rng.standard_normal((M, N)) * 2 + 0.3)
    gamma = f32(1 + 0.1 * rng.standard_normal(N))
    beta = f32(0.1 * rng.standard_normal(N))
    dy = f32(rng.standard_normal((M, N)))
    eps = 1e-6 if rms else 1e-5
    xt = t64(x).requires_grad_()
    gt = t64(gamma).requires_grad_()
    bt = t64(beta).requires_grad_()
    y = (F.rms_norm(xt, (N,), gt, eps) + bt) if rms else F.layer_norm(xt, (N,), gt, bt, eps)
    (y * t64(dy)).sum().backward()
    fwd = oracle_mod.norm_fwd(x, gamma=gamma, beta=beta, eps=eps, rms=rms, dtype=F32)
    b = oracle_mod.norm_bwd(dy, x, gamma, None if rms else fwd["mean"],
                            None if rms else fwd["rstd"], eps, rms=rms, dtype=F32)
    np.testing.assert_allclose(b["dx"], xt.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(b["dgamma"], gt.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(b["dbeta"], bt.grad.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("rms", [False, True])
@pytest.mark.parametrize("N", [1, 3, 8, 17])
def test_dbias_finite_differences(oracle_mod, rms, N):
    """dbias = dL/dbias for L = sum(dy * y(x + bias + residual)): central
    differences in bias through the oracle forward (fp32 I/O; every perturbed
    sum is exact in fp32), Richardson-extrapolated."""
    rng = np.random.default_rng(300 + N)
    M, eps = 4, 0.02
    x = dyadic(rng, (M, N))
    res = dyadic(rng, (M, N))
    bias = dyadic(rng, (N,))
    gamma = dyadic(rng, (N,), 64, 384)
    beta = dyadic(rng, (N,))
    dy = f32(rng.standard_normal((M, N)))
    fwd = oracle_mod.norm_fwd(x, bias, res, gamma, beta, eps, rms=rms, dtype=F32)
    b = oracle_mod.norm_bwd(dy, fwd["u"], gamma, None if rms else fwd["mean"], fwd["rstd"], eps,
                            rms=rms, dtype=F32, want_dbias=True)

    def loss(bb):
        r = oracle_mod.norm_fwd(x, f32(bb), res, gamma, beta, eps, rms=rms, dtype=F32)
        return float(np.sum(dy.astype(np.float64) * r["y"]))

    def fd(h):
        g = np.zeros(N)
        for j in range(N):
            hi = bias.astype(np.float64).copy()
            lo = hi.copy()
            hi[j] += h
            lo[j] -= h
            g[j] = (loss(hi) - loss(lo)) / (2 * h)
        return g

    est = (4 * fd(2.0**-11) - fd(2.0**-10)) / 3
    scale = max(1.0, float(np.max(fwd["rstd"])))
    np.testing.assert_allclose(b["dbias"], est, rtol=0, atol=4e-8 * scale * M)


@pytest.mark.parametrize("rms", [False, True])
def test_dbias_matches_autograd_float64(oracle_mod, rms):
    """The gradient of the bias through u = (x + bias) + residual, by float64
    autograd (x, residual and bias dyadic, so u is exact in fp32)."""
    M, N = 13, 40
    rng = np.random.default_rng(11)
    x, res, bias = dyadic(rng, (M, N)), dyadic(rng, (M, N)), dyadic(rng, (N,))
    gamma = f32(1 + 0.1 * rng.standard_normal(N))
    beta = f32(0.1 * rng.standard_normal(N))
    dy = f32(rng.standard_normal((M, N)))
    eps = 1e-6 if rms else 1e-5
    bt = t64(bias).requires_grad_()
    u = t64(x) + bt + t64(res)
    y = (F.rms_norm(u, (N,), t64(gamma), eps) + t64(beta)) if rms else \
        F.layer_norm(u, (N,), t64(gamma), t64(beta), eps)
    (y * t64(dy)).sum().backward()
    fwd = oracle_mod.norm_fwd(x, bias, res, gamma, beta, eps, rms=rms, dtype=F32)
    assert np.array_equal(fwd["u"].astype(np.float64), u.detach().numpy())
    b = oracle_mod.norm_bwd(dy, fwd["u"], gamma, None if rms else fwd["mean"],
                            None if rms else fwd["rstd"], eps, rms=rms, dtype=F32,
                            want_dbias=True)
    np.testing.assert_allclose(b["dbias"], bt.grad.numpy(), rtol=1e-10, atol=1e-10)


def test_dbias_layernorm_sums_to_zero(oracle_mod):
    """LayerNorm's dx sums to zero over every row, so the column sums of dx
    (dbias) sum to zero over the columns; their 2-norm scale is the root of
    the column sums of dx^2."""
    M, N = 37, 96
    inp = synth.make_inputs(M, N, dtype=BF16, seed=12, names=("x", "gamma", "dy"))
    fwd = oracle_mod.norm_fwd(inp["x"], eps=1e-5, dtype=BF16)
    b = oracle_mod.norm_bwd(inp["dy"], inp["x"], inp["gamma"], fwd["mean"], fwd["rstd"], 1e-5,
                            want_dbias=True)
    assert abs(float(np.sum(b["dbias"]))) <= 1e-10 * float(np.sum(b["dbias_l2"]))
    np.testing.assert_allclose(b["dbias_l2"], np.sqrt(np.sum(b["dx"] ** 2, axis=0)), rtol=1e-12)
    c = oracle_mod.norm_bwd(inp["dy"], inp["x"], inp["gamma"], fwd["mean"], fwd["rstd"], 1e-5,
                            want_dbias=True, want_dx=False)
    assert np.array_equal(c["dbias"], b["dbias"])


@pytest.mark.parametrize("rms", [False, True])
def test_dx_row_invariants(oracle_mod, rms):
    """LayerNorm: sum_j dx_j = 0 and sum_j dx_j xhat_j = eps rstd^3 sum_j g_j xhat_j.
    RMSNorm: sum_j dx_j x_j = eps rstd^3 sum_j g_j x_j (g = dy * gamma)."""
    M, N = 11, 64
    eps = 0.01
    inp = synth.make_inputs(M, N, dtype=F32, seed=8, names=("x", "gamma", "dy"))
    x, gamma, dy = inp["x"], inp["gamma"], inp["dy"]
    fwd = oracle_mod.norm_fwd(x, eps=eps, rms=rms, dtype=F32)
    b = oracle_mod.norm_bwd(dy, x, gamma, fwd["mean"], fwd["rstd"], eps, rms=rms, dtype=F32)
    xd, dyd, gd = (a.astype(np.float64) for a in (x, dy, gamma))
    g = dyd * gd
    r = fwd["rstd"][:, None]
    if rms:
        lhs = (b["dx"] * xd).sum(1)
        rhs = eps * r[:, 0] ** 3 * (g * xd).sum(1)
    else:
        np.testing.assert_allclose(b["dx"].sum(1), 0.0, atol=1e-12)
        xhat = (xd - fwd["mean"][:, None]) * r
        lhs = (b["dx"] * xhat).sum(1)
        rhs = eps * r[:, 0] ** 3 * (g * xhat).sum(1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-9, atol=1e-12)


def test_dx_special_cases(oracle_mod):
    """LayerNorm with gamma = 1: dy constant along a row gives dx = 0, and
    with eps = 0, dy = xhat (a pure rescale of the row) gives dx = 0."""
    rng = np.random.default_rng(9)
    M, N = 5, 24
    x = dyadic(rng, (M, N))
    fwd = oracle_mod.norm_fwd(x, eps=1e-5, dtype=F32)
    dy = f32(np.repeat(rng.standard_normal((M, 1)), N, axis=1))
    b = oracle_mod.norm_bwd(dy, x, None, fwd["mean"], fwd["rstd"], 1e-5, dtype=F32)
    np.testing.assert_allclose(b["dx"], 0.0, atol=1e-12)
    fwd0 = oracle_mod.norm_fwd(x, eps=0.0, dtype=F32)
    xhat = f32(fwd0["y"])   # y = xhat when gamma = 1, beta = 0
    b = oracle_mod.norm_bwd(xhat, x, None, fwd0["mean"], fwd0["rstd"], 0.0, dtype=F32)
    np.testing.assert_allclose(b["dx"], 0.0, atol=1e-6)  # xhat was rounded to fp32


def test_column_sums_brute_force_and_additivity(oracle_mod):
    """dgamma_j = sum_i dy_ij xhat_ij, dbeta_j = sum_i dy_ij by explicit
    loops, and the column sums over rows [0, M) equal the sums over
    [0, M1) plus [M1, M)."""
    M, N = 30, 9
    inp = synth.make_inputs(M, N, dtype=BF16, seed=10, names=("x", "gamma", "dy"))
    fwd = oracle_mod.norm_fwd(inp["x"], eps=1e-5, dtype=BF16)
    b = oracle_mod.norm_bwd(inp["dy"], inp["x"], inp["gamma"], fwd["mean"], fwd["rstd"], 1e-5)
    x = synth.to_f64(inp["x"], BF16)
    dy = synth.to_f64(inp["dy"], BF16)
    for j in range(N):
        sg = sb = 0.0
        for i in range(M):
            xh = (x[i, j] - fwd["mean"][i]) * fwd["rstd"][i]
            sg += dy[i, j] * xh
            sb += dy[i, j]
        assert abs(b["dgamma"][j] - sg) <= 1e-12 * max(1.0, abs(sg))
        assert abs(b["dbeta"][j] - sb) <= 1e-12 * max(1.0, abs(sb))
    M1 = 13
    p1 = oracle_mod.norm_bwd(inp["dy"][:M1], inp["x"][:M1], inp["gamma"], fwd["mean"][:M1],
                             fwd["rstd"][:M1], 1e-5)
    p2 = oracle_mod.norm_bwd(inp["dy"][M1:], inp["x"][M1:], inp["gamma"], fwd["mean"][M1:],
                             fwd["rstd"][M1:], 1e-5)
    np.testing.assert_allclose(p1["dgamma"] + p2["dgamma"], b["dgamma"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(p1["dbeta"] + p2["dbeta"], b["dbeta"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(b["dbeta_l2"], np.sqrt((dy ** 2).sum(0)), rtol=1e-12)
    # dgamma_l2 (the scale every dgamma comparison divides by) is the 2-norm
    # of the terms dy_ij xhat_ij that dgamma_j adds, by explicit loops
    for j in range(N):
        q = 0.0
        for i in range(M):
            t = dy[i, j] * (x[i, j] - fwd["mean"][i]) * fwd["rstd"][i]
            q += t * t
        assert abs(b["dgamma_l2"][j] - math.sqrt(q)) <= 1e-12 * math.sqrt(q)
    # and it bounds the sum it scales: |dgamma_j| <= sqrt(M) * dgamma_l2_j
    assert np.all(np.abs(b["dgamma"]) <= math.sqrt(M) * b["dgamma_l2"] * (1 + 1e-12))


def test_column_l2_scales_of_rank_one_terms(oracle_mod):
    """Closed forms of the 2-norm scales: with dy_ij = a_i (the same value
    across a row) the terms of dbeta_j are a_i, so dbeta_l2_j = ||a||_2 for
    every j; and with gamma = 1 and dy = xhat (LayerNorm, eps = 0 on rows of
    nonzero variance) the terms of dgamma_j are xhat_ij^2, so dgamma_l2_j^2 =
    sum_i xhat_ij^4."""
    M, N = 12, 8
    rng = np.random.default_rng(23)
    x = dyadic(rng, (M, N))
    a = dyadic(rng, (M,), -64, 64, 4)
    dy = f32(np.broadcast_to(a[:, None], (M, N)))
    fwd = oracle_mod.norm_fwd(x, eps=0.0, dtype=F32)
    b = oracle_mod.norm_bwd(dy, x, None, fwd["mean"], fwd["rstd"], 0.0, dtype=F32)
    np.testing.assert_allclose(b["dbeta_l2"], np.linalg.norm(a.astype(np.float64)), rtol=1e-14)
    xh = (x.astype(np.float64) - fwd["mean"][:, None]) * fwd["rstd"][:, None]
    dy2 = f32(xh)
    b2 = oracle_mod.norm_bwd(dy2, x, None, fwd["mean"], fwd["rstd"], 0.0, dtype=F32)
    t = dy2.astype(np.float64) * xh
    np.testing.assert_allclose(b2["dgamma_l2"], np.sqrt((t ** 2).sum(0)), rtol=1e-13)
    # every term dy * xhat is within fp32 rounding of xhat^2 >= 0, so the sum
    # and the 2-norm scale of dgamma meet the norm inequalities of
    # nonnegative terms: l2 <= sum <= sqrt(M) l2
    assert np.all(b2["dgamma_l2"] <= b2["dgamma"] * (1 + 1e-6))
    assert np.all(b2["dgamma"] <= math.sqrt(M) * b2["dgamma_l2"] * (1 + 1e-12))


def test_distributive_identity_on_column_sums(oracle_mod):
    """nvFuser issue #1660, opening comment and its repro: for x of shape
    (8, 4, 1) and b of shape (8, 1, 4), sum(x, 1) * sum(b, 1) equals
    sum(x * b, 1).  On the outer (column) reduction of the backward this is:
    with dy_ij = a_i * c_j (a rank-1, broadcast product) over 4 rows and 4
    columns, dbeta_j = (sum_i a_i) * c_j and dgamma_j = c_j * sum_i a_i xhat_ij.
    Run on the repro's 8 independent (4 x 4) problems."""
    with open(os.path.join(GOLDEN, "distributive_broadcast.json")) as fh:
        g = json.load(fh)
    B, R, _ = g["x_shape"]
    _, _, C = g["b_shape"]
    rng = np.random.default_rng(11)
    for k in range(B):
        a = dyadic(rng, (R,), -64, 64, 4)
        c = dyadic(rng, (C,), -64, 64, 4)
        dy = f32(np.outer(a.astype(np.float64), c))      # exact in fp32
        x = dyadic(rng, (R, C))
        fwd = oracle_mod.norm_fwd(x, eps=1e-5, dtype=F32)
        b = oracle_mod.norm_bwd(dy, x, None, fwd["mean"], fwd["rstd"], 1e-5, dtype=F32)
        lhs = a.astype(np.float64).sum() * c.astype(np.float64)
        np.testing.assert_allclose(b["dbeta"], lhs, rtol=0, atol=1e-12)
        xhat = fwd["y"]
        want = c * (a[:, None] * xhat).sum(0)
        np.testing.assert_allclose(b["dgamma"], want, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ threading

def test_thread_count_does_not_change_results(oracle_mod):
    M, N = 301, 45
    inp = synth.make_inputs(M, N, dtype=BF16, seed=12, names=("x", "residual", "bias", "gamma",
                                                               "beta", "dy"))
    outs = []
    for t in (1, 3, 8):
        f = oracle_mod.norm_fwd(inp["x"], inp["bias"], inp["residual"], inp["gamma"],
                                inp["beta"], 1e-5, nthreads=t)
        b = oracle_mod.norm_bwd(inp["dy"], f["u"], inp["gamma"], f["mean"], f["rstd"], 1e-5,
                                nthreads=t)
        outs.append((f, b))
    for f, b in outs[1:]:
        for k in ("u", "y", "mean", "rstd"):
            assert np.array_equal(f[k], outs[0][0][k])
        assert f["amax"] == outs[0][0]["amax"]
        for k in ("dx", "dgamma", "dbeta"):
            assert np.array_equal(b[k], outs[0][1][k])


def test_rms_backward_recomputes_rstd(oracle_mod):
    """RMSNorm backward with rstd = None recomputes rstd from x and eps and
    matches the backward given the forward's rstd."""
    inp = synth.make_inputs(40, 33, dtype=BF16, seed=13, names=("x", "gamma", "dy"))
    f = oracle_mod.norm_fwd(inp["x"], eps=1e-6, rms=True)
    a = oracle_mod.norm_bwd(inp["dy"], inp["x"], inp["gamma"], None, None, 1e-6, rms=True)
    b = oracle_mod.norm_bwd(inp["dy"], inp["x"], inp["gamma"], None, f["rstd"], 1e-6, rms=True)
    for k in ("dx", "dgamma"):
        np.testing.assert_array_equal(a[k], b[k])


def test_bad_arguments_are_rejected(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.norm_fwd(np.zeros((2, 3), np.uint16), eps=-1.0)
    with pytest.raises(ValueError):
        oracle_mod.norm_bwd(np.zeros((2, 3), np.uint16), np.zeros((2, 3), np.uint16))  # no stats


# ------------------------------------------------------------ FP8 output

def _e4m3_values():
    """Every finite OCP E4M3 value, by code (sign, 4-bit exponent bias 7,
    3-bit mantissa; exponent field 0 is subnormal k * 2^-9)."""
    vals = {}
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        v = m * 2.0**-9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        vals[c] = -v if s else v
    return vals


def test_e4m3_matches_torch_cast(oracle_mod):
    vals = _e4m3_values()
    pos = sorted(v for c, v in vals.items() if c < 128)
    probe = [v for v in vals.values()]
    for lo, hi in zip(pos, pos[1:]):
        mid = np.float32((lo + hi) / 2)
        probe += [mid, np.nextafter(mid, np.float32(1e30)), np.nextafter(mid, np.float32(-1e30))]
    rng = np.random.default_rng(13)
    probe += list(rng.uniform(-448, 448, 20000)) + list(rng.uniform(-0.02, 0.02, 20000))
    v = f32(probe)
    v = np.concatenate([v, -v])
    got = oracle_mod.quantize_e4m3(v, 1.0)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_e4m3_fixed_codes_saturation_and_nan(oracle_mod):
    cases = {1.0: 0x38, -1.0: 0xB8, 448.0: 0x7E, -448.0: 0xFE, 2.0**-6: 0x08, 2.0**-9: 0x01,
             0.0: 0x00, 449.0: 0x7E, 464.0: 0x7E, 1e9: 0x7E, -3e38: 0xFE, 2.0**-11: 0x00,
             1.5 * 2.0**-10: 0x01, 0.1: 0x1D}
    v = f32(list(cases))
    got = oracle_mod.quantize_e4m3(v, 1.0)
    assert [int(g) for g in got] == list(cases.values())
    assert int(oracle_mod.quantize_e4m3(f32([np.nan]), 1.0)[0]) & 0x7F == 0x7F
    assert int(oracle_mod.quantize_e4m3(f32([-0.0]), 1.0)[0]) == 0x80


def test_e4m3_scale_applies_in_fp32(oracle_mod):
    """The code is that of the fp32 product v * scale."""
    # (1.0625 - 2^-23) * (1 + 2^-23) is 1.0625 + 2^-27 - 2^-46 exactly, which
    # fp32 rounds to 1.0625, the midpoint of codes 0x38 (1.0) and 0x39
    # (1.125): the tie goes to the even code; the exact product would round up
    v = f32([1.0625 - 2.0**-23])
    assert int(oracle_mod.quantize_e4m3(v, np.float32(1 + 2.0**-23))[0]) == 0x38
    rng = np.random.default_rng(14)
    v = f32(rng.standard_normal(5000) * 3)
    for scale in (1.0, 0.37, 57.5, 3.1e-3):
        p = v * np.float32(scale)
        ref = torch.from_numpy(np.clip(p, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8)
        assert np.array_equal(oracle_mod.quantize_e4m3(v, scale), ref.numpy())


# ----------------------------------------------- zero-centred gamma, mean

@pytest.mark.parametrize("rms", [False, True])
@pytest.mark.parametrize("dtype", [BF16, F32])
def test_zero_centered_gamma_matches_torch(oracle_mod, rms, dtype):
    """w = 1 + gamma formed by torch in the I/O dtype, then the float64
    normalisation with that weight (the nvFuser comment's expression)."""
    M, N = 9, 50
    inp = synth.make_inputs(M, N, dtype=dtype, seed=15, names=("x", "gamma", "beta"))
    tdt = torch.bfloat16 if dtype == BF16 else torch.float32
    def t_of(a):
        return (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if dtype == BF16
                else torch.from_numpy(a))
    # a zero-centred weight ~ 0.1 * N(0,1), finer than the I/O dtype's
    # spacing near 1, so that forming 1 + gamma rounds
    gamma = synth.make_inputs(1, N, dtype=dtype, seed=19, names=("beta",))["beta"]
    g0 = t_of(gamma)
    assert dtype == F32 or bool(((1 + g0).double() != 1 + g0.double()).any())
    w = (1 + g0).to(torch.float64)
    x, beta = t_of(inp["x"]).to(torch.float64), t_of(inp["beta"]).to(torch.float64)
    eps = 1e-5
    ref = (F.rms_norm(x, (N,), w, eps) + beta) if rms else F.layer_norm(x, (N,), w, beta, eps)
    r = oracle_mod.norm_fwd(inp["x"], gamma=gamma, beta=inp["beta"], eps=eps, rms=rms,
                            dtype=dtype, zero_centered_gamma=True)
    np.testing.assert_allclose(r["y"], ref.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("rms", [False, True])
def test_zero_centered_gamma_backward_autograd(oracle_mod, rms):
    """dx and dgamma through w = 1 + gamma (gamma chosen so that 1 + gamma
    is exact in fp32; autograd in float64)."""
    M, N = 7, 33
    rng = np.random.default_rng(16)
    x = f32(rng.standard_normal((M, N)))
    gamma = dyadic(rng, (N,), -40, 40, 8)
    dy = f32(rng.standard_normal((M, N)))
    eps = 1e-5
    gt = t64(gamma).requires_grad_()
    xt = t64(x).requires_grad_()
    w = 1 + gt
    y = F.rms_norm(xt, (N,), w, eps) if rms else F.layer_norm(xt, (N,), w, None, eps)
    (y * t64(dy)).sum().backward()
    f = oracle_mod.norm_fwd(x, gamma=gamma, eps=eps, rms=rms, dtype=F32,
                            zero_centered_gamma=True)
    b = oracle_mod.norm_bwd(dy, x, gamma, None if rms else f["mean"], f["rstd"], eps, rms=rms,
                            dtype=F32, zero_centered_gamma=True)
    np.testing.assert_allclose(b["dx"], xt.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(b["dgamma"], gt.grad.numpy(), rtol=1e-11, atol=1e-11)


def test_dparam_mean_divides_by_rows(oracle_mod):
    """With dy constant c_j down every column, dbeta's row mean is c_j
    exactly; every mean is the sum over the M rows divided by M."""
    M, N = 24, 16
    rng = np.random.default_rng(17)
    inp = synth.make_inputs(M, N, dtype=F32, seed=18, names=("x", "gamma"))
    c = dyadic(rng, (N,))
    dy = f32(np.broadcast_to(c, (M, N)))
    f = oracle_mod.norm_fwd(inp["x"], eps=1e-5, dtype=F32)
    s = oracle_mod.norm_bwd(dy, inp["x"], inp["gamma"], f["mean"], f["rstd"], 1e-5, dtype=F32,
                            want_dbias=True)
    m = oracle_mod.norm_bwd(dy, inp["x"], inp["gamma"], f["mean"], f["rstd"], 1e-5, dtype=F32,
                            want_dbias=True, dparam_mean=True)
    np.testing.assert_array_equal(m["dbeta"], c.astype(np.float64))
    for k in ("dgamma", "dbeta", "dbias", "dgamma_l2", "dbeta_l2", "dbias_l2"):
        np.testing.assert_allclose(m[k], s[k] / M, rtol=1e-15, atol=0)
    np.testing.assert_array_equal(m["dx"], s["dx"])


# ------------------------------------------------------------- softmax

@pytest.mark.parametrize("dtype", [BF16, F32])
def test_softmax_matches_torch_and_sums_to_one(oracle_mod, dtype):
    M, N = 21, 67
    inp = synth.make_inputs(M, N, dtype=dtype, seed=20, names=("x",))
    y = oracle_mod.softmax_fwd(inp["x"], dtype=dtype)
    xd = synth.to_f64(inp["x"], dtype)
    ref = torch.softmax(t64(xd), dim=1).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(y.sum(1), 1.0, rtol=0, atol=1e-14)


def test_softmax_closed_forms(oracle_mod):
    # two elements: y0 = 1 / (1 + e^(b - a))
    x = f32([[1.5, -0.25], [0.0, 0.0], [3.0, 3.0]])
    y = oracle_mod.softmax_fwd(x, dtype=F32)
    np.testing.assert_allclose(y[0, 0], 1.0 / (1.0 + math.exp(-1.75)), rtol=1e-15)
    np.testing.assert_array_equal(y[1], [0.5, 0.5])
    # a constant row is uniform: 1 / N
    c = f32(np.full((2, 10), -7.25))
    np.testing.assert_allclose(oracle_mod.softmax_fwd(c, dtype=F32), 0.1, rtol=1e-15)


def test_softmax_shift_invariance_and_large_offsets(oracle_mod):
    rng = np.random.default_rng(21)
    x = dyadic(rng, (6, 40))
    y0 = oracle_mod.softmax_fwd(x, dtype=F32)
    for c in (1000.0, -1000.0, 60000.0):
        y = oracle_mod.softmax_fwd(f32(x + np.float32(c)), dtype=F32)
        np.testing.assert_allclose(y, y0, rtol=1e-12, atol=1e-300)
