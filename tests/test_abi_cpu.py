"""The C ABI on the CPU: the library loads, exports what include/normfuse.h
declares, and rejects bad arguments before touching a device.

No call here reaches a kernel launch: every call has exactly one fault that
the argument checks catch first (fake pointers are never dereferenced).  The
one check of a fault-free call (NORM_ERR_DEVICE) runs only where no GPU is
visible.
"""
import ctypes
import math
import os
import re

import pytest

import normalization_ln_fwd_amd as nf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "normfuse.h")

# Fake, suitably aligned device addresses; never dereferenced.
P = 0x7F0000000000
BAD2 = P + 2    # aligned to 2, not 4
BAD1 = P + 1    # not aligned to 2


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(\w+)\s*\(", text, re.M)) - {"if"})


def header_defines():
    text = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"#define\s+(NORM_\w+)\s+(\d+)", text)}


@pytest.fixture(scope="module")
def lib():
    # NORMFUSE_TEST_LIB: run these checks on another build of the library
    # (the sanitizer test's host-instrumented build)
    path = os.environ.get("NORMFUSE_TEST_LIB")
    try:
        if path:
            nf._lib = nf.load(path)
        return nf.library()
    except nf.NormLibraryMissing as e:
        pytest.fail(str(e))


def test_exports_every_declared_function(lib):
    funcs = header_functions()
    assert set(funcs) == set(nf.EXPORTS), funcs
    for name in funcs:
        assert hasattr(lib, name), name


def test_binding_constants_match_header():
    d = header_defines()
    for op, code in nf.OPS.items():
        assert d["NORM_OP_" + op.replace("_fwd", "_FWD").replace("_bwd", "_BWD")
                 .replace("softmax_FWD", "SOFTMAX").upper()] == code
    assert (d["NORM_DESCRIBE_AMAX"], d["NORM_DESCRIBE_FP8"], d["NORM_DESCRIBE_DBIAS"],
            d["NORM_DESCRIBE_AMAX_WS"]) == \
        (nf.DESCRIBE_AMAX, nf.DESCRIBE_FP8, nf.DESCRIBE_DBIAS, nf.DESCRIBE_AMAX_WS)
    assert d["NORM_AMAX_WS_BYTES"] == nf.AMAX_WS_BYTES
    assert d["NORM_F32"] == nf.F32 and d["NORM_BF16"] == nf.BF16
    assert d["NORM_N_MAX"] == nf.N_MAX
    for code, name in nf.STATUS.items():
        assert d[name] == code


def test_status_strings(lib):
    for code in list(nf.STATUS) + [99]:
        s = lib.norm_status_string(code).decode()
        assert s and isinstance(s, str)
    assert lib.norm_status_string(0).decode() == "ok"


def fwd_args(**over):
    a = dict(x=P, bias=None, residual=None, gamma=P, beta=P, eps=1e-5, M=4, N=64, dtype=1,
             y=P, residual_out=None, mean=P, rstd=P, amax=None, amax_ws=None, flags=0,
             stream=None)
    a.update(over)
    return [a[k] for k in ("x", "bias", "residual", "gamma", "beta", "eps", "M", "N", "dtype",
                           "y", "residual_out", "mean", "rstd", "amax", "amax_ws", "flags",
                           "stream")]


@pytest.mark.parametrize("fn", ["ln_fwd", "rms_fwd"])
@pytest.mark.parametrize("over,code", [
    (dict(dtype=2), 4), (dict(dtype=-1), 4),
    (dict(x=None), 1), (dict(y=None), 1),
    (dict(M=-1), 2), (dict(N=0), 2), (dict(N=16385), 2), (dict(N=-5), 2),
    (dict(M=2**62), 2),
    (dict(eps=-1e-3), 3), (dict(eps=math.nan), 3), (dict(eps=math.inf), 3),
    (dict(x=BAD1), 5), (dict(gamma=BAD1), 5), (dict(y=BAD1), 5),
    (dict(dtype=0, x=BAD2), 5), (dict(dtype=0, residual=BAD2), 5),
    (dict(rstd=BAD2), 5), (dict(amax=BAD2), 5), (dict(amax=P, amax_ws=BAD2), 5),
])
def test_forward_rejects(lib, fn, over, code):
    if fn == "rms_fwd":
        over = dict(over, mean=None)
    assert getattr(lib, fn)(*fwd_args(**over)) == code


def test_no_rows_allows_null_row_tensors(lib):
    # validation passes (M = 0, NULL x / y), so the call only fails on the
    # missing device -- only checked where no GPU is visible
    if _gpu_visible():
        pytest.skip("would launch")
    assert lib.ln_fwd(*fwd_args(M=0, x=None, y=None, mean=None, rstd=None)) == 8
    assert lib.ln_bwd(*bwd_args("ln_bwd", M=0, dy=None, x=None, dx=None, mean=None,
                                rstd=None)) == 8


def fwd8_args(**over):
    a = dict(x=P, bias=None, res=None, gamma=None, beta=None, eps=1e-5, M=4, N=64, dtype=1,
             scale=P, y=P, res_out=None, mean=None, rstd=None, amax=None, amax_ws=None, flags=0,
             stream=None)
    a.update(over)
    return [a[k] for k in ("x", "bias", "res", "gamma", "beta", "eps", "M", "N", "dtype",
                           "scale", "y", "res_out", "mean", "rstd", "amax", "amax_ws", "flags",
                           "stream")]


@pytest.mark.parametrize("fn", ["ln_fwd_fp8", "rms_fwd_fp8"])
@pytest.mark.parametrize("over,code", [
    (dict(dtype=2), 4), (dict(scale=None), 1), (dict(y=None), 1), (dict(x=None), 1),
    (dict(N=0), 2), (dict(eps=-1.0), 3), (dict(scale=BAD2), 5), (dict(x=BAD1), 5),
    (dict(amax=BAD2), 5), (dict(amax=P, amax_ws=BAD2), 5), (dict(flags=2), 3),
    (dict(flags=8), 3),
])
def test_fp8_forward_rejects(lib, fn, over, code):
    assert getattr(lib, fn)(*fwd8_args(**over)) == code


def test_fp8_forward_takes_any_output_alignment(lib):
    """y_fp8 holds bytes: an odd address is not an argument error (it only
    leaves the vectorised kernels), so the check reaches the device."""
    if _gpu_visible():
        pytest.skip("would launch")
    assert lib.ln_fwd_fp8(*fwd8_args(y=P + 1)) == 8


@pytest.mark.parametrize("fn", ["ln_fwd", "rms_fwd"])
def test_forward_rejects_unknown_or_backward_flags(lib, fn):
    extra = dict(mean=None) if fn == "rms_fwd" else {}
    assert getattr(lib, fn)(*fwd_args(flags=2, **extra)) == 3   # a backward-only option
    assert getattr(lib, fn)(*fwd_args(flags=16, **extra)) == 3


def test_binding_option_bits_match_header():
    text = open(HEADER).read()
    assert int(re.search(r"#define NORM_ZERO_CENTERED_GAMMA (\d+)u", text).group(1)) == \
        nf.ZERO_CENTERED_GAMMA
    assert int(re.search(r"#define NORM_DPARAM_MEAN (\d+)u", text).group(1)) == nf.DPARAM_MEAN


@pytest.mark.parametrize("over,code", [
    (dict(dtype=5), 4), (dict(x=None), 1), (dict(y=None), 1), (dict(N=0), 2),
    (dict(M=-1), 2), (dict(flags=1), 3), (dict(x=BAD1), 5), (dict(dtype=0, y=BAD2), 5),
])
def test_softmax_rejects(lib, over, code):
    a = dict(x=P, M=4, N=64, dtype=1, y=P, flags=0, stream=None)
    a.update(over)
    assert lib.softmax_fwd(*[a[k] for k in ("x", "M", "N", "dtype", "y", "flags", "stream")]) == code


def test_rms_forward_takes_no_mean(lib):
    assert lib.rms_fwd(*fwd_args(mean=P)) == 3


def bwd_args(fn, **over):
    a = dict(dy=P, x=P, gamma=P, mean=P, rstd=P, eps=1e-6, M=4, N=64, dtype=1, dx=P,
             dgamma=P, dbeta=P, dbias=None, pdtype=0, ws=P, ws_bytes=1 << 20, flags=0,
             stream=None)
    a.update(over)
    keys = ["dy", "x", "gamma"] + (["rstd", "eps"] if fn == "rms_bwd" else ["mean", "rstd"]) + [
        "M", "N", "dtype", "dx", "dgamma", "dbeta", "dbias", "pdtype"] + \
        ([] if fn == "ln_bwd_noalloc" else ["ws", "ws_bytes"]) + ["flags", "stream"]
    return [a[k] for k in keys]


@pytest.mark.parametrize("over,code", [
    (dict(dtype=3), 4), (dict(pdtype=7), 4), (dict(dy=None), 1), (dict(mean=None), 1),
    (dict(M=-1), 2), (dict(N=16385), 2), (dict(flags=4), 3), (dict(dx=BAD1), 5),
    (dict(rstd=BAD2), 5),
])
def test_noalloc_backward_rejects(lib, over, code):
    """ln_bwd_noalloc checks its arguments as ln_bwd does, before touching a
    device (it takes no workspace)."""
    assert lib.ln_bwd_noalloc(*bwd_args("ln_bwd_noalloc", **over)) == code


@pytest.mark.parametrize("fn", ["ln_bwd", "rms_bwd"])
@pytest.mark.parametrize("over,code", [
    (dict(dtype=3), 4), (dict(pdtype=7), 4),
    (dict(dy=None), 1), (dict(x=None), 1), (dict(dx=None), 1),
    (dict(M=-2), 2), (dict(N=0), 2), (dict(N=16385), 2),
    (dict(dy=BAD1), 5), (dict(dx=BAD1), 5), (dict(rstd=BAD2), 5), (dict(ws=BAD2), 5), (dict(ws=P + 4), 5),
    (dict(pdtype=0, dgamma=BAD2), 5), (dict(pdtype=1, dbeta=BAD1), 5),
    (dict(pdtype=0, dbias=BAD2), 5), (dict(pdtype=1, dbias=BAD1), 5),
    (dict(flags=4), 3), (dict(flags=0x80000000), 3),
])
def test_backward_rejects(lib, fn, over, code):
    assert getattr(lib, fn)(*bwd_args(fn, **over)) == code


def test_ln_backward_needs_stats(lib):
    assert lib.ln_bwd(*bwd_args("ln_bwd", mean=None)) == 1
    assert lib.ln_bwd(*bwd_args("ln_bwd", rstd=None)) == 1


def test_rms_backward_eps_only_checked_when_recomputing(lib):
    assert lib.rms_bwd(*bwd_args("rms_bwd", rstd=None, eps=-1.0)) == 3
    assert lib.rms_bwd(*bwd_args("rms_bwd", rstd=None, eps=math.nan)) == 3


def test_workspace_size_rejects(lib):
    n = ctypes.c_size_t(0)
    assert lib.norm_bwd_workspace_size(4, 64, 1, None) == 1
    assert lib.norm_bwd_workspace_size(4, 64, 9, ctypes.byref(n)) == 4
    assert lib.norm_bwd_workspace_size(4, 0, 1, ctypes.byref(n)) == 2
    assert lib.norm_bwd_workspace_size(-1, 64, 1, ctypes.byref(n)) == 2


def _gpu_visible():
    import torch
    return torch.cuda.is_available()


@pytest.mark.skipif(_gpu_visible(), reason="only meaningful without a GPU (would launch)")
def test_valid_call_without_device_reports_device_error(lib):
    assert lib.ln_fwd(*fwd_args()) == 8
    n = ctypes.c_size_t(0)
    assert lib.norm_bwd_workspace_size(4, 64, 1, ctypes.byref(n)) == 8


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    """The Python layer has no fallback: a missing library is an error."""
    monkeypatch.setattr(nf, "_lib", None)
    monkeypatch.setattr(nf, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(nf.NormLibraryMissing):
        nf.library()


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asked for more it exits before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_product_library_reads_no_tuning_variables(lib):
    """Only the test build's host code reads the NORMFUSE_* overrides: the
    names are in libnormfuse_tuning.so and absent from the product library,
    whose results and workspace sizes follow from a call's arguments."""
    from normalization_ln_fwd_amd import build as b
    prod = open(b.LIB, "rb").read()
    test_build = open(b.TUNING_LIB, "rb").read()
    for name in (b"NORMFUSE_BWD_SPLIT", b"NORMFUSE_WT_BYTES", b"NORMFUSE_FWD_SHAPE",
                 b"NORMFUSE_BWD_GROUPS_PER_WG"):
        assert name not in prod, name
        assert name in test_build, name


def test_binding_rejects_unsupported_dparam_dtype():
    """dgamma / dbeta are fp32 or bf16; any other dparam_dtype is refused
    before anything reaches the library (no silent bf16 bit patterns in an
    fp16 tensor)."""
    import torch
    x = torch.zeros(2, 8, dtype=torch.bfloat16)
    for bad in (torch.float16, torch.float64, torch.int32):
        with pytest.raises(TypeError, match="dparam_dtype"):
            nf.ln_bwd(x, x, None, None, None, dparam_dtype=bad)
        with pytest.raises(TypeError, match="dparam_dtype"):
            nf.rms_bwd(x, x, None, dparam_dtype=bad)
    with pytest.raises(TypeError, match="dparam_dtype"):
        nf.ln_bwd(x.half(), x.half(), None, None, None)  # defaults to x's dtype


def test_describe_names_the_planned_kernels(lib):
    """norm_describe runs the calls' planning code without a device: the
    benchmark's shapes take the kernels its roofline names."""
    d = nf.describe("ln_fwd", 576000, 384, nf.BF16, amax=True)
    assert d.startswith("fwd_kernel<bf16, VEC 8, LPR 16, VPL 3, TEAMS 32, LayerNorm>"), d
    assert "grid 18000 x 512 threads" in d, d
    assert "reset kernel" in d, d
    d = nf.describe("ln_fwd", 576000, 384, nf.BF16, amax=True, amax_ws=True)
    assert "written by the last workgroup" in d, d
    d = nf.describe("rms_fwd", 576000, 384, nf.BF16, amax=True)
    assert "TEAMS 32, RMSNorm>" in d, d
    d = nf.describe("ln_bwd", 576000, 384, nf.BF16)
    assert d.startswith("bwd_kernel<bf16, VEC 8, LPR 16, VPL 3, TEAMS 16, LayerNorm>"), d
    assert "grid 508 x 256 threads, 71 row group(s)" in d, d
    assert "column sums of 508 partial rows in 1" in d, d
    d = nf.describe("ln_bwd", 8192, 4096, nf.BF16, dbias=True)
    assert d.startswith("bwd_kernel<bf16, VEC 8, LPR 512, VPL 1, TEAMS 2, LayerNorm, dbias>"), d
    assert "grid 256 x 1024 threads, 16 row group(s)" in d, d
    assert nf.describe("softmax_fwd", 576000, 384, nf.BF16).startswith(
        "softmax_kernel<bf16, VEC 8, LPR 16, VPL 3, TEAMS 32>")
    assert "bwd_split_kernel" in nf.describe("ln_bwd", 64, 16384, nf.BF16)
    # one wave per row holding five vectors only from 2048 row groups on
    assert nf.describe("ln_fwd", 8192, 2560, nf.BF16).startswith(
        "fwd_kernel<bf16, VEC 8, LPR 64, VPL 5, TEAMS 4,")
    assert nf.describe("ln_fwd", 8188, 2560, nf.BF16).startswith(
        "fwd_kernel<bf16, VEC 8, LPR 320, VPL 1, TEAMS 2,")
    assert nf.describe("ln_bwd", 8192, 5120, nf.BF16).startswith(
        "bwd_kernel<bf16, VEC 8, LPR 320, VPL 2, TEAMS 2,")


def test_describe_walk_rules(lib):
    """The walk rules the measurements chose: wide backward rows take as many
    workgroups as the CUs hold (no second round behind the first), the
    forward's 16-byte wide rows walk two groups beyond 4096 row groups and
    four up to them, the 8-byte bf16 backward on 512-thread workgroups runs
    two per CU."""
    def grid_k(op, M, N, dtype=nf.BF16):
        m = re.search(r"grid (\d+) x \d+ threads, (\d+) row group", nf.describe(op, M, N, dtype))
        return int(m.group(1)), int(m.group(2))
    assert grid_k("ln_bwd", 52428, 2560) == (255, 103)
    assert grid_k("ln_bwd", 131072, 4096) == (256, 256)
    assert grid_k("ln_bwd", 8192, 4096) == (256, 16)
    assert grid_k("ln_fwd", 43690, 3072) == (10923, 2)
    assert grid_k("ln_fwd", 8192, 4096) == (1024, 4)
    assert grid_k("ln_fwd", 10922, 12288) == (5461, 2)     # 768 lanes x 2 vectors
    assert grid_k("ln_fwd", 8192, 16384) == (2048, 4)      # 512 lanes x 4 vectors
    assert grid_k("ln_bwd", 43633, 3076)[0] == 508
    # softmax keeps walks of four; odd-N softmax one group per workgroup
    assert grid_k("softmax_fwd", 43690, 3072)[1] == 4
    assert grid_k("softmax_fwd", 32760, 4097)[1] == 1


def _odd_unit(op, M, N, dtype):
    """The odd-row unit a call would take (0: another kernel)."""
    m = re.search(r"odd_kernel<\w+, unit (\d+),", nf.describe(op, M, N, dtype))
    return int(m.group(1)) if m else 0


def test_describe_names_the_odd_row_kernels(lib):
    """Rows of an odd multiple of a unit (1, 2 or, bf16, 4 elements) take the
    odd-row kernels of that unit up to the longest row their tables hold;
    rows of whole 16-byte vectors do not."""
    BF16, F32 = nf.BF16, nf.F32
    for dt in (BF16, F32):
        for op in ("ln_fwd", "rms_fwd", "softmax_fwd"):
            longest = 8193 if dt == F32 and op != "softmax_fwd" else 16383
            assert _odd_unit(op, 1000, longest, dt) == 1
            assert _odd_unit(op, 3, 1, dt) == 1
            if longest + 2 <= 16384:
                assert _odd_unit(op, 1000, longest + 2, dt) == 0
            assert _odd_unit(op, 1000, 1002, dt) == 2
            assert _odd_unit(op, 1000, 2, dt) == 2
            assert _odd_unit(op, 1000, 1004, dt) == (4 if dt == BF16 else 0)
            assert _odd_unit(op, 1000, 1024, dt) == 0
    assert _odd_unit("ln_fwd", 10, 8194, F32) == 2 and _odd_unit("ln_fwd", 10, 8198, F32) == 0
    # softmax of 2- and 4-element units on a wide team only where that
    # leaves fewer lanes idle than the vector kernel
    assert _odd_unit("softmax_fwd", 10, 10242, F32) == 2      # 10240 of 10240 vs 12288
    assert _odd_unit("softmax_fwd", 10, 16382, F32) == 0      # 16380 of 16384 vs 16382 of 16384
    assert _odd_unit("softmax_fwd", 10, 6004, BF16) == 0      # 8192-column teams either way
    assert _odd_unit("softmax_fwd", 10, 6002, BF16) == 0 and _odd_unit("ln_fwd", 10, 6002, BF16) == 2
    # one wave per row (a narrow layout) at any fill
    assert _odd_unit("softmax_fwd", 10, 4100, BF16) == 4 and _odd_unit("softmax_fwd", 10, 3076, BF16) == 4
    assert _odd_unit("ln_fwd", 10, 16380, BF16) == 4 and _odd_unit("ln_fwd", 10, 16382, BF16) == 2


def test_describe_names_the_odd_row_backward(lib):
    """The backward takes the odd-row kernels for odd N up to 8193 columns;
    for units of 2 and 4 elements it takes a wide odd-row shape only where
    that leaves fewer lanes idle than the vector kernel would."""
    BF16, F32 = nf.BF16, nf.F32
    for dt in (BF16, F32):
        assert _odd_unit("ln_bwd", 1000, 8193, dt) == 1
        assert _odd_unit("rms_bwd", 3, 1, dt) == 1
        assert _odd_unit("ln_bwd", 1000, 8195, dt) == 0
        assert _odd_unit("ln_bwd", 1000, 1024, dt) == 0
        assert _odd_unit("ln_bwd", 1000, 4098, dt) == 2
        assert _odd_unit("ln_bwd", 1000, 1002, dt) == 2      # narrow: always
    assert _odd_unit("ln_bwd", 1000, 8194, BF16) == 2 and _odd_unit("ln_bwd", 1000, 8198, BF16) == 0
    assert _odd_unit("ln_bwd", 1000, 8194, F32) == 2 and _odd_unit("ln_bwd", 1000, 8198, F32) == 0
    assert _odd_unit("ln_bwd", 1000, 4100, BF16) == 4 and _odd_unit("ln_bwd", 1000, 8196, BF16) == 4
    assert _odd_unit("ln_bwd", 1000, 8204, BF16) == 0 and _odd_unit("ln_bwd", 1000, 4102, F32) == 0
    # the same fill as the vector kernel's (6000 of 6144 lanes' columns)
    assert _odd_unit("ln_bwd", 1000, 6004, BF16) == 0
    assert _odd_unit("ln_bwd", 1000, 6002, BF16) == 0
    # more idle lanes than the vector kernel's
    assert _odd_unit("ln_bwd", 1000, 5124, BF16) == 0


def test_describe_rejects(lib):
    buf = ctypes.create_string_buffer(64)
    assert lib.norm_describe(0, 4, 64, 1, 0, None, 64) == 1
    assert lib.norm_describe(0, 4, 64, 1, 0, buf, 0) == 1
    assert lib.norm_describe(0, 4, 64, 7, 0, buf, 64) == 4
    assert lib.norm_describe(0, 4, 0, 1, 0, buf, 64) == 2
    assert lib.norm_describe(9, 4, 64, 1, 0, buf, 64) == 3
    assert lib.norm_describe(0, 4, 64, 1, 16, buf, 64) == 3
    # a short buffer holds a truncated, terminated text
    small = ctypes.create_string_buffer(8)
    assert lib.norm_describe(0, 4, 64, 1, 0, small, 8) == 0
    assert small.value == b"fwd_ker"


def test_binding_dtype_arguments(lib):
    """describe / bwd_workspace_size take a dtype code, a torch dtype or its
    name, and refuse any other type instead of mapping it to bf16."""
    import torch
    for bf in ("bf16", "bfloat16", torch.bfloat16):
        assert nf.describe("ln_fwd", 4096, 384, bf) == nf.describe("ln_fwd", 4096, 384, nf.BF16)
    for f in ("f32", "fp32", "float32", torch.float32):
        assert nf.describe("ln_fwd", 64, 384, f) == nf.describe("ln_fwd", 64, 384, nf.F32)
    for bad in (torch.float16, "fp16", 7, None):
        with pytest.raises(TypeError, match="unsupported dtype"):
            nf.describe("ln_fwd", 64, 384, bad)
        with pytest.raises(TypeError, match="unsupported dtype"):
            nf.bwd_workspace_size(64, 384, bad)
