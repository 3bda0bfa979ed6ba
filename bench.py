#!/usr/bin/env python3
"""Benchmark of the fused LayerNorm forward + mix-order backward on one MI355X.

A step is one pass of the whole path over one batch: ln_fwd (bias + residual
+ LayerNorm; y, residual_out, mean, rstd, amax) followed by ln_bwd on its
outputs (dx, dgamma, dbeta in bf16), at M = 1152 * 500 = 576000 rows by
N = 384, bf16 tensors, fp32 arithmetic.  Inputs are seeded synthetic
Gaussians (x, residual, dy ~ N(0,1); bias, beta ~ N(0, 0.1); gamma ~ 1 +
N(0, 0.1)) resident in HBM before timing starts.

value = algorithmic bytes of a step / time of a step (GB/s): each [M, N]
tensor read or written once plus the fp32 per-row statistics (forward
8N + 8 bytes per row, backward 6N + 8).  Prints ONE JSON line on stdout;
progress goes to stderr.

Also reported: the roofline of the dominant kernel (the forward): its
algorithmic bytes over the per-launch duration of K forward calls run back
to back between two HIP events; a per-case breakdown (each case timed the
same way, cycling through buffers that together exceed the last-level
cache); and the CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0  # MI355X HBM3E
M_BIG, N_BIG = 1152 * 500, 384
CALIB_BYTES = 512 << 20
# every source that decides what the measured kernels do (the kernels, the
# host code that picks their shapes, grids and cache policies, the header)
KERNEL_SOURCE_DIRS = ("normalization_ln_fwd_amd/csrc", "include")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_576000x384_8192x4096.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fwd_bytes(M, N, es=2, stats=2, io_tensors=4):
    return M * (io_tensors * N * es + 4 * stats)


def bwd_bytes(M, N, es=2, stats=2):
    return M * (3 * N * es + 4 * stats)


def kernel_source_hash():
    h = hashlib.sha256()
    for d in KERNEL_SOURCE_DIRS:
        for name in sorted(os.listdir(os.path.join(ROOT, d))):
            if name.endswith((".hip", ".hpp", ".cpp", ".h")):
                h.update(name.encode())
                with open(os.path.join(ROOT, d, name), "rb") as fh:
                    h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per forward launch from the committed counter summary, if it
    was taken on the current kernel sources (else None)."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    src = re.search(r"kernel_source_hash:\s*([0-9a-f]+)", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not src or not val or src.group(1) != kernel_source_hash():
        return None
    return float(val.group(1))


class HipEvents:
    """n timing events of the HIP runtime, recorded on a given stream.

    Created with hipEventDisableSystemFence: recording a default event ends
    with a system-scope release (cache write-back) that costs several
    microseconds and lands inside the interval being timed; these events only
    take timestamps.  The runtime is the one already loaded in this process
    (by torch and the library)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        import ctypes
        path = None
        with open("/proc/self/maps") as fh:
            for line in fh:
                if "libamdhip64.so" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        self.ct = ctypes
        self.hip = ctypes.CDLL(path)
        self.ev = [ctypes.c_void_p() for _ in range(n)]
        for e in self.ev:
            self._check(self.hip.hipEventCreateWithFlags(ctypes.byref(e),
                                                         ctypes.c_uint(self.DISABLE_SYSTEM_FENCE)))

    def _check(self, rc):
        if rc != 0:
            raise RuntimeError(f"HIP event call failed with status {rc}")

    def record(self, i, stream):
        self._check(self.hip.hipEventRecord(self.ev[i], self.ct.c_void_p(stream)))

    def elapsed_ms(self, i, j):
        ms = self.ct.c_float()
        self._check(self.hip.hipEventElapsedTime(self.ct.byref(ms), self.ev[i], self.ev[j]))
        return ms.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--breakdown-iters", type=int, default=50)
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=M_BIG,
                    help="rows of the workload the CPU oracle is timed on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 512 MiB device copy (counter calibration)")
    ap.add_argument("--no-alt-sets", action="store_true",
                    help="skip the step timed on two alternating buffer sets")
    ap.add_argument("--cases", default="",
                    help="comma-separated breakdown cases to run (name prefixes; default all)")
    ap.add_argument("--large-m", action="store_true",
                    help="also time the forward and backward at 2, 4 and 8 times the rows")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: measures one GPU only (the path has no multi-GPU component); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import normalization_ln_fwd_amd as nf
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    nf.library()  # fails loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    M, N = M_BIG, N_BIG
    t0 = time.time()
    h = synth.make_inputs(M, N, dtype=synth.BF16, seed=0,
                          names=("x", "residual", "bias", "gamma", "beta", "dy"))
    log(f"inputs generated in {time.time() - t0:.1f}s")
    d = {k: to_dev(v) for k, v in h.items()}
    y = torch.empty_like(d["x"])
    res_out = torch.empty_like(d["x"])
    mean = torch.empty(M, dtype=torch.float32, device=dev)
    rstd = torch.empty(M, dtype=torch.float32, device=dev)
    amax = torch.empty(1, dtype=torch.float32, device=dev)
    dx = torch.empty_like(d["x"])
    dgamma = torch.empty(N, dtype=torch.bfloat16, device=dev)
    dbeta = torch.empty(N, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(4, nf.bwd_workspace_size(M, N, torch.bfloat16)), dtype=torch.uint8,
                     device=dev)
    fwd_out = {"y": y, "residual_out": res_out, "mean": mean, "rstd": rstd, "amax": amax}
    bwd_out = {"dx": dx, "dgamma": dgamma, "dbeta": dbeta}
    # amax in one kernel launch: the forward's workspace (zero-filled once,
    # left zero-filled by every call)
    amax_ws = nf.amax_workspace(dev)

    def fwd():
        nf.ln_fwd(d["x"], d["bias"], d["residual"], d["gamma"], d["beta"], 1e-5,
                  want_amax=True, amax_workspace=amax_ws, out=fwd_out)

    def bwd():
        nf.ln_bwd(d["dy"], res_out, d["gamma"], mean, rstd, dparam_dtype=torch.bfloat16,
                  workspace=ws, out=bwd_out)

    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    # Timed region: K steps on the current stream (the binding launches on
    # it), one event before and one after: recording an event costs a few
    # microseconds of idle GPU, so none is recorded between the steps.
    K = args.steps
    stream = torch.cuda.current_stream().cuda_stream
    ev = HipEvents(2)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev.record(0, stream)
    for k in range(K):
        fwd()
        bwd()
    ev.record(1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = ev.elapsed_ms(0, 1) / K
    ev.close()
    step_bytes = fwd_bytes(M, N) + bwd_bytes(M, N)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    log(f"timed {K} steps: {ms_step:.4f} ms/step (wall {wall / K * 1e3:.4f} ms/step), "
        f"{value:.1f} GB/s")
    # The same steps alternating between this buffer set and a second one
    # (same shapes, seed 1), reported beside the value: a step on one set
    # measures slightly faster than steps that alternate sets, although
    # either moves far more than the last-level cache between two uses of a
    # buffer.
    alt_ms = None
    if not args.no_alt_sets:
        h1 = synth.make_inputs(M, N, dtype=synth.BF16, seed=1,
                               names=("x", "residual", "bias", "gamma", "beta", "dy"))
        d1 = {k: to_dev(v) for k, v in h1.items()}
        del h1
        fo1 = {k: torch.empty_like(v) for k, v in fwd_out.items()}
        bo1 = {k: torch.empty_like(v) for k, v in bwd_out.items()}
        ws1 = torch.empty_like(ws)
        aws1 = nf.amax_workspace(dev)

        def step1():
            nf.ln_fwd(d1["x"], d1["bias"], d1["residual"], d1["gamma"], d1["beta"], 1e-5,
                      want_amax=True, amax_workspace=aws1, out=fo1)
            nf.ln_bwd(d1["dy"], fo1["residual_out"], d1["gamma"], fo1["mean"], fo1["rstd"],
                      dparam_dtype=torch.bfloat16, workspace=ws1, out=bo1)

        def step0():
            fwd()
            bwd()

        alt_ms = time_calls([step0, step1], K, torch)[0] * 1e-3
        del d1, fo1, bo1, ws1
        log(f"steps alternating two buffer sets: {alt_ms:.4f} ms/step, "
            f"{step_bytes / (alt_ms * 1e-3) / 1e9:.1f} GB/s")

    # Per-launch durations of the two halves of the step: K forward calls back
    # to back between two events, then K backward calls.  A forward call is
    # one kernel (amax through the workspace).
    fwd_avg = time_calls([fwd], K, torch)[2]
    bwd_avg = time_calls([bwd], K, torch)[2]
    fwd_gbs = fwd_bytes(M, N) / (fwd_avg * 1e-6) / 1e9
    traffic = recorded_traffic()
    roofline = {"bound": "hbm", "achieved": round(fwd_gbs, 1), "peak": PEAK_GBS, "unit": "GB/s",
                "frac": round(fwd_gbs / PEAK_GBS, 4), "traffic": traffic,
                "kernel": nf.describe("ln_fwd", M, N, torch.bfloat16, amax=True, amax_ws=True),
                "bytes_per_launch": fwd_bytes(M, N), "avg_launch_us": round(fwd_avg, 2),
                "kernel_source_hash": kernel_source_hash()}

    result = {
        "metric": "achieved HBM GB/s (% of MI355X peak) for fused LN/RMSNorm fwd and bwd",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "fused bias+residual LayerNorm fwd (y, residual_out, mean, rstd, "
                               "amax) + mix-order LayerNorm bwd (dx, dgamma, dbeta), "
                               "M=576000 (1152x500) x N=384",
                   "M": M, "N": N, "io_dtype": "bf16", "compute_dtype": "f32",
                   "step_bytes": step_bytes, "frac_of_peak": round(value / PEAK_GBS, 4),
                   "fwd_us": round(fwd_avg, 2), "bwd_us": round(bwd_avg, 2),
                   "ms_per_step_two_sets": round(alt_ms, 5) if alt_ms else None,
                   "frac_of_peak_two_sets": (round(step_bytes / (alt_ms * 1e-3) / 1e9 / PEAK_GBS, 4)
                                             if alt_ms else None)},
        "roofline": roofline,
    }

    if args.calib_copy:
        src = torch.empty(CALIB_BYTES // 2, dtype=torch.bfloat16, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["calib_copy_bytes"] = 2 * src.numel() * src.element_size()
        log("calibration copies done")

    if not args.no_breakdown:
        cases = [c for c in args.cases.split(",") if c]
        result["breakdown"] = breakdown(args.breakdown_iters, nf, torch, np, synth, d, h, dev,
                                        fwd_out, ws, cases, amax_ws)

    if args.large_m:
        cases = [c for c in args.cases.split(",") if c]
        result["large_m"] = large_m(args.breakdown_iters, nf, torch, d, dev, cases)

    # free the device copies before the CPU leg
    del d
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(h, args.cpu_rows)

    print(json.dumps(result), flush=True)


WARM_S = 0.02  # untimed calls before each breakdown case, in seconds of GPU work
PREQUEUE = 4   # untimed calls queued right before a timed interval starts
FLUSH_BYTES = 512 << 20  # scratch written before each call of a flushed timing


def time_flushed(fns, iters, torch, scratch):
    """Microseconds of single calls that each follow a write of FLUSH_BYTES
    to a scratch buffer (larger than the 256 MB last-level cache plus the L2s,
    so no input of the call is cached when it starts): events bracket each
    call, the write runs outside them.  Returns the median over `iters`
    calls, cycling through fns."""
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(3):
        scratch.fill_(i)
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    ev = HipEvents(2 * iters)
    for i in range(iters):
        scratch.fill_(i & 0x7F)
        ev.record(2 * i, stream)
        fns[i % len(fns)]()
        ev.record(2 * i + 1, stream)
    torch.cuda.synchronize()
    us = sorted(ev.elapsed_ms(2 * i, 2 * i + 1) * 1e3 for i in range(iters))
    ev.close()
    return us[len(us) // 2]


def time_calls(fns, iters, torch):
    """Microseconds per call in steady state: after untimed calls that keep
    the GPU busy for WARM_S (after host-side work the GPU runs slower for a
    few milliseconds), `iters` calls run back to back between two events,
    cycling through fns (the same operation on different buffers, so that
    small cases do not run out of the 256 MB last-level cache).  A few
    untimed calls are queued right before the first event, so that the GPU
    is still busy with them while the host issues the timed ones (otherwise
    the first timed call waits for the host, a gap of tens of microseconds
    inside the timed interval).  Returns (per call over the whole run, best
    of 5 equal slices, per call of the run)."""
    stream = torch.cuda.current_stream().cuda_stream
    t0, n = time.perf_counter(), 0
    while n < 10 or time.perf_counter() - t0 < WARM_S:
        for _ in range(5):
            fns[n % len(fns)]()
            n += 1
        torch.cuda.synchronize()
    slices = 5
    per = max(1, iters // slices)
    ev = HipEvents(slices + 1)
    torch.cuda.synchronize()
    for i in range(PREQUEUE):
        fns[(n + i) % len(fns)]()
    ev.record(0, stream)
    for j in range(slices):
        for i in range(per):
            fns[(j * per + i) % len(fns)]()
        ev.record(j + 1, stream)
    torch.cuda.synchronize()
    sl = [ev.elapsed_ms(j, j + 1) * 1e3 / per for j in range(slices)]
    total = ev.elapsed_ms(0, slices) * 1e3 / (per * slices)
    ev.close()
    return total, min(sl), total


def time_graph(fns, torch, replays=20):
    """Microseconds per call of fns (a list of calls, each run once) captured
    into one HIP graph and replayed: the GPU time of a launch-bound case
    without the host's per-call cost (Python binding, launch API)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in fns:  # warm-up on the capture stream
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for f in fns:
            f()
    stream = torch.cuda.current_stream().cuda_stream
    t0, n = time.perf_counter(), 0
    while n < 3 or time.perf_counter() - t0 < WARM_S:
        g.replay()
        n += 1
        torch.cuda.synchronize()
    ev = HipEvents(2)
    ev.record(0, stream)
    for _ in range(replays):
        g.replay()
    ev.record(1, stream)
    torch.cuda.synchronize()
    us = ev.elapsed_ms(0, 1) * 1e3 / (replays * len(fns))
    ev.close()
    del g
    return us


def breakdown(iters, nf, torch, np, synth, d, h, dev, fwd_out, ws, cases=(), amax_ws=None):
    out = {}

    def want(*names):
        return not cases or any(n.startswith(c) for n in names for c in cases)

    def rec(name, fn, nbytes, gated):
        if not want(name):
            return
        fns = fn if isinstance(fn, list) else [fn]
        med, mn, _ = time_calls(fns, iters, torch)
        gbs = nbytes / (med * 1e-6) / 1e9
        out[name] = {"us_per_call": round(med, 2), "us_best_slice": round(mn, 2), "bytes": nbytes,
                     "GB_s": round(gbs, 1), "frac_peak": round(gbs / PEAK_GBS, 4),
                     "gated_70pct": gated}
        log(f"  {name}: {med:.1f} us, {gbs:.0f} GB/s ({100 * gbs / PEAK_GBS:.1f}% of peak)")

    def graph_rec(name, fns, nbytes):
        if not want(name):
            return
        us = time_graph(fns, torch)
        gbs = nbytes / (us * 1e-6) / 1e9
        out[name] = {"us_per_call": round(us, 2), "bytes": nbytes, "GB_s": round(gbs, 1),
                     "frac_peak": round(gbs / PEAK_GBS, 4), "gated_70pct": False,
                     "timing": f"HIP graph of {len(fns)} calls, replayed"}
        log(f"  {name}: {us:.1f} us, {gbs:.0f} GB/s ({100 * gbs / PEAK_GBS:.1f}% of peak)")

    M, N = M_BIG, N_BIG
    rec("ln_fwd_576000x384", lambda: nf.ln_fwd(d["x"], d["bias"], d["residual"], d["gamma"],
                                                d["beta"], 1e-5, want_amax=True,
                                                amax_workspace=amax_ws, out=fwd_out),
        fwd_bytes(M, N), True)
    # the same without the amax workspace: a one-thread kernel zeroes amax first
    rec("ln_fwd_576000x384_amax_reset", lambda: nf.ln_fwd(
        d["x"], d["bias"], d["residual"], d["gamma"], d["beta"], 1e-5, want_amax=True,
        out=fwd_out), fwd_bytes(M, N), False)
    # FP8 output (E4M3 codes, one byte per element) with the scale taken from
    # the amax of a previous call, as a training step would
    y8 = torch.empty((M, N), dtype=torch.float8_e4m3fn, device=dev)
    sc = (448.0 / fwd_out["amax"]).to(torch.float32)
    fp8_out = {"y": y8, "residual_out": fwd_out["residual_out"], "mean": fwd_out["mean"],
               "rstd": fwd_out["rstd"], "amax": fwd_out["amax"]}
    rec("ln_fwd_fp8_576000x384", lambda: nf.ln_fwd_fp8(d["x"], sc, d["bias"], d["residual"],
                                                        d["gamma"], d["beta"], 1e-5,
                                                        want_amax=True, amax_workspace=amax_ws,
                                                        out=fp8_out),
        M * (7 * N + 8), False)
    del y8
    rec("ln_fwd_576000x384_zero_centered", lambda: nf.ln_fwd(
        d["x"], d["bias"], d["residual"], d["gamma"], d["beta"], 1e-5, want_amax=True,
        zero_centered_gamma=True, amax_workspace=amax_ws, out=fwd_out), fwd_bytes(M, N), False)
    rms_out = {"y": fwd_out["y"], "residual_out": fwd_out["residual_out"],
               "rstd": fwd_out["rstd"], "amax": fwd_out["amax"]}
    rec("rms_fwd_576000x384", lambda: nf.rms_fwd(d["x"], d["bias"], d["residual"], d["gamma"],
                                                  None, 1e-6, want_amax=True,
                                                  amax_workspace=amax_ws, out=rms_out),
        fwd_bytes(M, N, stats=1), False)
    # the 576000 x 384 backwards (RMSNorm with rstd recomputed, LayerNorm from
    # saved statistics): on x = N(0,1) (the generator's x), dy
    dx = torch.empty_like(d["x"])
    dg = torch.empty(N, dtype=torch.bfloat16, device=dev)
    db = torch.empty(N, dtype=torch.bfloat16, device=dev)
    nf.ln_fwd(d["x"], None, None, None, None, 1e-5, out=fwd_out)  # mean / rstd of x
    rec("rms_bwd_576000x384_recompute", lambda: nf.rms_bwd(
        d["dy"], d["x"], d["gamma"], None, 1e-6, dparam_dtype=torch.bfloat16, workspace=ws,
        out={"dx": dx, "dgamma": dg}), bwd_bytes(M, N, stats=0), True)
    rec("ln_bwd_576000x384", lambda: nf.ln_bwd(
        d["dy"], d["x"], d["gamma"], fwd_out["mean"], fwd_out["rstd"],
        dparam_dtype=torch.bfloat16, workspace=ws, out={"dx": dx, "dgamma": dg, "dbeta": db}),
        bwd_bytes(M, N), True)
    dbias = torch.empty(N, dtype=torch.bfloat16, device=dev)
    rec("ln_bwd_576000x384_dbias", lambda: nf.ln_bwd(
        d["dy"], d["x"], d["gamma"], fwd_out["mean"], fwd_out["rstd"],
        dparam_dtype=torch.bfloat16, workspace=ws,
        out={"dx": dx, "dgamma": dg, "dbeta": db, "dbias": dbias}), bwd_bytes(M, N), False)
    rec("ln_bwd_576000x384_mean", lambda: nf.ln_bwd(
        d["dy"], d["x"], d["gamma"], fwd_out["mean"], fwd_out["rstd"],
        dparam_dtype=torch.bfloat16, dparam_mean=True, workspace=ws,
        out={"dx": dx, "dgamma": dg, "dbeta": db}), bwd_bytes(M, N), False)
    del dx
    # row softmax on the same rows (x in, y out, bf16)
    smx = torch.empty_like(d["x"])
    rec("softmax_fwd_576000x384", lambda: nf.softmax_fwd(d["x"], out=smx), M * 4 * N, False)
    del smx
    # 4096 x 384 bf16 forward with amax (launch-bound size): consecutive calls take consecutive
    # 4096-row slices of the large tensors
    M2 = 4096
    subs = [{k: (v[i * M2:(i + 1) * M2] if v.dim() == 2 else v) for k, v in d.items()}
            for i in range(M // M2)]
    rec("ln_fwd_4096x384_amax", [
        (lambda s=s: nf.ln_fwd(s["x"], s["bias"], s["residual"], s["gamma"], s["beta"], 1e-5,
                               want_amax=True, amax_workspace=amax_ws)) for s in subs],
        fwd_bytes(M2, N), False)
    # the same calls replayed from a captured graph (outputs preallocated):
    # the GPU time of the launch-bound size, with the amax workspace (one
    # kernel per call) and with the reset kernel (two)
    outs2 = [{"y": torch.empty_like(s["x"]), "residual_out": torch.empty_like(s["x"]),
              "mean": torch.empty(M2, device=dev), "rstd": torch.empty(M2, device=dev),
              "amax": torch.empty(1, device=dev)} for s in subs[:64]]
    graph_rec("ln_fwd_4096x384_amax_graph", [
        (lambda s=s, o=o: nf.ln_fwd(s["x"], s["bias"], s["residual"], s["gamma"], s["beta"],
                                    1e-5, want_amax=True, amax_workspace=amax_ws, out=o))
        for s, o in zip(subs[:64], outs2)], fwd_bytes(M2, N))
    graph_rec("ln_fwd_4096x384_amax_reset_graph", [
        (lambda s=s, o=o: nf.ln_fwd(s["x"], s["bias"], s["residual"], s["gamma"], s["beta"],
                                    1e-5, want_amax=True, out=o))
        for s, o in zip(subs[:64], outs2)], fwd_bytes(M2, N))
    del outs2
    # LayerNorm forward, fp32, 64 x 384, bias + residual; y, mean, rstd
    M1 = 64
    g1 = synth.make_inputs(M1 * 64, N, dtype=synth.F32, seed=0,
                           names=("x", "residual", "bias", "gamma", "beta"))
    d1 = {k: torch.from_numpy(v).to(dev) for k, v in g1.items()}
    calls1 = []
    for i in range(64):
        o1 = {"y": torch.empty(M1, N, device=dev), "mean": torch.empty(M1, device=dev),
              "rstd": torch.empty(M1, device=dev)}
        xs, rs = d1["x"][i * M1:(i + 1) * M1], d1["residual"][i * M1:(i + 1) * M1]
        calls1.append(lambda xs=xs, rs=rs, o1=o1: nf.ln_fwd(
            xs, d1["bias"], rs, d1["gamma"], d1["beta"], 1e-5, want_residual_out=False, out=o1))
    graph_rec("ln_fwd_64x384_f32_graph", calls1, M1 * (3 * 4 * N + 8))
    del d1, calls1
    # 8192 x 4096 bf16, residual + LayerNorm, 1% outliers.  Four buffer sets
    # rotate: between two uses of a set the other three move 600 MB
    # (backward) to 800 MB (forward), more than twice the 256 MB last-level
    # cache, so no call finds its inputs cached from its previous use.  The
    # same calls are also timed one at a time, each after a 512 MB scratch
    # write ("_flushed"), and on two alternating sets ("_2sets"), whose
    # working set of 400-540 MB lets part of a set survive in the last-level
    # cache until its next use (for comparison only).
    if not want("ln_fwd_8192x4096", "ln_bwd_8192x4096"):
        return out
    M5, N5 = 8192, 4096
    sets = []
    for seed in range(4):
        g5 = synth.make_inputs(M5, N5, dtype=synth.BF16, seed=seed, outlier_p=0.01,
                               names=("x", "residual", "gamma", "beta", "dy"))
        d5 = {k: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to(dev)
              for k, v in g5.items()}
        o5 = nf.ln_fwd(d5["x"], None, d5["residual"], d5["gamma"], d5["beta"], 1e-5)
        b5 = {"dx": torch.empty_like(d5["x"]),
              "dgamma": torch.empty(N5, dtype=torch.bfloat16, device=dev),
              "dbeta": torch.empty(N5, dtype=torch.bfloat16, device=dev)}
        sets.append((d5, o5, b5))
    ws5 = torch.empty(max(4, nf.bwd_workspace_size(M5, N5, torch.bfloat16)), dtype=torch.uint8,
                      device=dev)
    fwd5 = [(lambda d5=d5, o5=o5: nf.ln_fwd(d5["x"], None, d5["residual"], d5["gamma"],
                                            d5["beta"], 1e-5, out=o5)) for d5, o5, _ in sets]
    bwd5 = [(lambda d5=d5, o5=o5, b5=b5: nf.ln_bwd(d5["dy"], o5["residual_out"], d5["gamma"],
                                                   o5["mean"], o5["rstd"],
                                                   dparam_dtype=torch.bfloat16, workspace=ws5,
                                                   out=b5)) for d5, o5, b5 in sets]
    rec("ln_fwd_8192x4096", fwd5, fwd_bytes(M5, N5), True)
    rec("ln_bwd_8192x4096", bwd5, bwd_bytes(M5, N5), True)
    scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    for name, fns, nbytes in (("ln_fwd_8192x4096_flushed", fwd5, fwd_bytes(M5, N5)),
                              ("ln_bwd_8192x4096_flushed", bwd5, bwd_bytes(M5, N5))):
        if not want(name):
            continue
        us = time_flushed(fns, iters, torch, scratch)
        gbs = nbytes / (us * 1e-6) / 1e9
        out[name] = {"us_per_call": round(us, 2), "bytes": nbytes, "GB_s": round(gbs, 1),
                     "frac_peak": round(gbs / PEAK_GBS, 4), "gated_70pct": False,
                     "timing": "median of single calls, each after a 512 MB scratch write"}
        log(f"  {name}: {us:.1f} us, {gbs:.0f} GB/s ({100 * gbs / PEAK_GBS:.1f}% of peak)")
    del scratch
    rec("ln_fwd_8192x4096_2sets", fwd5[:2], fwd_bytes(M5, N5), False)
    rec("ln_bwd_8192x4096_2sets", bwd5[:2], bwd_bytes(M5, N5), False)
    torch.cuda.synchronize()
    return out


LARGE_M = (2 * M_BIG, 4 * M_BIG, 8 * M_BIG)


def large_m(iters, nf, torch, d, dev, cases=()):
    """Per-call time of the forward (amax workspace) and of the backward at
    2, 4 and 8 times the benchmark's rows (its 576000-row inputs repeated),
    each timed back to back like the breakdown: how the kernels follow the
    HBM's sustained rate as transfers grow.  Cases as in the breakdown,
    named ln_fwd_{M}x384 / ln_bwd_{M}x384."""
    out = {}
    N = N_BIG
    for M in LARGE_M:
        names = (f"ln_fwd_{M}x{N}", f"ln_bwd_{M}x{N}")
        todo = [n for n in names if not cases or any(n.startswith(c) for c in cases)]
        if not todo:
            continue
        r = M // M_BIG
        x, res, dy = (d[k].repeat(r, 1) for k in ("x", "residual", "dy"))
        fo = {"y": torch.empty_like(x), "residual_out": torch.empty_like(x),
              "mean": torch.empty(M, dtype=torch.float32, device=dev),
              "rstd": torch.empty(M, dtype=torch.float32, device=dev),
              "amax": torch.empty(1, dtype=torch.float32, device=dev)}
        bo = {"dx": torch.empty_like(x),
              "dgamma": torch.empty(N, dtype=torch.bfloat16, device=dev),
              "dbeta": torch.empty(N, dtype=torch.bfloat16, device=dev)}
        aws = nf.amax_workspace(dev)
        ws = torch.empty(max(4, nf.bwd_workspace_size(M, N, torch.bfloat16)), dtype=torch.uint8,
                         device=dev)

        def fwd():
            nf.ln_fwd(x, d["bias"], res, d["gamma"], d["beta"], 1e-5, want_amax=True,
                      amax_workspace=aws, out=fo)

        def bwd():
            nf.ln_bwd(dy, fo["residual_out"], d["gamma"], fo["mean"], fo["rstd"],
                      dparam_dtype=torch.bfloat16, workspace=ws, out=bo)

        fwd()
        for name, fn, nbytes in ((names[0], fwd, fwd_bytes(M, N)), (names[1], bwd, bwd_bytes(M, N))):
            if name not in todo:
                continue
            med, mn, _ = time_calls([fn], iters, torch)
            gbs = nbytes / (med * 1e-6) / 1e9
            out[name] = {"us_per_call": round(med, 2), "us_best_slice": round(mn, 2),
                         "bytes": nbytes, "GB_s": round(gbs, 1),
                         "frac_peak": round(gbs / PEAK_GBS, 4)}
            log(f"  {name}: {med:.1f} us, {gbs:.0f} GB/s ({100 * gbs / PEAK_GBS:.1f}% of peak)")
        del x, res, dy, fo, bo, ws
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def cpu_baseline(h, rows):
    """The oracle (double precision, unchanged) on the first `rows` rows of
    the same workload: forward then backward, all host threads."""
    import oracle

    R = min(rows, M_BIG)
    sub = {k: (v[:R] if v.ndim == 2 else v) for k, v in h.items()}
    threads = oracle.default_threads()
    oracle._load()
    t0 = time.perf_counter()
    f = oracle.norm_fwd(sub["x"], sub["bias"], sub["residual"], sub["gamma"], sub["beta"], 1e-5,
                        nthreads=threads)
    oracle.norm_bwd(sub["dy"], f["u"], sub["gamma"], f["mean"], f["rstd"], 1e-5,
                    nthreads=threads)
    sec = time.perf_counter() - t0
    nbytes = fwd_bytes(R, N_BIG) + bwd_bytes(R, N_BIG)
    log(f"cpu oracle: {R} rows in {sec:.2f}s on {threads} threads")
    # one thread on a sixteenth of those rows
    R1 = max(1, R // 16)
    t0 = time.perf_counter()
    f1 = oracle.norm_fwd(sub["x"][:R1], sub["bias"], sub["residual"][:R1], sub["gamma"],
                         sub["beta"], 1e-5, nthreads=1)
    oracle.norm_bwd(sub["dy"][:R1], f1["u"], sub["gamma"], f1["mean"], f1["rstd"], 1e-5,
                    nthreads=1)
    sec1 = time.perf_counter() - t0
    log(f"cpu oracle: {R1} rows in {sec1:.2f}s on 1 thread")
    return {"value": round(nbytes / sec / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"first {R} of {M_BIG} rows of the same workload (fwd + bwd), "
                      f"{sec:.2f} s wall, same algorithmic-byte accounting",
            "single_thread_value": round((fwd_bytes(R1, N_BIG) + bwd_bytes(R1, N_BIG)) / sec1 / 1e9, 3),
            "single_thread_sample": f"first {R1} rows on 1 thread, {sec1:.2f} s wall"}


if __name__ == "__main__":
    main()
