"""Build ``libnormfuse.so`` (the HIP kernels and the C ABI) for gfx950, in-tree.

Every translation unit under ``csrc/`` is compiled by hipcc in parallel into
``_build/`` and linked into ``normalization_ln_fwd_amd/libnormfuse.so``.
The C-ABI layer ``api.cpp`` is compiled a second time with ``NORMFUSE_TUNING``
defined and linked with the same kernel objects into
``libnormfuse_tuning.so``: the test build, whose host code also reads the
``NORMFUSE_*`` tuning overrides from the environment.  Cross-compiles without
a GPU.
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libnormfuse.so")
TUNING_LIB = os.path.join(PKG, "libnormfuse_tuning.so")
TUNING_DEFINE = "-DNORMFUSE_TUNING"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: no packed fp32 VALU instructions are generated.
CFLAGS = ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wall"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src, verbose, defines=()):
    tag = "".join("." + d.lstrip("-D").lower() for d in defines)
    obj = os.path.join(BUILD, os.path.basename(src) + tag + ".o")
    cmd = [HIPCC] + CFLAGS + list(defines) + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in p.stderr.splitlines() if noise not in l)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    api = os.path.join(CSRC, "api.cpp")
    jobs_list = [(s, ()) for s in srcs] + [(api, (TUNING_DEFINE,))]
    with ThreadPoolExecutor(max_workers=min(jobs, len(jobs_list))) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1]), jobs_list))
    product = objs[:len(srcs)]
    tuning = [o for s, o in zip(srcs, product) if s != api] + [objs[-1]]
    _link(product, LIB, verbose)
    _link(tuning, TUNING_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
