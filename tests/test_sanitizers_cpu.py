"""The CPU sanitizer leg: the oracle and the library's host code built with
AddressSanitizer and UndefinedBehaviorSanitizer, and exercised by the CPU
suites that drive them.

  * oracle/oracle.c built by gcc with -fsanitize=address,undefined; the
    oracle's pins (tests/test_oracle.py) run against that build;
  * csrc/api.cpp (argument checks, planning, norm_describe) compiled by
    hipcc with both sanitizers on its host code only (each -fsanitize= after
    -Xarch_host; device code is not instrumented) and linked with the kernel
    objects; the C-ABI checks (tests/test_abi_cpu.py) run against it.

Each runs in a subprocess with the sanitizer runtime preloaded (the Python
interpreter is not instrumented) and must pass; a copy with one planted
memory error must abort with a sanitizer report, which shows that the
instrumentation is live (the control runs with output uncaptured, so that
the report is not lost with pytest's capture when the process aborts).  No GPU is used: the ABI checks stop before any
launch.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "oracle.c")
CSRC = os.path.join(ROOT, "normalization_ln_fwd_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG_RT = "/opt/rocm/llvm/lib/clang"
ASAN_OPTIONS = "detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0:abort_on_error=1"
UBSAN_OPTIONS = "halt_on_error=1:print_stacktrace=1"


def _gcc_runtime(name):
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True, check=True).stdout.strip()


def _clang_asan_runtime():
    for ver in sorted(os.listdir(CLANG_RT), reverse=True):
        p = os.path.join(CLANG_RT, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def _run(cmd, env_extra, timeout=600):
    env = dict(os.environ, ASAN_OPTIONS=ASAN_OPTIONS, UBSAN_OPTIONS=UBSAN_OPTIONS,
               OMP_NUM_THREADS="2", **env_extra)
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


def _build_oracle(src_text, out):
    c = out + ".c"
    with open(c, "w") as fh:
        fh.write(src_text)
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared",
                    "-pthread", "-ffp-contract=off", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", c, "-o", out,
                    "-lm"], check=True, capture_output=True)
    return out


def _oracle_env(so):
    pre = f"{_gcc_runtime('libasan.so')} {_gcc_runtime('libubsan.so')}"
    return {"LD_PRELOAD": pre, "NORMFUSE_ORACLE_LIB": so}


def test_oracle_under_asan_and_ubsan():
    src = open(ORACLE_C).read()
    with tempfile.TemporaryDirectory() as tmp:
        so = _build_oracle(src, os.path.join(tmp, "liboracle_san.so"))
        p = _run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                  os.path.join(ROOT, "tests", "test_oracle.py")], _oracle_env(so))
        assert p.returncode == 0, p.stdout[-2000:] + p.stderr[-3000:]
        # control: one row read past the end of dy in the column sums
        old = "for (int64_t i = 0; i < c->M; ++i) {\n            double d = elem(c->dy"
        assert old in src
        bad = _build_oracle(src.replace(old, old.replace("i < c->M", "i <= c->M")),
                            os.path.join(tmp, "liboracle_planted.so"))
        p = _run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                  os.path.join(ROOT, "tests", "test_oracle.py"), "-k", "column_sums_brute", "-s"],
                 _oracle_env(bad))
        assert p.returncode != 0 and "AddressSanitizer" in (p.stdout + p.stderr), \
            p.stdout[-1500:] + p.stderr[-1500:]


def _kernel_objects():
    """The kernel objects of the library build (built by the package build
    when absent)."""
    from normalization_ln_fwd_amd import build as b
    objs = [os.path.join(b.BUILD, os.path.basename(s) + ".o") for s in b.sources()
            if not s.endswith("api.cpp")]
    if not all(os.path.exists(o) for o in objs):
        b.build()
    return objs


def _build_api(api_text, tmp, name):
    src = os.path.join(tmp, name + ".cpp")
    with open(src, "w") as fh:
        fh.write(api_text)
    obj = os.path.join(tmp, name + ".o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
           "-fno-omit-frame-pointer"]
    subprocess.run([HIPCC, "-x", "hip", "-std=c++17", "-O1", "-g", "-fPIC",
                    "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops", "-DNORMFUSE_TUNING"] + san +
                   ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", src, "-o", obj],
                   check=True, capture_output=True)
    so = os.path.join(tmp, "lib" + name + ".so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host",
                    "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
                    "-shared-libsan", "-o", so, obj] + _kernel_objects(),
                   check=True, capture_output=True)
    return so


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_argument_checks_under_asan_and_ubsan():
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("clang's ASan runtime not found")
    api = open(os.path.join(CSRC, "api.cpp")).read()
    with tempfile.TemporaryDirectory() as tmp:
        so = _build_api(api, tmp, "normfuse_san")
        p = _run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                  os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                 {"LD_PRELOAD": rt, "NORMFUSE_TEST_LIB": so})
        assert p.returncode == 0, p.stdout[-2000:] + p.stderr[-3000:]
        # control: a heap overflow planted in norm_status_string for one code
        old = "const char *norm_status_string(norm_status_t st)\n{"
        assert old in api
        planted = api.replace(old, old + "\n    if (st == 12345) { char *q = static_cast<char *>("
                              "std::malloc(4)); q[4] = 1; std::free(q); }")
        bad = _build_api(planted, tmp, "normfuse_planted")
        code = ("import normalization_ln_fwd_amd as nf; import sys; "
                f"lib = nf.load({bad!r}); lib.norm_status_string(12345)")
        p = _run([sys.executable, "-c", code], {"LD_PRELOAD": rt})
        # either sanitizer may report it first (UBSan's object-size check does)
        out = p.stdout + p.stderr
        assert p.returncode != 0 and ("AddressSanitizer" in out or
                                      "UndefinedBehaviorSanitizer" in out), \
            p.stdout[-1500:] + p.stderr[-1500:]
