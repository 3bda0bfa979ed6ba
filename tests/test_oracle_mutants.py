"""The oracle's pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a temporary copy of ``oracle/oracle.c`` (on
the CPU only), builds it, and runs ``test_oracle.py`` against that build; at
least one pin has to fail.  The committed oracle is never altered.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("variance divides by N-1", "v /= (double)N;", "v /= (double)(N - 1);"),
    ("mean divides by N+1", "mean = s / (double)N;", "mean = s / (double)(N + 1);"),
    ("eps dropped in forward", "rstd = 1.0 / sqrt(v + c->eps);", "rstd = 1.0 / sqrt(v);"),
    ("eps outside the square root", "rstd = 1.0 / sqrt(v + c->eps);",
     "rstd = 1.0 / sqrt(v) + c->eps;"),
    ("beta sign", "double yv = (u[j] - mean) * rstd * g + b;",
     "double yv = (u[j] - mean) * rstd * g - b;"),
    ("gamma ignored", "double yv = (u[j] - mean) * rstd * g + b;",
     "double yv = (u[j] - mean) * rstd + b;"),
    ("residual subtracted", "elem_or(c->res, c->dtype, i * N + j, 0.0);",
     "-elem_or(c->res, c->dtype, i * N + j, 0.0);"),
    ("bias indexed by row", "elem_or(c->bias, c->dtype, j, 0.0)",
     "elem_or(c->bias, c->dtype, i % N, 0.0)"),
    ("sum not rounded before normalising", "u[j] = round_io(t, c->dtype);", "u[j] = t;"),
    ("RMS uses |u| not u^2", "s += u[j] * u[j];", "s += fabs(u[j]);"),
    ("bf16 keeps 9 bits", "int q = e - 8;", "int q = e - 9;"),
    ("bf16 truncates", "nearbyint(ldexp(fabs(v), -q))", "floor(ldexp(fabs(v), -q))"),
    ("bf16 ties away from zero", "nearbyint(ldexp(fabs(v), -q))", "round(ldexp(fabs(v), -q))"),
    ("amax of unrounded y", "double a = fabs(round_io(yv, c->dtype));", "double a = fabs(yv);"),
    ("dx loses the mean(g) term", "double c2 = c->is_rms ? 0.0 : s_g / (double)N;",
     "double c2 = 0.0;"),
    ("dx sign of the xhat term", "c->rstd[i] * (g - c2 - xhat_of(c, i, j) * c1)",
     "c->rstd[i] * (g - c2 + xhat_of(c, i, j) * c1)"),
    ("dx missing rstd", "c->rstd[i] * (g - c2 - xhat_of(c, i, j) * c1)",
     "(g - c2 - xhat_of(c, i, j) * c1)"),
    ("dx without gamma",
     "double g = elem(c->dy, c->dtype, i * N + j) *\n                       weight_of(c->gamma, c->dtype, c->zero_centered, j);\n            s_gx",
     "double g = elem(c->dy, c->dtype, i * N + j);\n            s_gx"),
    ("dgamma without xhat", "double tg = d * xhat_of(c, i, j);", "double tg = d;"),
    ("dbeta sums squares", "sb += d;", "sb += d * d;"),
    ("RMS recompute drops eps", "c->rstd[i] = 1.0 / sqrt(s / (double)c->N + c->eps);",
     "c->rstd[i] = 1.0 / sqrt(s / (double)c->N);"),
    ("xhat ignores the mean", "(xv - c->mean[i]) * c->rstd[i]", "xv * c->rstd[i]"),
    ("dbias sums dy instead of dx", "double t = c->dx[i * c->N + j];",
     "double t = elem(c->dy, c->dtype, i * c->N + j);"),
    ("e4m3 keeps 4 mantissa bits", "int q = e - 4;", "int q = e - 5;"),
    ("e4m3 subnormal spacing 2^-10", "q = -9; /* subnormal spacing */", "q = -10;"),
    ("e4m3 without saturation", "if (r > 448.0)\n        r = 448.0;", ""),
    ("e4m3 truncates", "double r = ldexp(nearbyint(ldexp(a, -q)), q);",
     "double r = ldexp(floor(ldexp(a, -q)), q);"),
    ("e4m3 product in double", "const float p = v[i] * scale;",
     "const double p = (double)v[i] * (double)scale;"),
    ("zero-centred weight not rounded", "return zero_centered ? round_io(1.0 + g, dtype) : g;",
     "return zero_centered ? 1.0 + g : g;"),
    ("zero-centred weight ignored in dx",
     "double g = elem(c->dy, c->dtype, i * N + j) *\n                       weight_of(c->gamma, c->dtype, c->zero_centered, j);\n            s_gx",
     "double g = elem(c->dy, c->dtype, i * N + j) *\n                       elem_or(c->gamma, c->dtype, j, 1.0);\n            s_gx"),
    ("mean epilogue divides by N", "outs[k][j] /= (double)M;", "outs[k][j] /= (double)N;"),
    ("softmax sum skips the first column", "for (int64_t j = 0; j < N; ++j)\n            s += exp(",
     "for (int64_t j = 1; j < N; ++j)\n            s += exp("),
    ("softmax numerator without the max",
     "c->y[i * N + j] = exp(elem(c->x, c->dtype, i * N + j) - m) / s;",
     "c->y[i * N + j] = exp(elem(c->x, c->dtype, i * N + j)) / s;"),
    ("dgamma_l2 scaled up", "qg += tg * tg;", "qg += 1e6 * tg * tg;"),
    ("dgamma_l2 sums |terms|", "qg += tg * tg;", "qg += fabs(tg);"),
    ("dgamma_l2 from dbeta's terms", "qg += tg * tg;", "qg += d * d;"),
    ("dbeta_l2 scaled up", "qb += d * d;", "qb += 4.0 * d * d;"),
    ("dbias_l2 scaled up", "q += t * t;", "q += 1e6 * t * t;"),
    ("dbias skips the last row", "for (int64_t i = 0; i < c->M; ++i) {\n            double t = c->dx",
     "for (int64_t i = 0; i + 1 < c->M; ++i) {\n            double t = c->dx"),
]


def _build_mutant(tmp, idx, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutant text not found: {old!r}"
    mutated = src.replace(old, new, 1)
    c_path = os.path.join(tmp, f"m{idx}.c")
    so_path = os.path.join(tmp, f"m{idx}.so")
    with open(c_path, "w") as fh:
        fh.write(mutated)
    subprocess.run(["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared", "-pthread",
                    "-ffp-contract=off", c_path, "-o", so_path, "-lm"], check=True,
                   capture_output=True)
    return so_path


def _pins_fail(so_path):
    env = dict(os.environ, NORMFUSE_ORACLE_LIB=so_path, OMP_NUM_THREADS="1")
    p = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return p.returncode != 0, p.stdout[-400:]


def test_every_mutant_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        sos = [_build_mutant(tmp, i, old, new) for i, (_, old, new) in enumerate(MUTANTS)]
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(_pins_fail, sos))
    survivors = [MUTANTS[i][0] for i, (failed, _) in enumerate(results) if not failed]
    assert not survivors, f"pins did not catch: {survivors}"


@pytest.mark.parametrize("name,old,new", MUTANTS[:1])
def test_unmutated_oracle_passes_the_same_runner(name, old, new):
    """Control: the same runner on the committed oracle passes."""
    import oracle
    oracle._load()
    failed, tail = _pins_fail(os.path.join(ROOT, "oracle", "liboracle.so"))
    assert not failed, tail
