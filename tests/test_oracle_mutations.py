"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of oracle/mra_oracle.c (on the CPU),
builds it, and runs the pin suite against it; the suite has to fail.  The
mistakes are the ones a reader of the pages could make: a dropped term, a
wrong sign or index, a transposed operand, a misread of the selection rule.
"""
import concurrent.futures
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mra_oracle.c")

MUTANTS = {
    "low-res weight drops cnt_j": ("double w = (double)cnt[j] * exp(s_lo[j] - shift);",
                                   "double w = exp(s_lo[j] - shift);"),
    "ranks raw logits, not row-normalised": ("s = (variant & 1) ? S[(int64_t)i * nb + j] : S[(int64_t)i * nb + j] - m;",
                                            "s = S[(int64_t)i * nb + j];"),
    "raw-logit ranking ignored": ("s = (variant & 1) ? S[(int64_t)i * nb + j] : S[(int64_t)i * nb + j] - m;",
                                  "s = S[(int64_t)i * nb + j] - m;"),
    "transposed low-res logits": ("acc = fmaf(qhat[(int64_t)i * d + c], khat[(int64_t)j * d + c], acc);",
                                  "acc = fmaf(qhat[(int64_t)j * d + c], khat[(int64_t)i * d + c], acc);"),
    "ties go to the larger flat index": ("return x->flat < y->flat ? -1 : (x->flat > y->flat ? 1 : 0);",
                                         "return x->flat > y->flat ? -1 : (x->flat < y->flat ? 1 : 0);"),
    "diagonal band too wide": (": dist <= prior_diag / 2", ": dist < prior_diag"),
    "exact-width band leans left": ("(j - i >= -((prior_diag - 1) / 2) && j - i <= prior_diag / 2)",
                                    "(j - i >= -(prior_diag / 2) && j - i <= (prior_diag - 1) / 2)"),
    "exact-width band option ignored": ("int32_t in_band = (variant & 2) ?", "int32_t in_band = 0 ?"),
    "first-n prior on rows only": ("if (j < prior_first)\n                    s = s + MRA_PRIOR_BIAS;", ""),
    "masked keys not skipped": ("s_hi[u] = -INFINITY;\n                    if (mask && !mask[u])\n"
                                "                        continue;", "s_hi[u] = -INFINITY;"),
    "low-res also covers selected blocks": ("if (!chosen[(int64_t)i * nb + j] && cnt[j] > 0) {",
                                            "if (cnt[j] > 0) {"),
    "no 1/sqrt(d) on exact logits": ("s_hi[u] = tau * dot;", "s_hi[u] = dot;"),
    "exponent sign flipped": ("double w = exp(s_hi[u] - shift);", "double w = exp(shift - s_hi[u]);"),
    "budget not capped": ("return k < cap ? k : cap;", "return k;"),
    "mean divides by 32, not the count": ("xhat[(int64_t)i * d + ch] = c > 0 ? acc / (float)c : 0.0f;",
                                          "xhat[(int64_t)i * d + ch] = c > 0 ? acc / 32.0f : 0.0f;"),
    "fp64 low-res values use the wrong pooled tensor": ("oracle_pool_f64(N, d, v, mask, vh64);",
                                                         "oracle_pool_f64(N, d, k, mask, vh64);"),
    "padded query rows not zeroed": ("if (mask && !mask[t])\n                continue; /* reading R12",
                                     "if (0)\n                continue; /* reading R12"),
    "BigBird window of one block": ("const int window = I - J <= 1 && J - I <= 1;", "const int window = I == J;"),
    "BigBird last block not global": ("const int global = I == 0 || I == nbb - 1 || J == 0 || J == nbb - 1;",
                                      "const int global = I == 0 || J == 0;"),
    "BigBird random picks ignored": ("                att[(int64_t)I * nbb + J] = 1;\n", "                (void)0;\n"),
    "backward drops D_t": ("const double ds = P * (dP - D);", "const double ds = P * dP;"),
    "backward drops tau on dk": ("dk[(int64_t)u * d + c] += tau * ds * (double)q[(int64_t)t * d + c];",
                                 "dk[(int64_t)u * d + c] += ds * (double)q[(int64_t)t * d + c];"),
    "backward skips the mean's 1/cnt": ("const double inv = 1.0 / (double)cnt[b];", "const double inv = 1.0;"),
    "backward low-res query gradient uses qhat": (
        "dqh[(int64_t)i * d + c] += tau * ds * kh64[(int64_t)j * d + c];",
        "dqh[(int64_t)i * d + c] += tau * ds * qh64[(int64_t)i * d + c];"),
    "backward drops the low-res value gradient": ("dvh[(int64_t)j * d + c] += Pi * (double)g[c];", ""),
}


def run_mutant(name, old, new, tmp):
    src = open(SRC).read()
    # an expression the backward recomputes from the forward appears in both:
    # the mistake is planted wherever it is written
    assert src.count(old) >= 1, "mutation anchor for %r not found" % name
    path = os.path.join(tmp, "m%d.c" % abs(hash(name)))
    open(path, "w").write(src.replace(old, new))
    so = path[:-2] + ".so"
    subprocess.check_call(["gcc", *oracle.CFLAGS, path, "-o", so, "-lm"])
    env = dict(os.environ, MRA_ORACLE_LIB=so)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda kv: run_mutant(kv[0], *kv[1], tmp), MUTANTS.items()))
    survivors = [n for n, rc in results if rc == 0]
    assert not survivors, "pins missed planted mistakes: %s" % survivors
