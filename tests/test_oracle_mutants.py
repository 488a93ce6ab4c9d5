"""The pins of the oracle must catch plausible mistakes in it.

Each mutant is a copy of oracle/oracle.c with one mistake planted (a dropped
term, a wrong sign, bias, index or operand, a wrong rounding), compiled on the
CPU into a temporary directory.  The pin suite (tests/test_oracle_pins.py,
without the golden-file regression, which the oracle itself wrote) is run
against each mutant through ORACLE_LIB and must fail; against an unmodified
copy built the same way it must pass.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement, occurrences replaced)
MUTANTS = [
    ("e4m3 exponent bias", "else        mag = ldexp(1.0 + (double)m / 8.0, e - 7);",
     "else        mag = ldexp(1.0 + (double)m / 8.0, e - 8);", 1),
    ("e4m3 subnormal step", "mag = ldexp((double)m / 8.0, -6);", "mag = ldexp((double)m / 8.0, -7);", 1),
    ("e8m0 bias", "return ldexp(1.0, (int)s - 127);", "return ldexp(1.0, (int)s - 126);", 1),
    ("dequant drops the scale", "return oracle_e4m3_value(code) * oracle_e8m0_value(scale);",
     "return oracle_e4m3_value(code);", 1),
    ("bf16 rounds ties away", "(lower == 0x8000u && (upper & 1u))", "(lower == 0x8000u)", 1),
    ("bf16 truncates", "if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1;", "", 1),
    ("silu sign", "if (g >= 0) return g / (1.0 + exp(-g));", "if (g >= 0) return g / (1.0 + exp(g));", 1),
    ("gate and up swapped",
     "double a = oracle_silu(g) * u;\n        act[t]", "double a = oracle_silu(u) * g;\n        act[t]", 1),
    ("up row uses the gate scale", "u += oracle_dequant(cu[h], su[h / 32]) * xv;\n        }\n        double a = oracle_silu(g)",
     "u += oracle_dequant(cu[h], sg[h / 32]) * xv;\n        }\n        double a = oracle_silu(g)", 1),
    ("gate/up drops the last term", "        for (long h = 0; h < H; ++h) {\n            double xv = oracle_bf16_value(x[b * H + h]);\n            g += oracle_dequant(cg[h], sg[h / 32]) * xv;\n            u += oracle_dequant(cu[h], su[h / 32]) * xv;\n        }\n        double a = oracle_silu(g) * u;\n        act[t]",
     "        for (long h = 0; h < H - 1; ++h) {\n            double xv = oracle_bf16_value(x[b * H + h]);\n            g += oracle_dequant(cg[h], sg[h / 32]) * xv;\n            u += oracle_dequant(cu[h], su[h / 32]) * xv;\n        }\n        double a = oracle_silu(g) * u;\n        act[t]", 1),
    ("down ignores the router weight", "acc += (double)w[b * K + k] * part;", "acc += part;", 1),
    ("down uses slot 0's router weight", "acc += (double)w[b * K + k] * part;", "acc += (double)w[b * K] * part;", 1),
    ("down reads slot 0's intermediate", "const uint16_t *a = act + (b * K + k) * (long)I;",
     "const uint16_t *a = act + (b * K) * (long)I;", 1),
    ("down row reversed", "const uint8_t *c = wd + (e * H + h) * (long)I;",
     "const uint8_t *c = wd + (e * H + (H - 1 - h)) * (long)I;", 1),
    ("e4m3 encode rounds ties up", "if (r > 0.5 || (r == 0.5 && fmod(m, 2.0) == 1.0)) m += 1.0;",
     "if (r >= 0.5) m += 1.0;", 2),
    ("mx shared exponent off by one", "sb = (ex - 1) - 8 + 127;", "sb = ex - 8 + 127;", 1),
    ("mx scale from amax / 448 rounded up", "sb = (ex - 1) - 8 + 127;",
     "sb = (int)ceil(log2(amax / 448.0)) + 127;", 1),
    ("mx scale byte not clamped to 254", "if (sb > 254) sb = 254;", "", 1),
    ("conventional keeps x unrounded", "for (long h = 0; h < H; ++h) xq[h] = oracle_dequant(xc[h], xs[h / 32]);",
     "for (long h = 0; h < H; ++h) xq[h] = xv[h];", 1),
    ("conventional skips the per-expert BF16",
     "y[b * H + h] += (double)w[b * K + k] * oracle_bf16_value(oracle_bf16_rne(oracle_round_f32(o)));",
     "y[b * H + h] += (double)w[b * K + k] * o;", 1),
    ("router ties take the higher index", "if (best < 0 || l[e] > l[best]) best = e;",
     "if (best < 0 || l[e] >= l[best]) best = e;", 1),
    ("router softmax misses the last choice", "for (int k = 0; k < K; ++k) z += exp((double)l[ids[b * K + k]] - lmax);",
     "for (int k = 0; k < K - 1; ++k) z += exp((double)l[ids[b * K + k]] - lmax);", 1),
]


def _build(src_text: str, out: str):
    path = out[:-3] + ".c"
    with open(path, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c11", path, "-o", out,
                    "-lm"], check=True, capture_output=True)


def _pins_pass(lib: str) -> bool:
    env = dict(os.environ, ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-k", "not golden",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode == 0


def test_every_mutant_is_caught(tmp_path):
    src = open(SRC).read()
    jobs = [("unmodified", src)]
    for name, old, new, count in MUTANTS:
        assert src.count(old) == count, f"mutation target for {name!r} not found {count} time(s) in oracle.c"
        jobs.append((name, src.replace(old, new)))

    def run(job):
        i, (name, text) = job
        lib = str(tmp_path / f"mutant{i}.so")
        _build(text, lib)
        return name, _pins_pass(lib)

    with ThreadPoolExecutor(4) as pool:
        results = dict(pool.map(run, enumerate(jobs)))
    assert results.pop("unmodified"), "the pin suite fails on an unmodified copy"
    missed = [n for n, passed in results.items() if passed]
    assert not missed, f"pins did not catch: {missed}"
