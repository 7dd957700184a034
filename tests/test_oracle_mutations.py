"""The oracle's pins bite: each plausible mistake, planted in a scratch copy
of oracle/ddl_oracle.c (never in the oracle itself), makes at least one pin
fail.

Every mutant is compiled with the oracle's own flags into a temporary
library, and the CPU pin suites (tests/test_oracle_pins.py,
test_oracle_f16.py, test_oracle_lars.py) are run against it through
DDL_ORACLE_LIB; the unmutated source, built the same way, passes them.
"""
import os
import subprocess
import sys

import pytest

import oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ddl_oracle.c")
PINS = [os.path.join(ROOT, "tests", f) for f in
        ("test_oracle_pins.py", "test_oracle_f16.py", "test_oracle_lars.py")]

# (name, text in ddl_oracle.c, replacement, occurrences replaced)
MUTANTS = [
    ("chain starts one rank late", "int c = pmod(x - t, m);", "int c = pmod(x - t + 1, m);", 2),
    ("all-gather sends the wrong chunk", "int c = pmod(x + 1 - t, m);",
     "int c = pmod(x - t, m);", 2),
    ("no mean", "a = a / (float)P;", "a = a;", 1),
    ("mean by a reciprocal multiply", "a = a / (float)P;", "a = a * (1.0f / (float)P);", 1),
    ("mean one step early", "divide && t == m - 2", "divide && t == m - 3", 1),
    ("binary16 mean not rounded through binary32", "a = f2h(h2f(a) / (float)P);",
     "a = f2h(h2f(a) * (1.0f / (float)P));", 1),
    ("torus column works on its own row-chunk", "int c = (j + 1) % C;", "int c = j % C;", 1),
    ("mean applied in the row phase too", "mean && R == 1", "mean", 1),
    ("binary16 ties rounded away from zero",
     "if (frac > 0.5f || (frac == 0.5f && fmodf(fl, 2.0f) == 1.0f))", "if (frac >= 0.5f)", 1),
    ("ceiling split", "uint64_t v = q * (((uint64_t)c * U) / (uint64_t)m);",
     "uint64_t v = q * (((uint64_t)c * U + (uint64_t)m - 1) / (uint64_t)m);", 1),
    ("SGD with a fused multiply-add", "float step = lr * g;\n            weights[r][e] = weights[r][e] - step;",
     "weights[r][e] = fmaf(-lr, g, weights[r][e]);", 1),
    ("SGD step added instead of subtracted",
     "float step = lr * g;\n            weights[r][e] = weights[r][e] - step;",
     "float step = lr * g;\n            weights[r][e] = weights[r][e] + step;", 1),
    ("LARS without eps", "trust = coeff * sqrt(W) / (sqrt(G) + eps);",
     "trust = coeff * sqrt(W) / sqrt(G);", 1),
    ("LARS without the coefficient", "trust = coeff * sqrt(W) / (sqrt(G) + eps);",
     "trust = sqrt(W) / (sqrt(G) + eps);", 1),
    ("LARS rate rounded in binary32 before the product",
     "rate[l] = (float)((double)lr * trust);", "rate[l] = lr * (float)trust;", 1),
    ("LARS trust 0 for a zero layer", "double trust = 1.0;", "double trust = 0.0;", 1),
]


def build(src_text, path):
    c = path.with_suffix(".c")
    c.write_text(src_text)
    subprocess.run(["gcc", *orc.CFLAGS, "-I", os.path.join(ROOT, "oracle"), "-o", str(path),
                    str(c), "-lm"], check=True,
                   capture_output=True)


def run_pins(lib):
    env = dict(os.environ, DDL_ORACLE_LIB=str(lib))
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                           "-p", "no:cacheprovider", *PINS], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=600)


def test_unmutated_build_passes_the_pins(tmp_path):
    with open(SRC) as f:
        build(f.read(), tmp_path / "liboracle_same.so")
    r = run_pins(tmp_path / "liboracle_same.so")
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name,old,new,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(tmp_path, name, old, new, count):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == count, f"mutation site of {name!r} not found as expected"
    build(text.replace(old, new), tmp_path / "liboracle_mutant.so")
    r = run_pins(tmp_path / "liboracle_mutant.so")
    assert r.returncode != 0, f"no pin caught: {name}"
