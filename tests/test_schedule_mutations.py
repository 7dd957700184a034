"""The host schedule generator's CPU checks bite: each plausible mistake,
planted in a scratch copy of sgd_gradient_all_amd/csrc/schedule.cpp (never in
the library's source), makes the CPU table-replay tests fail.

Every mutant is built host-only with g++ -- plan.cpp and the mutated
schedule.cpp against the fake device of tests/fake_device.inc, no GPU code --
into a temporary shared library; a child process points the binding at it
and runs tests/test_schedule_cpu.py's replays of the step tables and the
fused spans against the oracle.  The unmutated source, built the same way,
passes them.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sgd_gradient_all_amd", "csrc")
SRC = os.path.join(CSRC, "schedule.cpp")

MUTANTS = [
    ("reduce-scatter chunk off by one", "const int c = wrap(x - t, m);",
     "const int c = wrap(x - t + 1, m);", 1),
    ("all-gather chunk off by one", "const int c = wrap(x + 1 - t, m);",
     "const int c = wrap(x - t, m);", 1),
    ("mean on the first reduce step", "t == m - 2 ? last : 0u", "t == 0 ? last : 0u", 1),
    ("fused chain starts one rank late", "chain[i] = ring[(c + i) % P];",
     "chain[i] = ring[(c + i + 1) % P];", 1),
    ("torus fused chain groups by column", "chain[g * C + h] = ((d + g) % R) * C + (c + h) % C;",
     "chain[g * C + h] = ((d + h) % R) * C + (c + g) % C;", 1),
    ("torus column works on its own row-chunk", "const int c = (j + 1) % C;",
     "const int c = j % C;", 1),
    ("torus mean in the row phase", "reduce_scatter(ring.data(), C, bk.off, bk.len, 0, R == 1);",
     "reduce_scatter(ring.data(), C, bk.off, bk.len, 0, true);", 1),
    ("ceiling split", "b[c] = std::min(L, q * (((uint64_t)c * units) / (uint64_t)m));",
     "b[c] = std::min(L, q * (((uint64_t)c * units + (uint64_t)m - 1) / (uint64_t)m));", 1),
]

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
import sgd_gradient_all_amd._ddl as d
d._LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                      "-k", "replay", {testfile!r}]))
"""


def build(schedule_text, lib):
    sched = lib.parent / "schedule.cpp"
    sched.write_text(schedule_text)
    stub = lib.parent / "fake_device.cpp"
    stub.write_text('#include "{}"\n'.format(os.path.join(ROOT, "tests", "fake_device.inc")))
    subprocess.run(["g++", "-std=c++17", "-O1", "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__",
                    "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    str(stub), os.path.join(CSRC, "plan.cpp"), str(sched), "-o", str(lib)],
                   check=True, capture_output=True)


def run_replays(lib):
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=str(lib),
                        testfile=os.path.join(ROOT, "tests", "test_schedule_cpu.py"))
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True,
                          text=True, timeout=600)


def test_unmutated_host_build_passes_the_replays(tmp_path):
    with open(SRC) as f:
        build(f.read(), tmp_path / "libddl_host.so")
    r = run_replays(tmp_path / "libddl_host.so")
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert " passed" in r.stdout


@pytest.mark.parametrize("name,old,new,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_schedule_mistake_fails_a_replay(tmp_path, name, old, new, count):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == count, f"mutation site of {name!r} not found as expected"
    build(text.replace(old, new), tmp_path / "libddl_mutant.so")
    r = run_replays(tmp_path / "libddl_mutant.so")
    assert r.returncode != 0, f"no replay caught: {name}"
