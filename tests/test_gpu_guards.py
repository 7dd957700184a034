"""Guard regions and serialised launches.

- Poison guards: every rank buffer (and every weight replica of the SGD
  step) sits inside a larger allocation whose bytes before and after it hold
  a NaN sentinel.  After the all-reduce -- every topology, both element
  types, every form -- the buffers equal the oracle's walk and every guard
  byte is untouched: no kernel reads or writes outside [0, n).
- Serialised launches: the same event-gated, multi-stream plans run in a
  child process with AMD_SERIALIZE_KERNEL=3 (every launch waits for the one
  before it and is waited for), where a missing dependency between streams
  could not hide behind timing; the results equal the oracle's.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle as orc
import sgd_gradient_all_amd as ddl
from synth.workloads import Workload

from _helpers import ddl_topo, host_inputs, oracle_full, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SENTINEL = {"f32": (np.uint32, 0x7FC0DEAD), "f16": (np.uint16, 0x7E5A)}
TDT = {"f32": torch.float32, "f16": torch.float16}
IDT = {"f32": torch.int32, "f16": torch.int16}

CASES = [
    Workload("ring-P5", 5, 100_003, "f32", "sum", "ring", dist="normal", sigma=1e-2, seed=81,
             buckets=[(60_000, 40_003), (0, 60_000)]),
    Workload("mring-P6-k3-f16", 6, 77_777, "f16", "mean", "multiring", k=3, dist="normal",
             sigma=1e-2, seed=82),
    Workload("torus-2x3", 6, 50_001, "f32", "mean", "torus2d", rows=2, cols=3, dist="normal",
             sigma=1e-2, seed=83, buckets=[(25_000, 25_001), (1_000, 24_000), (0, 1_000)]),
    Workload("ring-P40-tiny", 40, 6_000, "f32", "mean", "ring", dist="normal", sigma=1e-2,
             seed=84, buckets=[(5_000, 1_000), (2_000, 3_000), (0, 2_000)]),
    Workload("torus-4x4-f16", 16, 300_001, "f16", "mean", "torus2d", rows=4, cols=4,
             dist="normal", sigma=1e-2, seed=85),
]

FRONT, BACK = 1024, 1027   # guard elements before (16-byte multiple) and after


def guarded(w, host):
    """Allocations holding each rank's n elements between two NaN guards;
    returns (allocations, views of the n elements)."""
    allocs, views = [], []
    sdt, bits = SENTINEL[w.dtype]
    for h in host:
        a = torch.empty(FRONT + w.n + BACK, dtype=TDT[w.dtype], device="cuda")
        a.view(IDT[w.dtype]).fill_(bits)   # the pattern fits the signed type: a positive value
        a[FRONT:FRONT + w.n].copy_(torch.from_numpy(h))
        allocs.append(a)
        views.append(a[FRONT:FRONT + w.n])
    return allocs, views


def check_guards(w, allocs, what):
    sdt, bits = SENTINEL[w.dtype]
    for r, a in enumerate(allocs):
        raw = a.cpu().numpy().view(sdt)
        assert (raw[:FRONT] == bits).all(), (w.name, what, r, "front guard")
        assert (raw[FRONT + w.n:] == bits).all(), (w.name, what, r, "back guard")


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("mode", ["fused1", "fused2", "step1", "step2"])
def test_guards_untouched_by_the_allreduce(w, mode):
    say(f"case guards {w.name} {mode}")
    g = host_inputs(w)
    ref = [x.copy() for x in g]
    oracle_full(w, ref)
    allocs, views = guarded(w, g)
    torch.cuda.synchronize()
    stepwise = mode.startswith("step")
    plan = ddl.Plan(w.P, w.n, w.dtype, w.op, ddl_topo(w), w.bucket_list(),
                    "stepwise" if stepwise else "fused")
    if stepwise:
        plan.set_step_form(int(mode[-1]))
    else:
        plan.set_fused_passes(1 if mode == "fused1" else 2)
    stream = torch.cuda.current_stream()
    events = [torch.cuda.Event() for _ in w.bucket_list()]
    for e in events:
        e.record(stream)
    plan.execute([v.data_ptr() for v in views], events=events, stream=stream)
    torch.cuda.synchronize()
    plan.destroy()
    for r, v in enumerate(views):
        assert v.cpu().numpy().tobytes() == ref[r].tobytes(), (w.name, mode, r)
    check_guards(w, allocs, mode)


@pytest.mark.parametrize("mode,keep", [("fused1", True), ("fused1", False), ("fused2", True),
                                       ("fused2", False), ("step1", True), ("step2", True)])
def test_guards_untouched_by_the_sgd_step(mode, keep):
    """The SGD step's weight replicas between guards as well."""
    w = CASES[0]
    say(f"case guards sgd {mode} keep={keep}")
    g = host_inputs(w)
    ref = [x.copy() for x in g]
    oracle_full(w, ref)
    w0 = np.linspace(-1.0, 1.0, w.n, dtype=np.float32)
    want = [w0.copy() for _ in range(w.P)]
    lr = 0.03125
    orc.sgd(want, ref[0], lr)
    allocs, views = guarded(w, g)
    wallocs, wviews = guarded(Workload("wts", w.P, w.n, "f32", "sum", "ring"), [w0] * w.P)
    torch.cuda.synchronize()
    plan = ddl.Plan(w.P, w.n, w.dtype, w.op, ddl_topo(w), w.bucket_list(),
                    "stepwise" if mode.startswith("step") else "fused")
    if mode.startswith("step"):
        plan.set_step_form(int(mode[-1]))
    else:
        plan.set_fused_passes(1 if mode == "fused1" else 2)
    plan.execute_sgd([v.data_ptr() for v in views], [v.data_ptr() for v in wviews], lr,
                     keep_grads=keep)
    torch.cuda.synchronize()
    plan.destroy()
    for r in range(w.P):
        assert wviews[r].cpu().numpy().tobytes() == want[r].tobytes(), (mode, keep, r)
        grads = ref[r] if keep else g[r]
        assert views[r].cpu().numpy().tobytes() == grads.tobytes(), (mode, keep, r)
    check_guards(w, allocs, f"sgd {mode}")
    check_guards(Workload("wts", w.P, w.n, "f32", "sum", "ring"), wallocs, f"sgd weights {mode}")


_SERIAL_CHILD = r"""
import sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
import numpy as np
import torch
import sgd_gradient_all_amd as ddl
from synth.workloads import Workload
from _helpers import ddl_topo, host_inputs, oracle_full
cases = [
    Workload("mring", 16, 200_003, "f32", "mean", "multiring", k=4, dist="normal", sigma=1e-2,
             seed=91, buckets=[(i * 12_500, 12_500 if i < 15 else 200_003 - 15 * 12_500)
                               for i in reversed(range(16))]),
    Workload("torus", 16, 100_001, "f16", "mean", "torus2d", rows=4, cols=4, dist="normal",
             sigma=1e-2, seed=92, buckets=[(50_000, 50_001), (0, 50_000)]),
]
stream = torch.cuda.current_stream()
for w in cases:
    g = host_inputs(w)
    ref = [x.copy() for x in g]
    oracle_full(w, ref)
    for mode, passes in (("fused", 1), ("fused", 2), ("stepwise", 0)):
        print("serial case", w.name, mode, passes, flush=True)
        bufs = [torch.from_numpy(x).cuda() for x in g]
        plan = ddl.Plan(w.P, w.n, w.dtype, w.op, ddl_topo(w), w.bucket_list(), mode)
        if passes:
            plan.set_fused_passes(passes)
        plan.set_side_streams(2)
        events = [torch.cuda.Event() for _ in w.bucket_list()]
        for e in events:
            e.record(stream)
        plan.execute(bufs, events=events, stream=stream)
        torch.cuda.synchronize()
        plan.destroy()
        for r in range(w.P):
            assert bufs[r].cpu().numpy().tobytes() == ref[r].tobytes(), (w.name, mode, passes, r)
print("serial ok", flush=True)
"""


def test_serialised_launches_give_the_oracles_bits():
    say("case AMD_SERIALIZE_KERNEL=3 child")
    env = dict(os.environ, AMD_SERIALIZE_KERNEL="3")
    code = _SERIAL_CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=240)
    print(r.stdout[-3000:], r.stderr[-3000:], flush=True)
    assert r.returncode == 0, r.stdout[-1500:] + r.stderr[-1500:]
    assert "serial ok" in r.stdout
