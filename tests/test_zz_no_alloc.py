"""The allocation-free LARS entry point (ddl_plan_execute_lars_noalloc),
called through the C ABI, against the allocating one (ddl_plan_execute_lars)
on the same plan and inputs: gradients, weights and rates bit for bit.  Two
calls in a row, the second on a smaller plan, so that the scratch holds the
first call's partial sums when the second runs."""
import numpy as np
import pytest

import sgd_gradient_all_amd as ddl
import synth

from _helpers import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [
    # (P, bucket sizes in issue order, dtype, topology, mode, weight replicas, events)
    (8, [300_000, 1_000_003, 5, 4096 * 3 + 7, 250_000], "f32", ("ring", 1, 0, 0), "fused", 8,
     True),
    (6, [33_333, 17, 20_000], "f16", ("torus2d", 1, 2, 3), "stepwise", 1, False),
]


def run(P, sizes, dtype, tk, mode, nrep, gated, noalloc):
    n = sum(sizes)
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(int).tolist()
    buckets = list(zip(offs, sizes))[::-1]
    sdt = synth.F32 if dtype == "f32" else synth.F16
    g = [synth.fill_host(n, sdt, "normal", 61, r, sigma=1e-2) for r in range(P)]
    w0 = synth.fill_host(n, synth.F32, "uniform", 62, 0)
    bufs = [torch.from_numpy(x).cuda() for x in g]
    weights = [torch.from_numpy(w0.copy()).cuda() for _ in range(nrep)]
    rates = torch.zeros(len(buckets), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    plan = ddl.Plan(P, n, dtype, "mean", ddl.topo(*tk), buckets, mode)
    # the allocation-free call needs a plan that has run on the device
    scratch_bufs = [torch.zeros_like(b) for b in bufs]
    plan.execute(scratch_bufs, stream=stream)
    torch.cuda.synchronize()
    events = None
    if gated:
        events = [torch.cuda.Event() for _ in buckets]
        for e in events:
            e.record(stream)
    call = plan.execute_lars_noalloc if noalloc else plan.execute_lars
    call(bufs, weights, 0.05, rates_out=rates, events=events, stream=stream)
    torch.cuda.synchronize()
    plan.destroy()
    return ([b.cpu().numpy() for b in bufs], [x.cpu().numpy() for x in weights],
            rates.cpu().numpy())


def test_noalloc_lars_matches_the_allocating_entry_point():
    for i, (P, sizes, dtype, tk, mode, nrep, gated) in enumerate(CASES):
        say(f"case no-alloc LARS call {i}: P={P} n={sum(sizes)} {dtype} {tk[0]} {mode}")
        want = run(P, sizes, dtype, tk, mode, nrep, gated, noalloc=False)
        got = run(P, sizes, dtype, tk, mode, nrep, gated, noalloc=True)
        for what, a, b in (("grads", want[0], got[0]), ("weights", want[1], got[1])):
            for r, (x, y) in enumerate(zip(a, b)):
                assert x.tobytes() == y.tobytes(), (i, what, r)
        assert want[2].tobytes() == got[2].tobytes(), (i, "rates")
        assert np.all(np.isfinite(got[2])) and np.all(got[2] > 0)
