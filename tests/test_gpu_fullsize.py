"""Full-size parity: every element of the 300M-element workloads against the
oracle, in the configuration the benchmark times.

The Baidu Ring-Allreduce article's workload is a language model of about 300
million parameters, a 1.2 GB binary32 gradient.  Two plans run on it here:
  - 40 ranks, 64 equal buckets issued last-first, each gated by its own ready
    event on the plan's side stream (the benchmark's headline step), in the
    plan's own form of the fused pass (two kernels at this size);
  - 8 ranks, one bucket, mean (one kernel).
Inputs are generated in HBM by the shared seeded generator.  After the plan
has run, the oracle walks the same schedule bucket by bucket (or window by
window) over host copies of the regenerated inputs, and every element of rank
0 is compared bit for bit; every other rank is compared with rank 0 on the
device.  The normwise error against the binary64 sum of the same inputs is
accumulated over the whole buffer.
"""
import numpy as np
import pytest

import oracle as orc
import sgd_gradient_all_amd as ddl
import synth
from synth.workloads import WORKLOADS

from _helpers import KINDS, OPS, ddl_topo, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def device_inputs(w):
    bufs = [torch.empty(w.n, dtype=torch.float32, device="cuda") for _ in range(w.P)]
    for r, b in enumerate(bufs):
        synth.fill_device(b.data_ptr(), w.n, synth.F32, w.dist, w.seed, r, sigma=w.sigma)
    torch.cuda.synchronize()
    return bufs


def ranks_identical(bufs):
    ref = bufs[0].view(torch.int32)
    return all(torch.equal(b.view(torch.int32), ref) for b in bufs[1:])


def check_windows(w, bufs, windows, buckets):
    """Every element of rank 0 in each window (lo, hi) against the oracle's
    walk of the plan's bucket list restricted to that window; returns the
    normwise relative error against the binary64 sum over all windows."""
    num = den = 0.0
    scratch = torch.empty(max(hi - lo for lo, hi in windows), dtype=torch.float32,
                          device="cuda")
    for i, (lo, hi) in enumerate(windows):
        cnt = hi - lo
        host = []
        for r in range(w.P):
            synth.fill_device(scratch.data_ptr(), cnt, synth.F32, w.dist, w.seed, r, first=lo,
                              sigma=w.sigma)
            host.append(scratch[:cnt].cpu().numpy())
        want = [x.copy() for x in host]
        orc.allreduce(want, op=OPS[w.op], kind=KINDS[w.topo], k=w.k, rows=w.rows, cols=w.cols,
                      buckets=buckets, window=(lo, hi), count_only_n=w.n)
        got = bufs[0][lo:hi].cpu().numpy()
        if got.tobytes() != want[0].tobytes():
            bad = int(np.flatnonzero(got.view(np.uint32) != want[0].view(np.uint32))[0])
            raise AssertionError(f"{w.name}: window {i} [{lo}, {hi}) differs from the oracle "
                                 f"at element {lo + bad}")
        y64 = orc.sum_f64(host, op=OPS[w.op])
        d = got.astype(np.float64) - y64
        num += float(np.dot(d, d))
        den += float(np.dot(y64, y64))
    return (num / den) ** 0.5


def test_headline_timed_plan_every_element():
    """The benchmark's step -- 40 ranks, 64 event-gated buckets, the plan's
    own fused form -- against the oracle, every element, bucket by bucket."""
    w = WORKLOADS["ring_p40_300m_64b"]
    say(f"case full size {w.name}: device inputs ({w.P} x {w.n})")
    bufs = device_inputs(w)
    buckets = w.bucket_list()
    stream = torch.cuda.current_stream()
    events = [torch.cuda.Event() for _ in buckets]
    for e in events:
        e.record(stream)
    plan = ddl.Plan(w.P, w.n, w.dtype, w.op, ddl_topo(w), buckets, "fused")
    assert plan.fused_passes() == 2
    say(f"case full size {w.name}: fused, {plan.fused_passes()} kernels per pass")
    plan.execute(bufs, events=events, stream=stream)
    torch.cuda.synchronize()
    plan.destroy()
    assert ranks_identical(bufs)
    say(f"case full size {w.name}: oracle over {len(buckets)} buckets")
    err = check_windows(w, bufs, [(off, off + cnt) for off, cnt in buckets], buckets)
    assert err <= 1e-6, err
    del bufs
    torch.cuda.empty_cache()


def test_eight_ranks_whole_buffer():
    """40-rank's smaller sibling: 8 ranks, one 300M bucket, mean, the plan's
    own form (one kernel), every element against the oracle in windows."""
    w = WORKLOADS["ring_p8_300m_mean"]
    say(f"case full size {w.name}: device inputs ({w.P} x {w.n})")
    bufs = device_inputs(w)
    plan = ddl.Plan(w.P, w.n, w.dtype, w.op, ddl_topo(w), w.bucket_list(), "fused")
    say(f"case full size {w.name}: fused, {plan.fused_passes()} kernel(s) per pass")
    plan.execute(bufs)
    torch.cuda.synchronize()
    plan.destroy()
    assert ranks_identical(bufs)
    step = 25_000_000
    windows = [(lo, min(lo + step, w.n)) for lo in range(0, w.n, step)]
    say(f"case full size {w.name}: oracle over {len(windows)} windows")
    err = check_windows(w, bufs, windows, w.bucket_list())
    assert err <= 1e-6, err
    del bufs
    torch.cuda.empty_cache()
