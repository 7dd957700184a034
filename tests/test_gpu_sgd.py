"""GPU parity of the SGD step fused into the all-reduce's epilogue.

Expected values: the oracle's all-reduce walk, then its plain SGD step
w - lr * y on every replica (binary32, two roundings).  Bit for bit.
"""
import numpy as np
import pytest

import oracle as orc
import sgd_gradient_all_amd as ddl
import synth
from synth.workloads import WORKLOADS, Workload

from _helpers import ddl_topo, host_inputs, oracle_at, oracle_full, say, synth_dtype

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TORCH_DT = {"f32": torch.float32, "f16": torch.float16}

CASES = [
    Workload("ring-P5", 5, 12_347, "f32", "mean", "ring", dist="normal", sigma=1e-2, seed=41),
    Workload("ring-P1", 1, 5_000, "f32", "mean", "ring", dist="normal", sigma=1e-2, seed=42),
    Workload("mring-P16-k4-f16", 16, 70_001, "f16", "mean", "multiring", k=4, dist="normal",
             sigma=1e-2, seed=43),
    Workload("torus-4x4-f16", 16, 65_539, "f16", "mean", "torus2d", rows=4, cols=4,
             dist="normal", sigma=1e-2, seed=44),
    Workload("torus-2x3-sum", 6, 33_333, "f32", "sum", "torus2d", rows=2, cols=3,
             dist="uniform", seed=45),
    Workload("buckets-ring-P4", 4, 37 + 4096 + 5 + 10_000, "f32", "mean", "ring",
             dist="normal", sigma=1e-2, seed=46,
             buckets=[(4138, 10_000), (4133, 5), (37, 4096), (0, 37)]),
]


def expected(w, weights0, lr):
    g = host_inputs(w)
    y = [x.copy() for x in g]
    oracle_full(w, y)
    ws = [x.copy() for x in weights0]
    orc.sgd(ws, y[0], lr)
    return g, y, ws


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("mode,keep,passes", [("fused", True, 1), ("fused", False, 1),
                                              ("fused", True, 2), ("fused", False, 2),
                                              ("step1", True, 0), ("step2", True, 0)],
                         ids=lambda v: str(v))
@pytest.mark.parametrize("shared", [False, True])
def test_sgd_bitwise(w, mode, keep, passes, shared):
    # passes 1: the update in the one-kernel pass's epilogue; 2: reduce
    # (to rank 0, or to the plan's scratch buffer without kept gradients),
    # broadcast, then the update kernel
    say(f"case sgd {w.name} mode={mode} keep={keep} passes={passes} shared={shared}")
    lr = 0.0125
    rng = np.random.default_rng(w.seed)
    nrep = 1 if shared else w.P
    w0 = [rng.standard_normal(w.n).astype(np.float32) for _ in range(nrep)]
    g, y, want_w = expected(w, w0, lr)
    bufs = [torch.from_numpy(x).cuda() for x in g]
    weights = [torch.from_numpy(x).cuda() for x in w0]
    plan = ddl.Plan(w.P, w.n, w.dtype, w.op, ddl_topo(w), w.bucket_list(),
                    "fused" if mode == "fused" else "stepwise")
    if mode == "fused":
        plan.set_fused_passes(passes)
    else:
        # one launch per step, or the persistent step kernel
        plan.set_step_form(int(mode[-1]))
    plan.execute_sgd(bufs, weights, lr, keep_grads=keep)
    torch.cuda.synchronize()
    plan.destroy()
    for r in range(nrep):
        got = weights[r].cpu().numpy()
        assert got.tobytes() == want_w[r].tobytes(), (w.name, mode, keep, shared, r)
    for r in range(w.P):
        got = bufs[r].cpu().numpy()
        assert got.tobytes() == (y[r] if keep else g[r]).tobytes(), (w.name, r)


@pytest.mark.parametrize("keep", [True, False])
def test_sgd_headline_sampled(keep):
    """40 ranks x 300M fp32, 64 event-gated buckets, one replica per rank, in
    the form bench.py times (two kernels and the update kernel): sampled
    elements against the oracle, every replica identical, and without kept
    gradients the buffers untouched."""
    w = WORKLOADS["ring_p40_300m_64b"]
    lr = 0.01
    say("case sgd headline: inputs")
    bufs = [torch.empty(w.n, dtype=torch.float32, device="cuda") for _ in range(w.P)]
    for r, b in enumerate(bufs):
        synth.fill_device(b.data_ptr(), w.n, synth.F32, w.dist, w.seed, r, sigma=w.sigma)
    weights = [torch.empty(w.n, dtype=torch.float32, device="cuda") for _ in range(w.P)]
    for t in weights:  # identical replicas, as data-parallel SGD keeps them
        synth.fill_device(t.data_ptr(), w.n, synth.F32, "uniform", 77, 0)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    events = [torch.cuda.Event() for _ in w.bucket_list()]
    for e in events:
        e.record(stream)
    say(f"case sgd headline: fused all-reduce + SGD keep={keep}")
    plan = ddl.Plan(w.P, w.n, w.dtype, w.op, ddl_topo(w), w.bucket_list(), "fused")
    assert plan.fused_passes() == 2
    plan.execute_sgd(bufs, weights, lr, keep_grads=keep, events=events, stream=stream)
    torch.cuda.synchronize()
    plan.destroy()
    assert all(torch.equal(weights[0].view(torch.int32), t.view(torch.int32))
               for t in weights[1:])
    from _helpers import sample_indices
    idx = sample_indices(w, 2000, seed=3)
    y, _ = oracle_at(w, idx)
    w0 = synth.gather_host(idx, synth.F32, "uniform", 77, 0)
    want = w0.copy()
    orc.sgd([want], y, lr)
    it = torch.from_numpy(idx.astype(np.int64)).cuda()
    got = weights[w.P // 3][it].cpu().numpy()
    assert got.tobytes() == want.tobytes()
    got_y = bufs[w.P - 1][it].cpu().numpy()
    if keep:
        assert got_y.tobytes() == y.tobytes()
    else:
        g = synth.gather_host(idx, synth.F32, w.dist, w.seed, w.P - 1, sigma=w.sigma)
        assert got_y.tobytes() == g.tobytes()
    del bufs, weights
    torch.cuda.empty_cache()
