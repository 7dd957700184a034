"""GPU parity of the LARS step after the all-reduce.

Expected values: the oracle's all-reduce walk, then its LARS step with the
plan's buckets as layers (binary64 norms in index order, rate rounded once to
binary32, then the SGD step with that rate).

The all-reduce result is compared bit for bit.  The library sums the norms
in another order (per lane, then a fixed tree), so its binary64 norms differ
from the oracle's in the last bits and a rate can differ in its last binary32
bit when lr * trust lies within about 1e-13 of a rounding boundary.  The
tolerance follows from that: every rate within one binary32 ulp of the
oracle's, at least 90% of them equal (a systematic error -- truncation
instead of rounding, a wrong norm -- moves far more), and the weights of a
layer whose rate is equal bit for bit; otherwise each weight within
|y| ulp(rate) + 2 ulp(rate y) + 2 ulp(w), the spread one ulp of the rate can
cause through the product and the difference.
"""
import math

import numpy as np
import pytest

import oracle as orc
import sgd_gradient_all_amd as ddl
import synth
from synth.workloads import WORKLOADS, Workload

from _helpers import ddl_topo, host_inputs, oracle_full, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [
    Workload("ring-P5", 5, 12_347, "f32", "mean", "ring", dist="normal", sigma=1e-2, seed=51),
    Workload("ring-P1", 1, 5_000, "f32", "mean", "ring", dist="normal", sigma=1e-2, seed=52),
    Workload("mring-P16-k4-f16", 16, 70_001, "f16", "mean", "multiring", k=4, dist="normal",
             sigma=1e-2, seed=53),
    Workload("torus-4x4-f16", 16, 65_539, "f16", "mean", "torus2d", rows=4, cols=4,
             dist="normal", sigma=1e-2, seed=54),
    Workload("torus-2x3-sum", 6, 33_333, "f32", "sum", "torus2d", rows=2, cols=3,
             dist="uniform", seed=55),
    Workload("buckets-ring-P4", 4, 37 + 4096 + 5 + 10_000, "f32", "mean", "ring",
             dist="normal", sigma=1e-2, seed=56,
             buckets=[(4138, 10_000), (4133, 5), (37, 4096), (0, 37)]),
    Workload("buckets-f16-P8", 8, 3 * 4096 + 5 + 20_003, "f16", "mean", "ring",
             dist="normal", sigma=1e-2, seed=57,
             buckets=[(3 * 4096 + 5, 20_003), (0, 3 * 4096), (3 * 4096, 5), (32_296, 0)]),
]

MODES = [("fused", 1), ("fused", 2), ("stepwise", 0)]


def check_lars(got_w, want_w, got_rates, want_rates, y, layers, tag):
    """The tolerance of the module docstring; returns the exact-rate count."""
    y32 = y.astype(np.float32)
    exact = 0
    for l, (o, c) in enumerate(layers):
        gr, wr = np.float32(got_rates[l]), np.float32(want_rates[l])
        ulp = np.spacing(np.abs(wr))
        assert abs(float(gr) - float(wr)) <= float(ulp), (tag, l, gr, wr)
        g, w = got_w[o:o + c], want_w[o:o + c]
        if gr == wr:
            exact += 1
            assert g.tobytes() == w.tobytes(), (tag, l)
        else:
            step = np.abs(wr * y32[o:o + c])
            bound = (np.abs(y32[o:o + c]) * ulp + 2 * np.spacing(step) +
                     2 * np.spacing(np.maximum(np.abs(g), np.abs(w))))
            assert np.all(np.abs(g.astype(np.float64) - w) <= bound), (tag, l)
    assert exact >= math.ceil(0.9 * len(layers)), (tag, exact, len(layers))
    return exact


def run_case(w, mode, passes, shared, lr=0.05, events=False, calls=1, zero_layers=()):
    rng = np.random.default_rng(w.seed)
    nrep = 1 if shared else w.P
    w0 = rng.standard_normal(w.n).astype(np.float32) * np.float32(0.1)
    layers = w.bucket_list()
    g = host_inputs(w)
    for li in zero_layers:  # ("w", i): zero weights of layer i; ("g", i): zero gradient
        kind, i = li
        o, c = layers[i]
        if kind == "w":
            w0[o:o + c] = 0
        else:
            for x in g:
                x[o:o + c] = 0
    weights0 = [w0.copy() for _ in range(nrep)]
    # expected: `calls` rounds of (all-reduce, LARS) on the host
    y = [x.copy() for x in g]
    want_w = [x.copy() for x in weights0]
    for _ in range(calls):
        oracle_full(w, y)
        want_rates = orc.lars(want_w, y[0], layers, lr)
    bufs = [torch.from_numpy(x).cuda() for x in g]
    weights = [torch.from_numpy(x).cuda() for x in weights0]
    rates = torch.full((max(1, len(layers)),), -1.0, dtype=torch.float32, device="cuda")
    plan = ddl.Plan(w.P, w.n, w.dtype, w.op, ddl_topo(w), layers, mode)
    if mode == "fused":
        plan.set_fused_passes(passes)
    stream = torch.cuda.current_stream()
    evs = None
    for _ in range(calls):
        if events:
            evs = [torch.cuda.Event() for _ in layers]
            for e in evs[::-1]:
                e.record(stream)
        plan.execute_lars(bufs, weights, lr, rates_out=rates, events=evs, stream=stream)
    torch.cuda.synchronize()
    plan.destroy()
    for r in range(w.P):
        assert bufs[r].cpu().numpy().tobytes() == y[r].tobytes(), (w.name, "grads", r)
    got_rates = rates.cpu().numpy()
    tag = (w.name, mode, passes, shared)
    for r in range(nrep):
        check_lars(weights[r].cpu().numpy(), want_w[r], got_rates, want_rates, y[0], layers,
                   tag + (r,))
    # replicas stay identical to each other
    for r in range(1, nrep):
        assert torch.equal(weights[0].view(torch.int32), weights[r].view(torch.int32))
    return got_rates, want_rates


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("mode,passes", MODES, ids=lambda m: str(m))
@pytest.mark.parametrize("shared", [False, True])
def test_lars_parity(w, mode, passes, shared):
    say(f"case lars {w.name} mode={mode} passes={passes} shared={shared}")
    run_case(w, mode, passes, shared)


@pytest.mark.parametrize("mode,passes", MODES, ids=lambda m: str(m))
def test_lars_events_two_calls_and_zero_layers(mode, passes):
    # per-bucket events on the side streams; two calls in a row on one plan
    # (the second all-reduces the first's result and steps again); a layer
    # of zero weights (trust 1 in the first call) and one of zero gradient
    # (trust 1 in both)
    w = CASES[5]
    say(f"case lars events/two calls {w.name} mode={mode} passes={passes}")
    got, want = run_case(w, mode, passes, False, lr=0.2, events=True, calls=2,
                         zero_layers=(("w", 1), ("g", 3)))
    assert got[3] == np.float32(0.2)
    say(f"case lars zero layers, one call {w.name} mode={mode} passes={passes}")
    got, want = run_case(w, mode, passes, True, lr=0.2, zero_layers=(("w", 1), ("g", 3)))
    assert got[1] == np.float32(0.2) and got[3] == np.float32(0.2)


@pytest.fixture
def restore_knobs():
    yield
    for k in ("update_reps", "update_batch", "reduce_ranks_min_p", "bcast_store_wait"):
        ddl.set_tuning(k, -1)


@pytest.mark.parametrize("knob,value", [("update_reps", g) for g in (0, 1, 3, 7, 100)] +
                         [("update_batch", b) for b in (1, 2, 8)] +
                         [("reduce_ranks_min_p", 0), ("reduce_ranks_min_p", 1000)] +
                         [("bcast_store_wait", 0), ("bcast_store_wait", 1)],
                         ids=lambda v: str(v))
def test_lars_knobs(knob, value, restore_knobs):
    # the update's replica split and load batch change launch shapes only
    # (in the one-kernel form the update kernel reads them, in the two-kernel
    # form the broadcast that steps the replicas reads the load batch); the
    # reduce kernel's loop order changes the order of nothing that is summed
    # (each tile's norm partial sums are formed as before)
    ddl.set_tuning(knob, value)
    for w in (CASES[2], CASES[5]):
        for passes in (1, 2):
            say(f"case lars knob {knob}={value} {w.name} passes={passes}")
            run_case(w, "fused", passes, False)


def test_lars_page_constants_closed_form():
    # every rank holds 2^-10 (64 elements per rank, 4 ranks, mean): y = 2^-10
    # exactly, ||y|| = 2^-7; weights 1.5: ||w|| = 12.  With the page's
    # coefficient and eps the rate is lr * 0.01 * 12 / (2^-7 + 1e-6), whose
    # exact binary32 rounding the oracle's pin derives; here it must match the
    # oracle's rate bit for bit and the weights 1.5 - rate * 2^-10.
    say("case lars closed form")
    P, n, lr = 4, 64, np.float32(0.1)
    bufs = [torch.full((n,), 2.0 ** -10, dtype=torch.float32, device="cuda") for _ in range(P)]
    weights = [torch.full((n,), 1.5, dtype=torch.float32, device="cuda")]
    rates = torch.zeros(1, dtype=torch.float32, device="cuda")
    plan = ddl.Plan(P, n, "f32", "mean", ddl.topo("ring"), None, "fused")
    plan.execute_lars(bufs, weights, float(lr), rates_out=rates)
    torch.cuda.synchronize()
    plan.destroy()
    want_w = np.full(n, 1.5, np.float32)
    want_r = orc.lars([want_w], np.full(n, 2.0 ** -10, np.float32), [(0, n)], lr)
    assert rates.cpu().numpy()[0] == want_r[0]
    assert weights[0].cpu().numpy().tobytes() == want_w.tobytes()


def test_lars_resnet50_layers():
    """The 161 ResNet-50 tensors as layers (16 ranks, 4 rings, binary32,
    mean), one replica per rank, every tensor its own event."""
    w = WORKLOADS["multiring_k4_p16_resnet50"]
    say("case lars resnet50: oracle")
    run_case(w, "fused", 0, False, lr=0.1, events=True)


def test_lars_headline_buckets():
    """40 ranks x 300M binary32, 64 event-gated buckets, one replica per
    rank: two whole buckets (the first issued and a middle one) against the
    oracle -- all-reduce, rate and every weight -- and the replicas equal."""
    w = WORKLOADS["ring_p40_300m_64b"]
    lr = 0.01
    layers = w.bucket_list()
    say("case lars headline: inputs")
    bufs = [torch.empty(w.n, dtype=torch.float32, device="cuda") for _ in range(w.P)]
    for r, b in enumerate(bufs):
        synth.fill_device(b.data_ptr(), w.n, synth.F32, w.dist, w.seed, r, sigma=w.sigma)
    weights = [torch.empty(w.n, dtype=torch.float32, device="cuda") for _ in range(w.P)]
    for t in weights:
        synth.fill_device(t.data_ptr(), w.n, synth.F32, "uniform", 77, 0)
    torch.cuda.synchronize()
    picks = [0, len(layers) // 2]
    host_g = {i: [b[layers[i][0]:layers[i][0] + layers[i][1]].cpu().numpy() for b in bufs]
              for i in picks}
    host_w = {i: weights[0][layers[i][0]:layers[i][0] + layers[i][1]].cpu().numpy()
              for i in picks}
    stream = torch.cuda.current_stream()
    events = [torch.cuda.Event() for _ in layers]
    for e in events:
        e.record(stream)
    rates = torch.zeros(len(layers), dtype=torch.float32, device="cuda")
    say("case lars headline: fused all-reduce + LARS")
    plan = ddl.Plan(w.P, w.n, w.dtype, w.op, ddl_topo(w), layers, "fused")
    plan.execute_lars(bufs, weights, lr, rates_out=rates, events=events, stream=stream)
    torch.cuda.synchronize()
    plan.destroy()
    for r in range(1, w.P):
        assert torch.equal(weights[0].view(torch.int32), weights[r].view(torch.int32)), r
    got_rates = rates.cpu().numpy()
    assert np.all(np.isfinite(got_rates)) and np.all(got_rates > 0)
    for i in picks:
        o, c = layers[i]
        say(f"case lars headline: oracle bucket {i}")
        y = host_g[i]
        orc.allreduce(y, op=orc.MEAN)   # the bucket alone: the same chains
        want_w = host_w[i].copy()
        want_r = orc.lars([want_w], y[0], [(0, c)], lr)
        got_y = bufs[w.P - 1][o:o + c].cpu().numpy()
        assert got_y.tobytes() == y[0].tobytes(), i
        check_lars(weights[w.P // 3][o:o + c].cpu().numpy(), want_w, got_rates[i:i + 1],
                   want_r, y[0], [(0, c)], ("headline", i))
    del bufs, weights
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kind,mode,passes", [("lars", "fused", 2), ("lars", "fused", 1),
                                              ("lars", "stepwise", 0), ("sgd_keep", "fused", 2),
                                              ("sgd_drop", "fused", 2)], ids=lambda v: str(v))
def test_graph_capture_lars_and_sgd(kind, mode, passes):
    """The LARS step and the two-kernel SGD step captured into a HIP graph
    (after one eager call has bound the plan and allocated its scratch)
    replay to the oracle's result, replay after replay, with the inputs and
    weights restored eagerly in between."""
    say(f"case graph capture {kind} {mode} passes={passes}")
    w = Workload("graph-lars", 16, 16 * 65_536, "f32", "mean", "multiring", k=4, dist="normal",
                 sigma=1e-2, seed=58, buckets=[(i * 65_536, 65_536) for i in reversed(range(16))])
    lr = 0.05
    layers = w.bucket_list()
    rng = np.random.default_rng(w.seed)
    w0 = (rng.standard_normal(w.n) * 0.1).astype(np.float32)
    g = host_inputs(w)
    y = [x.copy() for x in g]
    oracle_full(w, y)
    want_w = [w0.copy() for _ in range(w.P)]
    if kind == "lars":
        want_rates = orc.lars(want_w, y[0], layers, lr)
    else:
        orc.sgd(want_w, y[0], lr)
    src = [torch.from_numpy(x).cuda() for x in g]
    wsrc = torch.from_numpy(w0).cuda()
    bufs = [t.clone() for t in src]
    weights = [wsrc.clone() for _ in range(w.P)]
    rates = torch.zeros(len(layers), dtype=torch.float32, device="cuda")
    plan = ddl.Plan(w.P, w.n, w.dtype, w.op, ddl_topo(w), layers, mode)
    if mode == "fused":
        plan.set_fused_passes(passes)

    def call(stream):
        if kind == "lars":
            plan.execute_lars(bufs, weights, lr, rates_out=rates, stream=stream)
        else:
            plan.execute_sgd(bufs, weights, lr, keep_grads=kind == "sgd_keep", stream=stream)

    call(torch.cuda.current_stream())   # binds the plan, allocates its scratch
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            call(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for b, x in zip(bufs, src):
            b.copy_(x)
        for t in weights:
            t.copy_(wsrc)
        rates.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want_g = g if kind == "sgd_drop" else y
        for r in (0, 7, 15):
            assert bufs[r].cpu().numpy().tobytes() == want_g[r].tobytes(), (kind, rep, r)
        if kind == "lars":
            got_rates = rates.cpu().numpy()
            for r in (0, 15):
                check_lars(weights[r].cpu().numpy(), want_w[r], got_rates, want_rates, y[0],
                           layers, (kind, rep, r))
        else:
            for r in (0, 15):
                assert weights[r].cpu().numpy().tobytes() == want_w[r].tobytes(), (kind, rep, r)
    del graph
    torch.cuda.synchronize()
    plan.destroy()
