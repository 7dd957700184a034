"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bit-exact comparison of every element at sizes the oracle walks in seconds
(several tiles and ragged tails), and of sampled elements plus whole-buffer
properties at the full workload sizes, in the launch configuration the
benchmark times.  Every test names its case on stdout before touching the GPU.
"""
import os

import numpy as np
import pytest

import oracle as orc
import sgd_gradient_all_amd as ddl
import synth
from synth.workloads import WORKLOADS, Workload

from _helpers import (KINDS, OPS, bucket_of, ddl_topo, host_inputs, np_dtype, oracle_at,
                      oracle_full, say, synth_dtype, sample_indices)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TORCH_DT = {"f32": torch.float32, "f16": torch.float16}
# launches that the runtime serialises complete before the launch call returns
SERIALISED = os.environ.get("AMD_SERIALIZE_KERNEL", "0") not in ("", "0")


def to_device(arrs):
    return [torch.from_numpy(a).cuda() for a in arrs]


def to_host(ts):
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in ts]


def bitwise_equal(a, b):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    if a.tobytes() == b.tobytes():
        return True
    fa, fb = a.astype(np.float64), b.astype(np.float64)
    same = (a.view(np.uint16 if a.dtype == np.float16 else np.uint32)
            == b.view(np.uint16 if b.dtype == np.float16 else np.uint32))
    return bool(np.all(same | (np.isnan(fa) & np.isnan(fb))))


# "fused1" / "fused2": a fused plan forced to its one-kernel / two-kernel
# form; "fused" leaves the form to the plan.  "step1" / "step2": a stepwise
# plan forced to one launch per step / the persistent step kernel;
# "stepwise" leaves the form to the plan.
PASSES = {"fused1": 1, "fused2": 2}
STEP_FORMS = {"step1": 1, "step2": 2}


def make_plan(w, mode, op=None):
    plan = ddl.Plan(w.P, w.n, w.dtype, op or w.op, ddl_topo(w), w.bucket_list(),
                    "fused" if mode in PASSES else "stepwise" if mode in STEP_FORMS else mode)
    if mode in PASSES:
        plan.set_fused_passes(PASSES[mode])
    if mode in STEP_FORMS:
        plan.set_step_form(STEP_FORMS[mode])
    return plan


def run_ddl(bufs, w, mode, op=None, plan_api=True, events=None, stream=None):
    t = ddl_topo(w)
    if plan_api or mode in PASSES or mode in STEP_FORMS:
        plan = make_plan(w, mode, op)
        plan.execute(bufs, events=events, stream=stream)
        torch.cuda.synchronize()
        plan.destroy()
    else:
        ddl.ddl_allreduce(bufs, w.n, w.dtype, op or w.op, t, w.bucket_list(), mode,
                          stream=stream, events=events)
        torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# small cases: every element, every rank, bit for bit
# ---------------------------------------------------------------------------
def small_cases():
    cases = []
    for dtype in ("f32", "f16"):
        # (3, 400_003) and (2, 8_400_011) give step items long enough for the
        # step kernels' two- and one-vector-per-lane tiles
        for P, n in ((1, 1000), (2, 1), (3, 2), (4, 4099), (5, 12347), (8, 100_003),
                     (16, 70_001), (3, 400_003), (2, 8_400_011)):
            cases.append(Workload(f"ring-P{P}-n{n}-{dtype}", P, n, dtype, "sum", "ring",
                                  dist="uniform", seed=P + n))
        for P, k, n in ((4, 2, 9_999), (16, 4, 250_007), (6, 3, 17)):
            cases.append(Workload(f"mring-P{P}-k{k}-n{n}-{dtype}", P, n, dtype, "mean",
                                  "multiring", k=k, dist="normal", sigma=1e-2, seed=n))
        for R, C, n in ((2, 2, 5_003), (4, 4, 200_009), (2, 3, 77_777), (3, 1, 1_001),
                        (1, 5, 1_234)):
            cases.append(Workload(f"torus-{R}x{C}-n{n}-{dtype}", R * C, n, dtype, "mean",
                                  "torus2d", rows=R, cols=C, dist="normal", sigma=1e-2,
                                  seed=n + R))
    # bucket lists, reverse order, with offsets that are not multiples of 16 B
    sizes = [37, 4096, 5, 0, 100_000, 1, 2048, 777]
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).tolist()
    bl = list(zip(offs, sizes))[::-1]
    for dtype in ("f32", "f16"):
        cases.append(Workload(f"buckets-ring-P6-{dtype}", 6, sum(sizes), dtype, "mean", "ring",
                              dist="normal", sigma=1e-2, seed=99, buckets=bl))
        cases.append(Workload(f"buckets-torus-2x4-{dtype}", 8, sum(sizes), dtype, "sum",
                              "torus2d", rows=2, cols=4, dist="uniform", seed=98, buckets=bl))
    return cases


@pytest.mark.parametrize("w", small_cases(), ids=lambda w: w.name)
@pytest.mark.parametrize("mode", ["fused1", "fused2", "step1", "step2"])
@pytest.mark.parametrize("op", ["sum", "mean"])
def test_small_bitwise(w, mode, op):
    say(f"case {w.name} mode={mode} op={op}")
    g = host_inputs(w)
    ref = [x.copy() for x in g]
    oracle_full(w, ref, op=op)
    bufs = to_device(g)
    run_ddl(bufs, w, mode, op=op, plan_api=(mode == "fused"))
    out = to_host(bufs)
    for r in range(w.P):
        assert bitwise_equal(out[r], ref[r]), (w.name, mode, op, r)


TINY_TOPOS = [
    ("ring40", 40, dict(topo="ring")),
    ("mring16k4", 16, dict(topo="multiring", k=4)),
    ("torus4x4", 16, dict(topo="torus2d", rows=4, cols=4)),
    ("torus2x3", 6, dict(topo="torus2d", rows=2, cols=3)),
]


@pytest.mark.parametrize("name,P,tk", TINY_TOPOS, ids=[t[0] for t in TINY_TOPOS])
@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("op", ["sum", "mean"])
@pytest.mark.parametrize("gated", [True, False])
def test_tiny_spans_one_wave_each(name, P, tk, dtype, op, gated):
    """Buckets whose every span has at most 64 elements (one to a few
    elements per rank chunk) run one wave per span when a group holds only
    them; groups mixing them with larger spans take the tiled pass.  With one
    ready event per bucket every group is one bucket; without events the
    whole list is one mixed group.  Every element of every rank against the
    oracle, in the automatic (one-kernel) fused form and stepwise."""
    sizes = [1, 2, 7, 17, 64, 100, 333, 1000, 4096, 4100, 5000, 20000]
    buckets, at = [], 0
    for c in sizes:
        buckets.append((at, c))
        at += c
    w = Workload(f"tiny-{name}", P, at, dtype, op, tk["topo"], k=tk.get("k", 1),
                 rows=tk.get("rows", 0), cols=tk.get("cols", 0), dist="normal", sigma=1e-2,
                 seed=71, buckets=buckets[::-1])
    say(f"case tiny spans {name} {dtype} {op} gated={gated}")
    g = host_inputs(w)
    ref = [x.copy() for x in g]
    oracle_full(w, ref)
    stream = torch.cuda.current_stream()
    for mode in ("fused", "step1", "step2"):
        bufs = to_device(g)
        events = None
        if gated:
            events = [torch.cuda.Event() for _ in buckets]
            for e in events:
                e.record(stream)
        plan = make_plan(w, mode)
        plan.execute(bufs, events=events, stream=stream)
        torch.cuda.synchronize()
        plan.destroy()
        out = to_host(bufs)
        for r in range(P):
            assert bitwise_equal(out[r], ref[r]), (name, dtype, op, gated, mode, r)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_subnormals_and_specials(dtype):
    say(f"case subnormals/specials {dtype}")
    dt = np_dtype(dtype)
    P, n = 4, 4096
    rng = np.random.default_rng(3)
    tiny = np.float32(2.0 ** -130) if dtype == "f32" else np.float32(2.0 ** -20)
    g = [(rng.integers(-50, 50, n).astype(np.float32) * tiny).astype(dt) for _ in range(P)]
    g[1][7] = np.inf
    g[2][9] = np.nan
    g[0][11], g[3][11] = np.inf, -np.inf
    w = Workload("sub", P, n, dtype, "mean", "ring")
    for mode in ("fused1", "fused2", "step1", "step2"):
        for op in ("sum", "mean"):
            ref = [x.copy() for x in g]
            oracle_full(w, ref, op=op)
            assert np.any(ref[0][:] != 0)
            bufs = to_device(g)
            run_ddl(bufs, w, mode, op=op)
            out = to_host(bufs)
            for r in range(P):
                assert bitwise_equal(out[r], ref[r]), (mode, op, r)


def test_closed_form_rank_plus_one():
    for name in ("ring_p4_1m_sum", "multiring_k4_p16_resnet50", "torus_4x4_resnet50_f16"):
        w = WORKLOADS[name]
        say(f"case closed form {name}")
        bufs = [torch.full((w.n,), r + 1, dtype=TORCH_DT[w.dtype], device="cuda")
                for r in range(w.P)]
        for mode in ("fused", "stepwise", "step2"):
            for op, want in (("sum", w.P * (w.P + 1) / 2), ("mean", (w.P + 1) / 2)):
                for r, b in enumerate(bufs):
                    b.fill_(r + 1)
                run_ddl(bufs, w, mode, op=op)
                for b in bufs:
                    assert bool((b == want).all()), (name, mode, op)


# ---------------------------------------------------------------------------
# the measured workloads at full size
# ---------------------------------------------------------------------------
def device_inputs(w):
    bufs = [torch.empty(w.n, dtype=TORCH_DT[w.dtype], device="cuda") for _ in range(w.P)]
    for r, b in enumerate(bufs):
        synth.fill_device(b.data_ptr(), w.n, synth_dtype(w.dtype), w.dist, w.seed, r,
                          sigma=w.sigma)
    torch.cuda.synchronize()
    return bufs


def ranks_identical(bufs):
    iv = torch.int16 if bufs[0].dtype == torch.float16 else torch.int32
    return all(torch.equal(bufs[0].view(iv), b.view(iv)) for b in bufs[1:])


def test_synth_device_matches_host():
    for dtype in ("f32", "f16"):
        for dist, sigma in (("uniform", 1.0), ("normal", 1e-3), ("normal", 1e-2),
                            ("smallint", 1.0), ("rankconst", 1.0)):
            say(f"case synth {dtype} {dist}")
            n, first = 300_001, 123_456_789
            t = torch.empty(n, dtype=TORCH_DT[dtype], device="cuda")
            synth.fill_device(t.data_ptr(), n, synth_dtype(dtype), dist, 7, 3, first=first,
                              sigma=sigma)
            got = to_host([t])[0]
            want = synth.fill_host(n, synth_dtype(dtype), dist, 7, 3, first=first, sigma=sigma)
            assert got.tobytes() == want.tobytes(), (dtype, dist)


@pytest.mark.parametrize("name", ["ring_p4_1m_sum", "multiring_k4_p16_resnet50",
                                  "torus_4x4_resnet50_f16"])
def test_workload_full_bitwise(name):
    """Every element of every rank against the oracle's full walk, both
    modes, buckets as the workload issues them."""
    w = WORKLOADS[name]
    say(f"case workload {name}: host inputs")
    g = host_inputs(w)
    ref = [x.copy() for x in g]
    oracle_full(w, ref)
    for mode in ("fused", "fused1", "fused2", "stepwise", "step1", "step2"):
        say(f"case workload {name} mode={mode}")
        bufs = to_device(g)
        run_ddl(bufs, w, mode, plan_api=False)
        out = to_host(bufs)
        for r in range(w.P):
            assert bitwise_equal(out[r], ref[r]), (name, mode, r)
        del bufs
    ddl.ddl_cache_clear()
    y64 = orc.sum_f64(g, op=OPS[w.op])
    err = np.linalg.norm(ref[0].astype(np.float64) - y64) / np.linalg.norm(y64)
    assert err <= (1e-6 if w.dtype == "f32" else 2e-3), err


@pytest.mark.parametrize("name", ["ring_p8_300m_mean", "ring_p40_300m_64b"])
def test_workload_full_size_sampled(name):
    """Full size, generated on the GPU: sampled elements against the oracle,
    every rank bit-identical, fused and stepwise bit-identical everywhere."""
    w = WORKLOADS[name]
    say(f"case workload {name}: device inputs ({w.P} x {w.n})")
    bufs = device_inputs(w)
    copy = [b.clone() for b in bufs]
    stream = torch.cuda.current_stream()
    events = None
    if w.side_stream:
        events = [torch.cuda.Event() for _ in w.bucket_list()]
        for e in events:
            e.record(stream)
    say(f"case workload {name}: fused")
    plan = ddl.Plan(w.P, w.n, w.dtype, w.op, ddl_topo(w), w.bucket_list(), "fused")
    plan.execute(bufs, events=events, stream=stream)
    torch.cuda.synchronize()
    assert ranks_identical(bufs)
    idx = sample_indices(w, 3000, seed=1)
    want, inputs = oracle_at(w, idx)
    it = torch.from_numpy(idx.astype(np.int64)).cuda()
    for r in (0, w.P // 2, w.P - 1):
        got = bufs[r][it].cpu().numpy()
        assert bitwise_equal(got, want), (name, r)
    # accuracy against binary64 on the sample
    y64 = np.sum(np.stack(inputs).astype(np.float64), axis=0) / (w.P if w.op == "mean" else 1)
    err = np.linalg.norm(want.astype(np.float64) - y64) / np.linalg.norm(y64)
    assert err <= 1e-6, err
    plan.destroy()
    say(f"case workload {name}: stepwise")
    plan = ddl.Plan(w.P, w.n, w.dtype, w.op, ddl_topo(w), w.bucket_list(), "stepwise")
    plan.execute(copy, events=events, stream=stream)
    torch.cuda.synchronize()
    iv = torch.int32
    assert all(torch.equal(a.view(iv), b.view(iv)) for a, b in zip(bufs, copy))
    # the other step form (persistent, or one launch per step), fresh inputs
    other = 3 - plan.step_form()
    plan.set_step_form(other)
    say(f"case workload {name}: stepwise, form {other}")
    for r, b in enumerate(copy):
        synth.fill_device(b.data_ptr(), w.n, synth_dtype(w.dtype), w.dist, w.seed, r,
                          sigma=w.sigma)
    torch.cuda.synchronize()
    plan.execute(copy, events=events, stream=stream)
    torch.cuda.synchronize()
    assert all(torch.equal(a.view(iv), b.view(iv)) for a, b in zip(bufs, copy))
    plan.destroy()
    # the fused pass's other form, on fresh inputs: bit-identical as well
    plan = ddl.Plan(w.P, w.n, w.dtype, w.op, ddl_topo(w), w.bucket_list(), "fused")
    other = 3 - plan.fused_passes()
    say(f"case workload {name}: fused, {other} kernel(s)")
    plan.set_fused_passes(other)
    for r, b in enumerate(copy):
        synth.fill_device(b.data_ptr(), w.n, synth_dtype(w.dtype), w.dist, w.seed, r,
                          sigma=w.sigma)
    torch.cuda.synchronize()
    plan.execute(copy, events=events, stream=stream)
    torch.cuda.synchronize()
    assert all(torch.equal(a.view(iv), b.view(iv)) for a, b in zip(bufs, copy))
    plan.destroy()
    del bufs, copy
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,P,n", [("f16", 3, (1 << 32) + 4099), ("f32", 2, (1 << 31) + 13)])
def test_element_indices_beyond_32_bits(dtype, P, n):
    """Buffers of more than 2^32 (binary16) or 2^31 (binary32) elements per
    rank, so element indices and byte offsets pass 32 bits: sampled elements
    (chunk edges, the 2^31 and 2^32 boundaries, the ragged tail) against the
    oracle, every rank bit-identical, and the stepwise walk and both fused
    forms bit-identical everywhere."""
    half = (n // 2) // 8 * 8
    w = Workload("beyond32", P, n, dtype, "mean", "ring", dist="normal", sigma=1e-2, seed=97,
                 buckets=[(half, n - half), (0, half)])
    need = 2 * P * n * w.esize
    if torch.cuda.mem_get_info()[0] < need + (4 << 30):
        pytest.skip(f"needs {need >> 30} GiB of device memory")
    say(f"case beyond 32 bits: {dtype} P={P} n={n}: device inputs")
    bufs = device_inputs(w)
    copy = [b.clone() for b in bufs]
    iv = torch.int32 if dtype == "f32" else torch.int16
    plan = ddl.Plan(P, n, dtype, "mean", ddl_topo(w), w.bucket_list(), "fused")
    say(f"case beyond 32 bits: {dtype} fused, {plan.fused_passes()} kernel(s)")
    plan.execute(bufs)
    torch.cuda.synchronize()
    assert ranks_identical(bufs)
    idx = set(sample_indices(w, 1500, seed=3).tolist())
    for edge in (1 << 31, 1 << 32, half, n):
        idx.update(e for e in range(edge - 2, edge + 2) if 0 <= e < n)
    idx = np.array(sorted(idx), dtype=np.uint64)
    want, _ = oracle_at(w, idx)
    it = torch.from_numpy(idx.astype(np.int64)).cuda()
    for r in range(P):
        assert bitwise_equal(bufs[r][it].cpu().numpy(), want), (dtype, r)
    other = 3 - plan.fused_passes()
    plan.destroy()
    say(f"case beyond 32 bits: {dtype} stepwise")
    plan = ddl.Plan(P, n, dtype, "mean", ddl_topo(w), w.bucket_list(), "stepwise")
    plan.execute(copy)
    torch.cuda.synchronize()
    plan.destroy()
    assert all(torch.equal(a.view(iv), b.view(iv)) for a, b in zip(bufs, copy))
    say(f"case beyond 32 bits: {dtype} fused, {other} kernel(s)")
    for r, b in enumerate(copy):
        synth.fill_device(b.data_ptr(), n, synth_dtype(dtype), w.dist, w.seed, r, sigma=w.sigma)
    torch.cuda.synchronize()
    plan = ddl.Plan(P, n, dtype, "mean", ddl_topo(w), w.bucket_list(), "fused")
    plan.set_fused_passes(other)
    plan.execute(copy)
    torch.cuda.synchronize()
    plan.destroy()
    assert all(torch.equal(a.view(iv), b.view(iv)) for a, b in zip(bufs, copy))
    del bufs, copy
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# dispatcher: ready events gate buckets
# ---------------------------------------------------------------------------
def ready_event(kind):
    """A caller's ready event: torch's, or the binding's ReadyEvent, which
    skips the system-scope fence of the record."""
    return torch.cuda.Event() if kind == "torch" else ddl.ReadyEvent()


@pytest.mark.parametrize("ev", ["torch", "nofence"])
@pytest.mark.parametrize("mode", ["fused", "fused1", "step2"])
def test_ready_events_gate_buckets(mode, ev):
    """Inputs are written by kernels queued behind a long kernel on the main
    stream, bucket by bucket, each followed by its event.  The all-reduce is
    enqueued right after: correct results need every bucket to have waited
    for its own event, and the writes before each record to be visible to
    the library's kernels (also with records that skip the system-scope
    fence)."""
    say(f"case ready events {mode} {ev}")
    w = Workload("events", 8, 64 * 65_536, "f32", "mean", "ring", dist="normal", sigma=1e-3,
                 seed=11, buckets=[(i * 65_536, 65_536) for i in reversed(range(64))])
    bufs = [torch.full((w.n,), float("nan"), device="cuda") for _ in range(w.P)]
    scratch = torch.zeros(1 << 27, device="cuda")
    main = torch.cuda.current_stream()
    torch.cuda.synchronize()
    synth.stream_compute(scratch.data_ptr(), scratch.numel(), 1.0001, 0.5, main.cuda_stream)
    events = []
    for off, cnt in w.bucket_list():
        for r, b in enumerate(bufs):
            synth.fill_device(b.data_ptr() + 4 * off, cnt, synth.F32, w.dist, w.seed, r,
                              first=off, sigma=w.sigma, stream=main.cuda_stream)
        e = ready_event(ev)
        e.record(main)
        events.append(e)
    plan = make_plan(w, mode)
    plan.execute(bufs, events=events, stream=main)
    torch.cuda.synchronize()
    g = host_inputs(w)
    oracle_full(w, g)
    out = to_host(bufs)
    for r in range(w.P):
        assert bitwise_equal(out[r], g[r]), r
    plan.destroy()


def test_misaligned_buffer_is_rejected_and_nothing_runs():
    say("case misaligned")
    P, n = 4, 1000
    base = [torch.arange(n + 8, dtype=torch.float32, device="cuda") for _ in range(P)]
    before = [b.clone() for b in base]
    ptrs = [b.data_ptr() + 4 for b in base]  # 4-byte offset: not 16-byte aligned
    plan = ddl.Plan(P, n, "f32", "sum", ddl.topo("ring"))
    with pytest.raises(ddl.DDLError) as ei:
        plan.execute(ptrs)
    assert ei.value.code == -4
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(base, before))
    plan.destroy()


def test_profiling_counts_launches():
    say("case profiling")
    w = WORKLOADS["multiring_k4_p16_resnet50"]
    bufs = [torch.ones(w.n, device="cuda") for _ in range(w.P)]
    for mode, launches in (("fused1", {"fused": 1}),
                           ("fused2", {"fused_reduce": 1, "broadcast": 1}),
                           ("step1", {"reduce": 15, "gather": 15}),
                           ("stepwise", {"walk": 1})):
        plan = make_plan(w, mode, "sum")
        plan.set_profiling(True)
        plan.execute(bufs)
        plan.execute(bufs)
        total, cnt, mx = plan.profile_read()
        assert cnt == 2 * sum(launches.values()), (mode, cnt)
        assert total > 0 and mx <= total
        plan.execute(bufs)
        kinds = plan.profile_read_kinds()
        for k, (tot, c, m) in kinds.items():
            assert c == launches.get(k, 0), (mode, k, c)
            assert (tot > 0) == (c > 0) and m <= tot + 1e-12
        plan.destroy()


def test_plan_reuse_and_cache():
    say("case reuse")
    w = Workload("reuse", 5, 10_000, "f32", "sum", "ring", dist="smallint", seed=4)
    g = host_inputs(w)
    want = np.sum(np.stack(g).astype(np.int64), axis=0)
    for _ in range(3):
        bufs = to_device(g)
        ddl.ddl_allreduce(bufs, w.n, "f32", "sum", ddl.topo("ring"))
        out = to_host(bufs)
        for r in range(w.P):
            assert np.array_equal(out[r].astype(np.int64), want)
    ddl.ddl_cache_clear()


def test_plan_cache_is_bounded():
    """ddl_allreduce keeps at most 64 plans: 80 distinct shapes in a row all
    give the closed-form result, the cache never holds more than 64 plans, a
    repeated shape reuses its plan, and clearing empties it."""
    say("case plan cache bound")
    ddl.ddl_cache_clear()
    assert ddl.ddl_cache_count() == 0
    P = 3
    for i in range(80):
        n = 4096 + 8 * i
        bufs = [torch.full((n,), float(r + 1), device="cuda") for r in range(P)]
        ddl.ddl_allreduce(bufs, n, "f32", "sum", ddl.topo("ring"))
        torch.cuda.synchronize()
        for b in bufs:
            assert bool((b == 6.0).all()), (i, n)
        assert ddl.ddl_cache_count() == min(i + 1, 64), i
    bufs = [torch.full((4096 + 8 * 79,), 1.0, device="cuda") for _ in range(P)]
    ddl.ddl_allreduce(bufs, bufs[0].numel(), "f32", "sum", ddl.topo("ring"))
    torch.cuda.synchronize()
    assert ddl.ddl_cache_count() == 64
    assert bool((bufs[1] == 3.0).all())
    ddl.ddl_cache_clear()
    assert ddl.ddl_cache_count() == 0


def test_oneshot_from_several_threads():
    """ddl_allreduce from four host threads at once, each on its own stream,
    cycling through 20 shapes of its own (80 in all, so the 64-plan cache
    evicts while other threads' work is in flight): every call gives the
    closed form, and no plan is freed under running work."""
    import threading
    say("case one-shot from four threads")
    ddl.ddl_cache_clear()
    P, errors = 3, []

    def worker(t):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for i in range(40):
                    n = 4096 + 8 * (t * 1000 + i % 20)
                    bufs = [torch.full((n,), float(r + 1), device="cuda") for r in range(P)]
                    ddl.ddl_allreduce(bufs, n, "f32", "sum", ddl.topo("ring"), stream=s)
                    if i % 7 == 0:
                        s.synchronize()
                        if not all(bool((b == 6.0).all()) for b in bufs):
                            errors.append((t, i, "values"))
                s.synchronize()
                if not all(bool((b == 6.0).all()) for b in bufs):
                    errors.append((t, "last", "values"))
        except Exception as e:   # surfaced below
            errors.append((t, repr(e)))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads)
    torch.cuda.synchronize()
    assert not errors, errors
    assert ddl.ddl_cache_count() <= 64
    ddl.ddl_cache_clear()


# ---------------------------------------------------------------------------
# dispatcher: grouping threshold, stream semantics, busy plans; edge shapes
# ---------------------------------------------------------------------------
def test_coalesce_threshold_merges_event_gated_buckets():
    """161 ResNet-50 buckets, each with its own ready event: with a 16 MB
    threshold consecutive buckets share launches (fewer launches), results
    bit-identical to one group per bucket and to the oracle."""
    w = WORKLOADS["multiring_k4_p16_resnet50"]
    say("case coalesce threshold")
    g = host_inputs(w)
    ref = [x.copy() for x in g]
    oracle_full(w, ref)
    stream = torch.cuda.current_stream()
    counts = {}
    for mode in ("fused", "step1", "step2"):
        for thr in (0, 16 << 20):
            bufs = to_device(g)
            events = [torch.cuda.Event() for _ in w.bucket_list()]
            for e in events:
                e.record(stream)
            plan = make_plan(w, mode)
            plan.set_coalesce_bytes(thr)
            plan.set_profiling(True)
            plan.execute(bufs, events=events, stream=stream)
            kinds = plan.profile_read_kinds()
            # launches that start a group's work: the fused pass's first
            # kernel, or every step
            counts[(mode, thr)] = sum(kinds[k][1] for k in ("fused", "fused_reduce", "reduce",
                                                              "gather", "walk"))
            if mode == "fused":
                # groups of at least 200 MB over the ranks take the two-kernel
                # form (one broadcast each), smaller ones one kernel
                assert kinds["broadcast"][1] == kinds["fused_reduce"][1]
                if thr == 0:
                    assert kinds["fused_reduce"][1] == 0
            out = to_host(bufs)
            plan.destroy()
            for r in (0, 7, 15):
                assert bitwise_equal(out[r], ref[r]), (mode, thr, r)
    assert counts[("fused", 0)] == 161 and counts[("step1", 0)] == 161 * 30
    assert counts[("step2", 0)] == 161
    assert counts[("fused", 16 << 20)] < 20
    assert counts[("step1", 16 << 20)] == 30 * counts[("fused", 16 << 20)]
    assert counts[("step2", 16 << 20)] == counts[("fused", 16 << 20)]


@pytest.mark.parametrize("ev", ["torch", "nofence"])
@pytest.mark.parametrize("mode", ["fused1", "fused2", "step1", "step2"])
def test_ordered_events_gate_each_group_on_its_last_event(mode, ev):
    """Back-propagation's pattern: on one stream, behind a long streaming
    kernel, each bucket's gradient is written on every rank and then its
    ready event recorded, output layer first.  With ordered events and a
    grouping threshold, each group waits only for the event of its last
    bucket, and every element still matches the oracle: a group that
    started before its last gradient was written would read the zeros the
    buffers held before."""
    say(f"case ordered events {mode} {ev}")
    rng = np.random.default_rng(31)
    sizes = [int(x) for x in rng.choice([8, 64, 1000, 4096, 30_000, 120_000], 40)]
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(int).tolist()
    bl = list(zip(offs, sizes))[::-1]
    w = Workload("ordered", 8, sum(sizes), "f32", "mean", "ring", dist="normal", sigma=1e-2,
                 seed=31, buckets=bl)
    g = host_inputs(w)
    ref = [x.copy() for x in g]
    oracle_full(w, ref)
    src = to_device(g)
    bufs = [torch.zeros_like(x) for x in src]
    stream = torch.cuda.current_stream()
    plan = make_plan(w, mode)
    plan.set_ordered_events(True)
    plan.set_coalesce_bytes(256 << 10)
    plan.execute(bufs, stream=stream)   # binds the plan (its first call allocates)
    torch.cuda.synchronize()
    for b in bufs:
        b.zero_()
    hold = torch.zeros(1 << 27, device="cuda")
    for _ in range(6):
        synth.stream_compute(hold.data_ptr(), hold.numel(), 1.0, 0.0, stream.cuda_stream)
    events = []
    for off, cnt in bl:
        for r in range(w.P):
            bufs[r][off:off + cnt].copy_(src[r][off:off + cnt])
        e = ready_event(ev)
        e.record(stream)
        events.append(e)
    plan.execute(bufs, events=events, stream=stream)
    out = to_host(bufs)
    plan.destroy()
    for r in range(w.P):
        assert bitwise_equal(out[r], ref[r]), (mode, r)


@pytest.mark.parametrize("mode", ["fused1", "fused2", "step1", "step2"])
@pytest.mark.parametrize("ordered", [False, True])
def test_one_event_per_reported_group(mode, ordered):
    """The caller records one ready event per group that event_groups
    reports -- after the last gradient of the group is written, as
    back-propagation would -- and passes it for each of the group's buckets:
    every element matches the oracle, and the plan makes the same launches
    as with one event per bucket (a group that started before its last
    gradient was written would read the zeros the buffers held before)."""
    say(f"case group events {mode} ordered={ordered}")
    rng = np.random.default_rng(37)
    sizes = [int(x) for x in rng.choice([8, 64, 1000, 4096, 30_000, 120_000], 40)]
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(int).tolist()
    bl = list(zip(offs, sizes))[::-1]
    w = Workload("groups", 8, sum(sizes), "f32", "mean", "ring", dist="normal", sigma=1e-2,
                 seed=37, buckets=bl)
    g = host_inputs(w)
    ref = [x.copy() for x in g]
    oracle_full(w, ref)
    src = to_device(g)
    bufs = [torch.zeros_like(x) for x in src]
    stream = torch.cuda.current_stream()
    plan = make_plan(w, mode)
    plan.set_ordered_events(ordered)
    plan.set_coalesce_bytes(256 << 10)
    last = plan.event_groups()
    assert last[-1] == len(bl) - 1 and all(a < b for a, b in zip(last, last[1:]))
    assert 1 < len(last) < len(bl)
    plan.execute(bufs, stream=stream)   # binds the plan (its first call allocates)
    torch.cuda.synchronize()
    launches = {}
    for kind in ("own", "group"):
        for b in bufs:
            b.zero_()
        hold = torch.zeros(1 << 27, device="cuda")
        for _ in range(6):
            synth.stream_compute(hold.data_ptr(), hold.numel(), 1.0, 0.0, stream.cuda_stream)
        events, gi = [], 0
        for i, (off, cnt) in enumerate(bl):
            for r in range(w.P):
                bufs[r][off:off + cnt].copy_(src[r][off:off + cnt])
            if kind == "own" or i == last[gi]:
                e = torch.cuda.Event()
                e.record(stream)
                events.append(e)
                gi += i == last[gi]
        if kind == "group":
            # each bucket gets its group's event
            per, gi = [], 0
            for i in range(len(bl)):
                per.append(events[gi])
                gi += i == last[gi]
            events = per
        plan.set_profiling(1)
        plan.execute(bufs, events=events, stream=stream)
        out = to_host(bufs)
        launches[kind] = sum(v[1] for v in plan.profile_read_kinds().values())
        plan.set_profiling(0)
        for r in range(w.P):
            assert bitwise_equal(out[r], ref[r]), (mode, kind, r)
    plan.destroy()
    assert launches["own"] == launches["group"], launches


@pytest.mark.parametrize("mode", ["stepwise", "fused2"])
def test_caller_stream_waits_for_side_stream_work(mode):
    """Work enqueued on the caller's stream right after an event-gated
    all-reduce sees its result without any host synchronisation."""
    say(f"case caller stream ordering {mode}")
    w = Workload("order", 8, 1 << 22, "f32", "mean", "ring", dist="normal", sigma=1e-2,
                 seed=12, buckets=[(i << 18, 1 << 18) for i in reversed(range(16))])
    g = host_inputs(w)
    ref = [x.copy() for x in g]
    oracle_full(w, ref)
    bufs = to_device(g)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    events = [torch.cuda.Event() for _ in w.bucket_list()]
    for e in events:
        e.record(stream)
    plan = make_plan(w, mode)
    plan.execute(bufs, events=events, stream=stream)
    snap = bufs[3].clone()          # enqueued on the caller stream, no host sync
    torch.cuda.synchronize()
    assert bitwise_equal(snap.cpu().numpy(), ref[3])
    plan.destroy()


def test_destroy_with_work_in_flight_is_busy():
    say("case busy destroy")
    P, n = 8, 1 << 20
    bufs = [torch.ones(n, device="cuda") for _ in range(P)]
    scratch = torch.zeros(1 << 28, device="cuda")
    stream = torch.cuda.current_stream()
    plan = ddl.Plan(P, n, "f32", "sum", ddl.topo("ring"))
    # the first call binds the plan, whose synchronous table upload would
    # wait for the work below: bind it first
    plan.execute([torch.zeros(n, device="cuda") for _ in range(P)], stream=stream)
    torch.cuda.synchronize()
    for _ in range(8):   # keep the stream busy for several milliseconds
        synth.stream_compute(scratch.data_ptr(), scratch.numel(), 1.0, 0.0, stream.cuda_stream)
    plan.execute(bufs, stream=stream)
    rc = plan.try_destroy()
    # with launches serialised (AMD_SERIALIZE_KERNEL) nothing is ever in flight
    assert rc == -7 or (SERIALISED and rc == 0)
    torch.cuda.synchronize()
    plan.destroy()
    assert bool((bufs[5] == P).all())


def test_busy_tracks_every_stream_a_plan_ran_on():
    """One plan, two calls on two streams: the first queued behind several
    milliseconds of other work, the second free to finish at once.  Once the
    second has finished the plan is still busy with the first, so destroy
    refuses (DDL_E_BUSY) until that one is done too."""
    say("case busy over two streams")
    P, n = 8, 1 << 20
    bufs_a = [torch.ones(n, device="cuda") for _ in range(P)]
    bufs_b = [torch.full((n,), 2.0, device="cuda") for _ in range(P)]
    scratch = torch.zeros(1 << 28, device="cuda")
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    plan = ddl.Plan(P, n, "f32", "sum", ddl.topo("ring"))
    plan.execute(bufs_b, stream=torch.cuda.current_stream())   # binds the plan
    for b in bufs_b:
        b.fill_(2.0)
    torch.cuda.synchronize()
    for _ in range(8):   # keep stream a busy for several milliseconds
        synth.stream_compute(scratch.data_ptr(), scratch.numel(), 1.0, 0.0, sa.cuda_stream)
    plan.execute(bufs_a, stream=sa)
    plan.execute(bufs_b, stream=sb)
    sb.synchronize()
    assert bool((bufs_b[3] == 2.0 * P).all())
    rc = plan.try_destroy()
    assert rc == -7 or (SERIALISED and rc == 0)
    torch.cuda.synchronize()
    plan.destroy()
    assert bool((bufs_a[5] == P).all())


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_max_ranks(dtype):
    say(f"case 128 ranks {dtype}")
    for w in (Workload("ring128", 128, 40_003, dtype, "mean", "ring", dist="normal",
                       sigma=1e-2, seed=128),
              Workload("torus8x16", 128, 40_003, dtype, "mean", "torus2d", rows=8, cols=16,
                       dist="normal", sigma=1e-2, seed=129)):
        g = host_inputs(w)
        ref = [x.copy() for x in g]
        oracle_full(w, ref)
        for mode in ("fused1", "fused2", "step1", "step2"):
            bufs = to_device(g)
            run_ddl(bufs, w, mode)
            out = to_host(bufs)
            for r in (0, 63, 127):
                assert bitwise_equal(out[r], ref[r]), (w.name, mode, r)


def test_custom_ring_orders():
    say("case custom ring orders")
    rng = np.random.default_rng(17)
    for P, k, dtype in ((6, 1, "f32"), (16, 4, "f16"), (40, 3, "f32")):
        n = 50_021
        order = np.concatenate([rng.permutation(P) for _ in range(k)]).tolist()
        g = [rng.standard_normal(n).astype(np_dtype(dtype)) for _ in range(P)]
        ref = [x.copy() for x in g]
        kind = "ring" if k == 1 else "multiring"
        orc.allreduce(ref, op=orc.MEAN, kind=KINDS[kind], k=k, ring_order=order)
        for mode in ("fused1", "fused2", "step1", "step2"):
            bufs = to_device(g)
            plan = ddl.Plan(P, n, dtype, "mean", ddl.topo(kind, k, ring_order=order), None,
                            "fused" if mode in PASSES else "stepwise")
            if mode in PASSES:
                plan.set_fused_passes(PASSES[mode])
            else:
                plan.set_step_form(STEP_FORMS[mode])
            plan.execute(bufs)
            out = to_host(bufs)
            plan.destroy()
            for r in (0, P - 1):
                assert bitwise_equal(out[r], ref[r]), (P, k, mode, r)


@pytest.mark.parametrize("mode", ["fused1", "fused2", "step1", "step2"])
def test_hip_graph_capture_and_replay(mode):
    """An execution captured into a HIP graph (after one eager call has bound
    the plan) replays to the oracle's result, replay after replay, with the
    inputs restored eagerly in between."""
    say(f"case graph capture {mode}")
    w = Workload("graph", 16, 1 << 20, "f32", "mean", "multiring", k=4, dist="normal",
                 sigma=1e-2, seed=21, buckets=[(i << 16, 1 << 16) for i in reversed(range(16))])
    g = host_inputs(w)
    ref = [x.copy() for x in g]
    oracle_full(w, ref)
    src = to_device(g)
    bufs = [t.clone() for t in src]
    plan = make_plan(w, mode)
    plan.execute(bufs, stream=torch.cuda.current_stream())   # binds the plan
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            plan.execute(bufs, stream=s)
    torch.cuda.synchronize()
    for rep in range(4):
        for b, x in zip(bufs, src):
            b.copy_(x)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        out = [b.cpu().numpy() for b in bufs]
        for r in (0, 9, 15):
            assert bitwise_equal(out[r], ref[r]), (mode, rep, r)
    del graph
    torch.cuda.synchronize()
    plan.destroy()


def test_ddl_allreduce_with_bucket_events():
    say("case ddl_allreduce events")
    w = Workload("oneshot-ev", 6, 6 * 40_000, "f32", "mean", "ring", dist="normal", sigma=1e-2,
                 seed=22, buckets=[(i * 40_000, 40_000) for i in reversed(range(6))])
    g = host_inputs(w)
    ref = [x.copy() for x in g]
    oracle_full(w, ref)
    bufs = to_device(g)
    stream = torch.cuda.current_stream()
    events = [torch.cuda.Event() for _ in w.bucket_list()]
    for e in events:
        e.record(stream)
    ddl.ddl_allreduce(bufs, w.n, "f32", "mean", ddl.topo("ring"), w.bucket_list(), "stepwise",
                      stream=stream, events=events)
    out = to_host(bufs)
    for r in range(w.P):
        assert bitwise_equal(out[r], ref[r]), r
    ddl.ddl_cache_clear()


@pytest.mark.parametrize("nside", [2, 4])
def test_several_side_streams(nside):
    say(f"case side streams {nside}")
    w = Workload("sides", 8, 24 * 50_000, "f32", "mean", "ring", dist="normal", sigma=1e-2,
                 seed=23, buckets=[(i * 50_000, 50_000) for i in reversed(range(24))])
    g = host_inputs(w)
    ref = [x.copy() for x in g]
    oracle_full(w, ref)
    stream = torch.cuda.current_stream()
    for mode in ("fused1", "fused2", "stepwise"):
        bufs = to_device(g)
        events = [torch.cuda.Event() for _ in w.bucket_list()]
        for e in events:
            e.record(stream)
        plan = make_plan(w, mode)
        plan.set_side_streams(nside)
        plan.execute(bufs, events=events, stream=stream)
        snap = bufs[2].clone()       # on the caller stream, no host sync
        out = to_host(bufs)
        plan.destroy()
        for r in range(w.P):
            assert bitwise_equal(out[r], ref[r]), (mode, r)
        assert bitwise_equal(snap.cpu().numpy(), ref[2])


@pytest.mark.parametrize("mode", ["step1", "step2", "fused2"])
def test_graph_capture_with_bucket_events_and_side_streams(mode):
    """Capture with a ready event per bucket (recorded inside the capture),
    so the work forks onto the plan's side streams (two, automatically, for
    stepwise plans) and joins back; every replay gives the oracle's bits."""
    say(f"case graph capture with events {mode}")
    w = Workload("graph-ev", 8, 12 * 40_000, "f32", "mean", "ring", dist="normal", sigma=1e-2,
                 seed=24, buckets=[(i * 40_000, 40_000) for i in reversed(range(12))])
    g = host_inputs(w)
    ref = [x.copy() for x in g]
    oracle_full(w, ref)
    src = to_device(g)
    bufs = [t.clone() for t in src]
    plan = make_plan(w, mode)
    events = [torch.cuda.Event() for _ in w.bucket_list()]
    main = torch.cuda.current_stream()
    for e in events:
        e.record(main)
    plan.execute(bufs, events=events, stream=main)   # binds the plan
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(main)
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for e in events:
                e.record(s)
            plan.execute(bufs, events=events, stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        for b, x in zip(bufs, src):
            b.copy_(x)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        out = [b.cpu().numpy() for b in bufs]
        for r in (0, 3, 7):
            assert bitwise_equal(out[r], ref[r]), (mode, rep, r)
    del graph
    torch.cuda.synchronize()
    plan.destroy()


F16_MEAN_P = [2, 3, 5, 6, 7, 9, 11, 13, 16, 24, 40, 63, 100, 127, 128]


@pytest.mark.parametrize("mode", ["fused1", "fused2", "step1", "step2"])
def test_f16_mean_of_every_value(mode):
    """The binary16 mean (Sony article, "训练设置": binary16 gradients;
    Baidu article, "总结": averaged) of every binary16 value.  Rank 0 holds
    all 65536 bit patterns and the other ranks zeros, so each element's sum
    is the value itself (+0 for -0, which meets a +0), and its mean must be
    the binary32 quotient by P correctly rounded, then rounded to binary16:
    numpy's division in binary32 gives it.  The one-kernel form runs every P
    from 1 to 128, the other forms a spread of P."""
    x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    ps = range(1, 129) if mode == "fused1" else F16_MEAN_P
    say(f"case binary16 mean of every value {mode}")
    for P in ps:
        w = Workload("f16mean", P, x.size, "f16", "mean", "ring", dist="normal", sigma=1.0,
                     seed=1)
        bufs = [torch.from_numpy(x.copy()).cuda()] + [
            torch.zeros(x.size, dtype=torch.float16, device="cuda") for _ in range(P - 1)]
        plan = make_plan(w, mode)
        plan.execute(bufs)
        out = to_host(bufs)
        plan.destroy()
        s = x.copy()
        if P > 1:
            s[s.view(np.uint16) == 0x8000] = 0
        with np.errstate(invalid="ignore"):   # NaN inputs stay NaN
            want = (s.astype(np.float32) / np.float32(P)).astype(np.float16)
        for r in (0, P - 1):
            if not bitwise_equal(out[r], want):
                bad = np.flatnonzero(out[r].view(np.uint16) != want.view(np.uint16))
                raise AssertionError(f"{mode} P={P} rank {r}: {bad.size} values differ, "
                                     f"first x bits {int(x.view(np.uint16)[bad[0]]):#06x}")
