"""GPU parity over seeded random configurations.

Each case draws a rank count, a topology (ring or multi-ring with random
ring orders, or a torus grid), an element type, an op, a ragged bucket list
in a random issue order (empty buckets and offsets that are not multiples of
16 bytes included), ready events shared by runs of consecutive buckets, a
coalescing threshold, a side-stream count and an execution form (one-kernel
or two-kernel fused pass, or step by step).  Every element of every rank is
compared bit for bit with the oracle's walk of the same schedule.
"""
import os

import numpy as np
import pytest

import oracle as orc
import sgd_gradient_all_amd as ddl
import synth

from _helpers import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# more cases on request: DDL_RANDOM_CASES / DDL_RANDOM_STEP_CASES
NCASES = int(os.environ.get("DDL_RANDOM_CASES", "48"))
NSTEP_CASES = int(os.environ.get("DDL_RANDOM_STEP_CASES", "24"))


def draw(seed, wide=False):
    """wide: rank counts up to 128 and buckets up to 2M elements."""
    rng = np.random.default_rng((5000 if wide else 1000) + seed)
    P = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 12, 16, 24, 40] +
                       ([48, 64, 96, 100, 127, 128] if wide else [])))
    dtype = str(rng.choice(["f32", "f16"]))
    op = str(rng.choice(["sum", "mean"]))
    kind = str(rng.choice(["ring", "multiring", "torus2d"]))
    k, rows, cols, order = 1, 0, 0, None
    if kind == "torus2d":
        divs = [r for r in range(1, P + 1) if P % r == 0]
        rows = int(rng.choice(divs))
        cols = P // rows
    else:
        if kind == "multiring":
            k = int(rng.integers(1, 6))
        if rng.random() < 0.6:
            order = np.concatenate([rng.permutation(P) for _ in range(k)]).astype(np.int32)
    nb = int(rng.integers(1, 12))
    sizes = []
    for _ in range(nb):
        r = rng.random()
        if r < 0.1:
            sizes.append(0)
        elif r < 0.4:
            sizes.append(int(rng.integers(1, 200)))
        elif r < 0.8:
            sizes.append(int(rng.integers(200, 20_000)))
        else:
            sizes.append(int(rng.integers(20_000, 2_000_000 if wide else 150_000)))
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(int).tolist()
    buckets = [(int(o), int(c)) for o, c in zip(offs, sizes)]
    perm = rng.permutation(nb)
    buckets = [buckets[i] for i in perm]
    n = int(sum(sizes))
    # runs of consecutive buckets share one event; some buckets get none
    ev_of, cur = [], 0
    for b in range(nb):
        if b and rng.random() < 0.5:
            cur += 1
        ev_of.append(None if rng.random() < 0.15 else cur)
    use_events = rng.random() < 0.7
    form = str(rng.choice(["fused1", "fused2", "stepwise"]))
    coalesce = int(rng.choice([0, 0, 4096, 1 << 20]))
    nside = int(rng.integers(0, 5))
    # stepwise: one launch per step (1) or the persistent step kernel (2)
    step_form = int(rng.integers(1, 3))
    return dict(P=P, dtype=dtype, op=op, kind=kind, k=k, rows=rows, cols=cols, order=order,
                buckets=buckets, n=n, ev_of=ev_of if use_events else None, form=form,
                coalesce=coalesce, nside=nside, seed=seed, step_form=step_form)


NWIDE_CASES = int(os.environ.get("DDL_RANDOM_WIDE_CASES", "4"))


@pytest.mark.parametrize("seed", [("base", s) for s in range(NCASES)] +
                         [("wide", s) for s in range(NWIDE_CASES)], ids=str)
def test_random_configuration(seed):
    kind_, seed = seed
    run_drawn(draw(seed, wide=kind_ == "wide"), f"random {seed}")


NRANKS_CASES = int(os.environ.get("DDL_RANDOM_RANKS_CASES", "16"))


@pytest.mark.parametrize("seed", range(NRANKS_CASES))
def test_random_rank_by_rank_reduce(seed):
    """The two-kernel pass with its reduce kernel rank by rank at every rank
    count (reduce_ranks_min_p = 0: four tiles per workgroup under 32 ranks,
    six from 32 on), on drawn configurations -- ragged, empty and
    misaligned buckets, rings, multi-rings and tori, both element types --
    every rank bit for bit against the oracle."""
    c = draw(300 + seed, wide=seed % 4 == 3)
    c["form"] = "fused2"
    ddl.set_tuning("reduce_ranks_min_p", 0)
    try:
        run_drawn(c, f"random rank-by-rank {seed}")
    finally:
        ddl.set_tuning("reduce_ranks_min_p", -1)


def run_drawn(c, tag):
    """One all-reduce of a drawn configuration against the oracle."""
    seed = c["seed"]
    say(f"case {tag}: P={c['P']} {c['dtype']} {c['op']} {c['kind']} k={c['k']} "
        f"grid={c['rows']}x{c['cols']} n={c['n']} buckets={len(c['buckets'])} "
        f"form={c['form']}/{c['step_form']} events={c['ev_of'] is not None} "
        f"coalesce={c['coalesce']} "
        f"side={c['nside']}")
    P, n = c["P"], c["n"]
    sdt = synth.F32 if c["dtype"] == "f32" else synth.F16
    g = [synth.fill_host(n, sdt, "normal", 500 + c["seed"], r, sigma=1e-2) for r in range(P)]
    want = [x.copy() for x in g]
    kinds = {"ring": orc.RING, "multiring": orc.MULTIRING, "torus2d": orc.TORUS2D}
    orc.allreduce(want, op=orc.SUM if c["op"] == "sum" else orc.MEAN, kind=kinds[c["kind"]],
                  k=c["k"], rows=c["rows"], cols=c["cols"], ring_order=c["order"],
                  buckets=c["buckets"])
    bufs = [torch.from_numpy(x).cuda() for x in g]
    topo = ddl.topo(c["kind"], c["k"], c["rows"], c["cols"],
                    ring_order=None if c["order"] is None else c["order"].tolist())
    mode = "stepwise" if c["form"] == "stepwise" else "fused"
    plan = ddl.Plan(P, n, c["dtype"], c["op"], topo, c["buckets"], mode)
    if mode == "fused":
        plan.set_fused_passes(1 if c["form"] == "fused1" else 2)
    else:
        plan.set_step_form(c["step_form"])
    plan.set_coalesce_bytes(c["coalesce"])
    plan.set_side_streams(c["nside"])
    stream = torch.cuda.current_stream()
    events = None
    if c["ev_of"] is not None:
        pool = {}
        events = []
        for e in c["ev_of"]:
            if e is None:
                events.append(None)
            else:
                if e not in pool:
                    pool[e] = torch.cuda.Event()
                    pool[e].record(stream)
                events.append(pool[e])
    plan.execute(bufs, events=events, stream=stream)
    torch.cuda.synchronize()
    plan.destroy()
    for r in range(P):
        got = bufs[r].cpu().numpy()
        assert got.tobytes() == want[r].tobytes(), (seed, r)


@pytest.mark.parametrize("seed", range(NSTEP_CASES))
def test_random_sgd_and_lars(seed):
    """The SGD step (kept or dropped gradients) or the LARS step on a drawn
    configuration, with shared or per-rank weight replicas; SGD bit for bit,
    LARS to the tolerance of tests/test_gpu_lars.py."""
    from test_gpu_lars import check_lars
    c = draw(100 + seed)
    rng = np.random.default_rng(7000 + seed)
    step = str(rng.choice(["sgd_keep", "sgd_drop", "lars"]))
    if step == "sgd_drop" and c["form"] == "stepwise":
        c["form"] = "fused2"
    shared = bool(rng.random() < 0.4)
    lr = float(rng.choice([0.01, 0.1, 0.5]))
    say(f"case random {step} {seed}: P={c['P']} {c['dtype']} {c['op']} {c['kind']} "
        f"k={c['k']} grid={c['rows']}x{c['cols']} n={c['n']} buckets={len(c['buckets'])} "
        f"form={c['form']} shared={shared} events={c['ev_of'] is not None}")
    P, n = c["P"], c["n"]
    sdt = synth.F32 if c["dtype"] == "f32" else synth.F16
    g = [synth.fill_host(n, sdt, "normal", 800 + seed, r, sigma=1e-2) for r in range(P)]
    w0 = (rng.standard_normal(n) * 0.1).astype(np.float32)
    nrep = 1 if shared else P
    y = [x.copy() for x in g]
    kinds = {"ring": orc.RING, "multiring": orc.MULTIRING, "torus2d": orc.TORUS2D}
    orc.allreduce(y, op=orc.SUM if c["op"] == "sum" else orc.MEAN, kind=kinds[c["kind"]],
                  k=c["k"], rows=c["rows"], cols=c["cols"], ring_order=c["order"],
                  buckets=c["buckets"])
    want_w = [w0.copy() for _ in range(nrep)]
    if step == "lars":
        want_rates = orc.lars(want_w, y[0], c["buckets"], lr)
    else:
        orc.sgd(want_w, y[0], lr)
    bufs = [torch.from_numpy(x).cuda() for x in g]
    weights = [torch.from_numpy(w0.copy()).cuda() for _ in range(nrep)]
    rates = torch.zeros(max(1, len(c["buckets"])), dtype=torch.float32, device="cuda")
    topo = ddl.topo(c["kind"], c["k"], c["rows"], c["cols"],
                    ring_order=None if c["order"] is None else c["order"].tolist())
    mode = "stepwise" if c["form"] == "stepwise" else "fused"
    plan = ddl.Plan(P, n, c["dtype"], c["op"], topo, c["buckets"], mode)
    if mode == "fused":
        plan.set_fused_passes(1 if c["form"] == "fused1" else 2)
    else:
        plan.set_step_form(c["step_form"])   # the SGD and LARS steps ride on either form
    plan.set_side_streams(c["nside"])
    stream = torch.cuda.current_stream()
    events = None
    if c["ev_of"] is not None:
        pool, events = {}, []
        for e in c["ev_of"]:
            if e is None:
                events.append(None)
            else:
                if e not in pool:
                    pool[e] = torch.cuda.Event()
                    pool[e].record(stream)
                events.append(pool[e])
    if step == "lars":
        plan.execute_lars(bufs, weights, lr, rates_out=rates, events=events, stream=stream)
    else:
        plan.execute_sgd(bufs, weights, lr, keep_grads=step == "sgd_keep", events=events,
                         stream=stream)
    torch.cuda.synchronize()
    plan.destroy()
    want_g = g if step == "sgd_drop" else y
    for r in range(P):
        assert bufs[r].cpu().numpy().tobytes() == want_g[r].tobytes(), (seed, "grads", r)
    for r in range(nrep):
        got = weights[r].cpu().numpy()
        if step == "lars":
            check_lars(got, want_w[r], rates.cpu().numpy(), want_rates, y[0], c["buckets"],
                       (seed, r))
        else:
            assert got.tobytes() == want_w[r].tobytes(), (seed, "weights", r)


NTYPED_CASES = int(os.environ.get("DDL_RANDOM_TYPED_CASES", "16"))


@pytest.mark.parametrize("seed", range(NTYPED_CASES))
def test_random_typed_configuration(seed):
    """Plans whose buckets carry their own element type: a drawn topology and
    form over a random mixed layout (binary16 and binary32 buckets, odd
    binary16 counts, empty buckets), with or without shared ready events;
    every byte against the oracle's walk of each bucket alone."""
    from test_gpu_typed import expected, fill
    c = draw(3000 + seed)
    rng = np.random.default_rng(9000 + seed)
    P = c["P"]
    segs, at = [], 0
    for _ in range(int(rng.integers(1, 14))):
        dt = "f16" if rng.random() < 0.5 else "f32"
        esz = 4 if dt == "f32" else 2
        if at % esz:
            off, cnt, pdt = segs[-1]
            segs[-1] = (off, cnt + 1, pdt)
            at += 2
        r = rng.random()
        cnt = 0 if r < 0.08 else int(rng.integers(1, 300 if r < 0.4 else 60_000))
        segs.append((at, cnt, dt))
        at += cnt * esz
    if at % 4:   # keep the total a whole number of binary32 elements
        off, cnt, pdt = segs[-1]
        segs[-1] = (off, cnt + 1, pdt)
        at += 2
    order = list(rng.permutation(len(segs)))
    segs = [segs[i] for i in order]
    nbytes = at
    tk = {"kind": c["kind"], "k": c["k"], "rows": c["rows"], "cols": c["cols"]}
    say(f"case random typed {seed}: P={P} {c['kind']} k={c['k']} grid={c['rows']}x{c['cols']} "
        f"buckets={len(segs)} bytes={nbytes} form={c['form']} events={c['ev_of'] is not None}")
    host = fill(P, segs, nbytes, 60 + seed)
    want = expected(P, segs, host, c["op"], c["kind"], c["k"], c["rows"], c["cols"])
    dev = [torch.zeros(nbytes + 16, dtype=torch.uint8, device="cuda") for _ in range(P)]
    for d, h in zip(dev, host):
        d[:nbytes].copy_(torch.from_numpy(h))
    mode = "stepwise" if c["form"] == "stepwise" else "fused"
    plan = ddl.Plan.typed(P, nbytes, c["op"],
                          ddl.topo(tk["kind"], tk["k"], tk["rows"], tk["cols"]), segs, mode)
    if mode == "fused":
        plan.set_fused_passes(1 if c["form"] == "fused1" else 2)
    plan.set_side_streams(c["nside"])
    stream = torch.cuda.current_stream()
    events = None
    if rng.random() < 0.7:
        pool, events = {}, []
        for b in range(len(segs)):
            key = b // int(rng.integers(1, 4))
            if key not in pool:
                pool[key] = torch.cuda.Event()
                pool[key].record(stream)
            events.append(pool[key])
    plan.execute(dev, events=events, stream=stream)
    torch.cuda.synchronize()
    plan.destroy()
    for r in range(P):
        assert dev[r][:nbytes].cpu().numpy().tobytes() == want[r].tobytes(), (seed, r)
