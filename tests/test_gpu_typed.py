"""GPU parity of plans whose buckets carry their own element type.

Each rank's buffer is raw bytes; bucket b is a binary32 or binary16 segment
at its byte offset.  Every bucket is an independent all-reduce of its dtype,
so the expected bytes are the oracle's walk of that bucket alone.
"""
import numpy as np
import pytest

import oracle as orc
import sgd_gradient_all_amd as ddl
import synth

from _helpers import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

KINDS = {"ring": orc.RING, "multiring": orc.MULTIRING, "torus2d": orc.TORUS2D}


def layout(seed, nb, max_count):
    """Typed buckets in reverse memory order (output layer first), sizes
    ragged, binary16 offsets often not 16-byte multiples."""
    rng = np.random.default_rng(seed)
    segs, at = [], 0
    for _ in range(nb):
        dt = "f16" if rng.random() < 0.5 else "f32"
        esz = 4 if dt == "f32" else 2
        if at % esz:
            # a binary32 bucket after an odd binary16 one: the binary16
            # bucket takes one more element, so the buckets tile the buffer
            off, cnt, pdt = segs[-1]
            segs[-1] = (off, cnt + 1, pdt)
            at += 2
        cnt = int(rng.integers(1, max_count))
        segs.append((at, cnt, dt))
        at += cnt * esz
    return segs[::-1], at


def fill(P, segs, nbytes, seed):
    bufs = [np.zeros(nbytes, dtype=np.uint8) for _ in range(P)]
    for b, (off, cnt, dt) in enumerate(segs):
        sdt = synth.F32 if dt == "f32" else synth.F16
        for r in range(P):
            v = synth.fill_host(cnt, sdt, "normal", seed + b, r, sigma=1e-2)
            bufs[r][off:off + v.nbytes] = v.view(np.uint8)
    return bufs


def expected(P, segs, bufs, op, kind, k, rows, cols):
    out = [x.copy() for x in bufs]
    for off, cnt, dt in segs:
        npdt = np.float32 if dt == "f32" else np.float16
        nbytes = cnt * np.dtype(npdt).itemsize
        seg = [out[r][off:off + nbytes].view(npdt).copy() for r in range(P)]
        orc.allreduce(seg, op=orc.MEAN if op == "mean" else orc.SUM, kind=KINDS[kind], k=k,
                      rows=rows, cols=cols)
        for r in range(P):
            out[r][off:off + nbytes] = seg[r].view(np.uint8)
    return out


CASES = [
    # P, topology kwargs, buckets, max count
    (5, dict(kind="ring"), 9, 20_000),
    (16, dict(kind="multiring", k=4), 12, 30_000),
    (16, dict(kind="torus2d", rows=4, cols=4), 7, 50_000),
    (40, dict(kind="ring"), 6, 40_000),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("mode", ["fused1", "fused2", "step1", "step2"])
@pytest.mark.parametrize("gated", [False, True])
def test_typed_buckets_bitwise(case, mode, gated):
    P, tk, nb, mx = CASES[case]
    segs, nbytes = layout(100 + case, nb, mx)
    say(f"case typed P={P} {tk} buckets={nb} bytes={nbytes} mode={mode} gated={gated}")
    host = fill(P, segs, nbytes, 7 + case)
    want = expected(P, segs, host, "mean", tk["kind"], tk.get("k", 1), tk.get("rows", 0),
                    tk.get("cols", 0))
    # pad each rank's device buffer to 16 bytes (the library's alignment rule)
    dev = [torch.zeros(nbytes + 16, dtype=torch.uint8, device="cuda") for _ in range(P)]
    for d, h in zip(dev, host):
        d[:nbytes].copy_(torch.from_numpy(h))
    plan = ddl.Plan.typed(P, nbytes, "mean", ddl.topo(**tk), segs,
                          "stepwise" if mode.startswith("step") else "fused")
    if mode.startswith("step"):
        plan.set_step_form(int(mode[-1]))
    else:
        plan.set_fused_passes(1 if mode == "fused1" else 2)
    stream = torch.cuda.current_stream()
    events = None
    if gated:
        events = [torch.cuda.Event() for _ in segs]
        for e in events:
            e.record(stream)
    plan.execute(dev, events=events, stream=stream)
    torch.cuda.synchronize()
    plan.destroy()
    for r in (0, P // 2, P - 1):
        got = dev[r][:nbytes].cpu().numpy()
        assert got.tobytes() == want[r].tobytes(), (case, mode, r)


def test_resnet50_mixed_precision_full_size():
    """The mixed-precision ResNet-50 gradient at full size (16 ranks, 4
    rings; binary16 weights, binary32 BatchNorm and bias tensors), every
    byte of three ranks against the oracle, fused and stepwise."""
    from synth.workloads import resnet50_mixed_typed_buckets
    segs, nbytes = resnet50_mixed_typed_buckets()
    P, tk = 16, dict(kind="multiring", k=4)
    say(f"case typed resnet50 mixed: {len(segs)} buckets, {nbytes} bytes per rank")
    host = fill(P, segs, nbytes, 31)
    want = expected(P, segs, host, "mean", "multiring", 4, 0, 0)
    for mode in ("fused", "stepwise"):
        say(f"case typed resnet50 mixed mode={mode}")
        dev = [torch.zeros(nbytes, dtype=torch.uint8, device="cuda") for _ in range(P)]
        for d, h in zip(dev, host):
            d.copy_(torch.from_numpy(h))
        plan = ddl.Plan.typed(P, nbytes, "mean", ddl.topo(**tk), segs, mode)
        plan.execute(dev)
        torch.cuda.synchronize()
        plan.destroy()
        for r in (0, 7, P - 1):
            assert dev[r].cpu().numpy().tobytes() == want[r].tobytes(), (mode, r)
        del dev


def _paired_events(segs, stream):
    """One ready event per pair of consecutive buckets: groups of two
    buckets, often of two element types, whose passes run side by side."""
    evs = [torch.cuda.Event() for _ in range((len(segs) + 1) // 2)]
    for e in evs:
        e.record(stream)
    return [evs[b // 2] for b in range(len(segs))]


@pytest.mark.parametrize("mode", ["fused1", "fused2", "step1", "step2"])
def test_typed_mixed_groups_on_side_streams(mode):
    """Groups that hold both element types: the smaller type's pass runs on
    the plan's part stream beside the larger one's; every byte checked."""
    P, tk, nb, mx = CASES[1]
    segs, nbytes = layout(300, 14, mx)
    say(f"case typed mixed groups P={P} buckets={len(segs)} mode={mode}")
    host = fill(P, segs, nbytes, 17)
    want = expected(P, segs, host, "mean", "multiring", 4, 0, 0)
    dev = [torch.zeros(nbytes + 16, dtype=torch.uint8, device="cuda") for _ in range(P)]
    for d, h in zip(dev, host):
        d[:nbytes].copy_(torch.from_numpy(h))
    plan = ddl.Plan.typed(P, nbytes, "mean", ddl.topo(**tk), segs,
                          "stepwise" if mode.startswith("step") else "fused")
    if mode.startswith("step"):
        plan.set_step_form(int(mode[-1]))
    else:
        plan.set_fused_passes(1 if mode == "fused1" else 2)
    stream = torch.cuda.current_stream()
    plan.execute(dev, events=_paired_events(segs, stream), stream=stream)
    torch.cuda.synchronize()
    plan.destroy()
    for r in range(P):
        assert dev[r][:nbytes].cpu().numpy().tobytes() == want[r].tobytes(), (mode, r)


@pytest.mark.parametrize("mode", ["fused2", "step1", "step2"])
@pytest.mark.parametrize("gated", [False, True])
def test_typed_graph_capture_and_replay(mode, gated):
    """A typed plan's execution captured into a HIP graph (the element-type
    passes forked onto the part stream and joined back inside the capture)
    replays to the oracle's bytes, replay after replay, with the inputs
    restored eagerly in between."""
    P, tk, nb, mx = CASES[2]
    segs, nbytes = layout(301, 10, mx)
    say(f"case typed graph P={P} buckets={len(segs)} mode={mode} gated={gated}")
    host = fill(P, segs, nbytes, 19)
    want = expected(P, segs, host, "mean", "torus2d", 1, 4, 4)
    src = [torch.zeros(nbytes + 16, dtype=torch.uint8, device="cuda") for _ in range(P)]
    for d, h in zip(src, host):
        d[:nbytes].copy_(torch.from_numpy(h))
    dev = [t.clone() for t in src]
    plan = ddl.Plan.typed(P, nbytes, "mean", ddl.topo(**tk), segs,
                          "stepwise" if mode.startswith("step") else "fused")
    if mode.startswith("step"):
        plan.set_step_form(int(mode[-1]))
    else:
        plan.set_fused_passes(2)
    plan.execute(dev, stream=torch.cuda.current_stream())   # binds the plan
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            plan.execute(dev, events=_paired_events(segs, s) if gated else None, stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        for d, x in zip(dev, src):
            d.copy_(x)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for r in (0, 5, P - 1):
            assert dev[r][:nbytes].cpu().numpy().tobytes() == want[r].tobytes(), (mode, rep, r)
    del graph
    torch.cuda.synchronize()
    plan.destroy()
