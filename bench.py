#!/usr/bin/env python3
"""Benchmark of the gradient all-reduce on one MI355X.

One step = one all-reduce of the workload (default: 40 virtual ranks of 300M
fp32 gradients each, 48 GB, 64 equal buckets issued last-first, each gated
by its own ready event on the library's side stream), inputs resident in HBM.
Prints one JSON line: achieved HBM GB/s (the algorithmic bytes of the fused
pass, every rank's input read once and its result written once, over the
step time), the roofline of the dominant kernel from HIP events around each
of its launches, the CPU oracle timed on a bounded sample of the same
workload, and side measurements (step-by-step mode, overlap with a streaming
compute kernel).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s and % of peak per all-reduce (300M fp32, P=40 ring)"
LEGS = ("stepwise", "overlap", "sgd", "lars", "typed", "per_gpu_step", "configs")
PEAK_HBM_GBPS = 8000.0
# committed counter summaries: one file per form of the fused pass
TRAFFIC_FILES = {1: ("fused_kernel", "hbm_bytes_per_launch"),
                 2: ("fused_pass", "hbm_bytes_per_pass")}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    """Hash of the fused pass's sources (kernels, launch configuration, tile
    tables): counter figures taken on another version are not reported."""
    h = hashlib.sha256()
    for name in ("fused_kernel.hip", "device_common.h", "ddl_internal.h", "plan.cpp",
                 "schedule.cpp"):
        with open(os.path.join(ROOT, "sgd_gradient_all_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, mode, passes):
    """HBM bytes per launch (one-kernel form) or per reduce + broadcast pair
    (two-kernel form) from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source."""
    if mode != "fused" or passes not in TRAFFIC_FILES:
        return None
    stem, key = TRAFFIC_FILES[passes]
    path = os.path.join(ROOT, "profiles", f"{stem}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get(key)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="ring_p40_300m_64b")
    ap.add_argument("--mode", default=os.environ.get("DDL_MODE", "fused"),
                    choices=["fused", "stepwise"], help="default: $DDL_MODE, else fused")
    ap.add_argument("--coalesce-bytes", type=int,
                    default=int(os.environ.get("DDL_COALESCE", "0")),
                    help="the headline plan's grouping threshold in bytes per rank "
                         "(ddl_plan_set_coalesce_bytes; default: $DDL_COALESCE, else 0)")
    ap.add_argument("--passes", type=int, default=0, choices=[0, 1, 2],
                    help="fused pass form: 0 the plan's choice, 1 one kernel, "
                         "2 reduce + broadcast kernels")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip every side measurement (--legs)")
    ap.add_argument("--legs", default=",".join(LEGS),
                    help="comma-separated side measurements to run, of: " + ", ".join(LEGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-buckets", type=int, default=64,
                    help="buckets of the workload the CPU oracle is timed on")
    ap.add_argument("--calib-copy-gib", type=float, default=0.0,
                    help="also run one plain device copy of this size (counter calibration)")
    args = ap.parse_args()
    args.legs = [] if args.no_extras else [x for x in args.legs.split(",") if x]
    for leg in args.legs:
        if leg not in LEGS:
            ap.error(f"unknown leg {leg!r}; known: {', '.join(LEGS)}")

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the all-reduce runs P virtual ranks on a single "
              f"MI355X, so --gpus {args.gpus} (WORLD_SIZE={world}) is not supported; "
              f"run with --gpus 1", flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import sgd_gradient_all_amd as ddl
    import synth
    from synth.workloads import WORKLOADS

    w = WORKLOADS[args.workload]
    tdt = torch.float32 if w.dtype == "f32" else torch.float16
    sdt = synth.F32 if w.dtype == "f32" else synth.F16
    torch.cuda.set_device(0)
    dev_name = torch.cuda.get_device_name(0)
    log(f"bench: {w.name} ({w.description}) on {dev_name}, mode={args.mode}")

    # inputs, generated in HBM
    bufs = [torch.empty(w.n, dtype=tdt, device="cuda") for _ in range(w.P)]
    for r, b in enumerate(bufs):
        synth.fill_device(b.data_ptr(), w.n, sdt, w.dist, w.seed, r, sigma=w.sigma)
    torch.cuda.synchronize()
    log("bench: inputs ready")

    topo = ddl.topo(w.topo, w.k, w.rows, w.cols)
    buckets = w.bucket_list()
    main_stream = torch.cuda.current_stream()

    def make_events():
        return [torch.cuda.Event() for _ in buckets] if w.side_stream else None

    def record_all(evs):
        if evs:
            for e in evs:
                e.record(main_stream)

    def run_steps(plan, evs, steps):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(main_stream)
        for _ in range(steps):
            record_all(evs)
            plan.execute(bufs, events=evs, stream=main_stream)
        t1.record(main_stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    t_plan = time.perf_counter()
    plan = ddl.Plan(w.P, w.n, w.dtype, w.op, topo, buckets, args.mode)
    plan_build_ms = (time.perf_counter() - t_plan) * 1e3
    if args.mode == "fused":
        plan.set_fused_passes(args.passes)
    if args.coalesce_bytes:
        plan.set_coalesce_bytes(args.coalesce_bytes)
    passes = plan.fused_passes()
    _, hbm_bytes = plan.traffic()
    evs = make_events()
    for _ in range(args.warmup):
        record_all(evs)
        plan.execute(bufs, events=evs, stream=main_stream)
    torch.cuda.synchronize()
    # timed region 1: the steps alone -> value, ms_per_step
    ms = run_steps(plan, evs, args.steps)
    # timed region 2: the same steps with a HIP event pair around every
    # launch, on the stream it is launched on -> the kernel's roofline
    plan.set_profiling(True)
    plan.profile_read()
    ms_prof = run_steps(plan, evs, args.steps)
    kinds = plan.profile_read_kinds()
    value = hbm_bytes / (ms * 1e-3) / 1e9
    kernels = {}
    if passes == 2:
        # the unit is one reduce + broadcast pair: the fused pass of a group,
        # credited with the pass's algorithmic bytes (every rank's input read
        # once, every rank's result written once); the reduced values the
        # broadcast re-reads are counted in the per-kernel figures
        red, bc = kinds["fused_reduce"], kinds["broadcast"]
        launches = red[1]
        avg_launch_ms = red[0] / red[1] + bc[0] / bc[1]
        kmax = red[2] + bc[2]
        bytes_per_launch = hbm_bytes / (launches / args.steps)
        rk = bytes_per_launch * (w.P + 1) / (2 * w.P)   # P reads + 1 write
        bk = bytes_per_launch / 2                        # 1 read + P-1 writes
        for name, (tot, cnt, mx), nb in (("fused_reduce_kernel", red, rk),
                                          ("bcast_kernel", bc, bk)):
            kernels[name] = {"launches_per_step": cnt / args.steps,
                             "avg_launch_us": round(tot / cnt * 1e3, 2),
                             "max_launch_us": round(mx * 1e3, 2),
                             "algorithmic_bytes_per_launch": int(nb),
                             "GBps": round(nb / (tot / cnt * 1e-3) / 1e9, 1)}
        kernel_name = "fused pass: fused_reduce_kernel + bcast_kernel"
    else:
        kms = sum(v[0] for v in kinds.values())
        launches = sum(v[1] for v in kinds.values())
        kmax = max(v[2] for v in kinds.values())
        avg_launch_ms = kms / launches
        bytes_per_launch = hbm_bytes / (launches / args.steps)
        kernel_name = "fused_kernel" if args.mode == "fused" else "step_kernel"
    launches_per_step = launches / args.steps
    achieved = bytes_per_launch / (avg_launch_ms * 1e-3) / 1e9
    log(f"bench: {ms:.3f} ms/step, {value:.1f} GB/s; {launches_per_step:.0f} "
        f"{'passes' if passes == 2 else 'launches'}/step, avg {avg_launch_ms * 1e3:.1f} us, "
        f"kernel-side {achieved:.1f} GB/s (profiled steps {ms_prof:.3f} ms) {kernels or ''}")
    esize = 4 if w.dtype == "f32" else 2
    bus_bw = 2 * (w.P - 1) / w.P * w.n * esize / (ms * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded counter-based generator, generated in HBM)",
        "config": {"workload": w.name, "P": w.P, "n": w.n, "topology": w.topo, "k": w.k,
                   "rows": w.rows, "cols": w.cols, "op": w.op, "buckets": len(buckets),
                   "side_stream": w.side_stream, "mode": args.mode,
                   "coalesce_bytes": args.coalesce_bytes,
                   "fused_passes": passes, "bytes_per_step": hbm_bytes},
        "pct_of_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "bus_bw_GBps": round(bus_bw, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": kernel_name,
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": measured_traffic(w.name, args.mode, passes),
            "launches_per_step": launches_per_step,
            "avg_launch_us": round(avg_launch_ms * 1e3, 2),
            "max_launch_us": round(kmax * 1e3, 2),
            "algorithmic_bytes_per_launch": int(bytes_per_launch),
            "profiled_ms_per_step": round(ms_prof, 4),
        },
        **({"pass_kernels": kernels} if kernels else {}),
        "plan_build_ms": round(plan_build_ms, 2),
        "device": dev_name,
    }
    plan.destroy()

    if args.calib_copy_gib > 0:
        nel = int(args.calib_copy_gib * (1 << 30) / 4)
        a = torch.empty(nel, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1.0)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        result["calib_copy_bytes"] = 2 * nel * 4
        del a, b

    if args.legs:
        result.update(extras(args, w, bufs, topo, buckets, main_stream, torch, ddl, synth,
                             hbm_bytes, ms))

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, w, topo, torch, ddl, synth, np)

    print(json.dumps(result), flush=True)


def extras(args, w, bufs, topo, buckets, main_stream, torch, ddl, synth, fused_bytes, fused_ms):
    out = {}
    if "stepwise" in args.legs:
        out["stepwise"] = stepwise_leg(w, bufs, topo, buckets, main_stream, torch, ddl,
                                       fused_bytes)
    if "overlap" in args.legs and w.side_stream:
        out["overlap"] = overlap_leg(w, bufs, topo, buckets, main_stream, torch, ddl, synth,
                                     fused_bytes, fused_ms)
    if "sgd" in args.legs:
        out["sgd"] = sgd_leg(w, bufs, topo, buckets, main_stream, torch, ddl, synth, fused_ms,
                             args.passes)
    if "lars" in args.legs:
        out["lars"] = lars_leg(w, bufs, topo, buckets, main_stream, torch, ddl, synth, fused_ms,
                               args.passes)
    if "typed" in args.legs:
        out["typed"] = typed_leg(main_stream, torch, ddl, synth)
    if "configs" in args.legs:
        out["configs"] = configs_leg(w, main_stream, torch, ddl, synth)
    if "per_gpu_step" in args.legs:
        out["per_gpu_step"] = per_gpu_step_leg(w, main_stream, torch, ddl)
    return out


def configs_leg(head, main_stream, torch, ddl, synth):
    """The other workloads, each in its plan's default fused form on fresh
    inputs: ms per all-reduce and HBM GB/s over its algorithmic bytes (the
    4-rank 2^20 case fits the caches, so its figure is not an HBM one)."""
    from synth.workloads import WORKLOADS
    out = {}
    for name, w in WORKLOADS.items():
        if name == head.name:
            continue
        tdt = torch.float32 if w.dtype == "f32" else torch.float16
        sdt = synth.F32 if w.dtype == "f32" else synth.F16
        bufs = [torch.empty(w.n, dtype=tdt, device="cuda") for _ in range(w.P)]
        for r, b in enumerate(bufs):
            synth.fill_device(b.data_ptr(), w.n, sdt, w.dist, w.seed, r, sigma=w.sigma)
        torch.cuda.synchronize()
        buckets = w.bucket_list()
        evs = [torch.cuda.Event() for _ in buckets] if w.side_stream else None
        plan = ddl.Plan(w.P, w.n, w.dtype, w.op, ddl.topo(w.topo, w.k, w.rows, w.cols),
                        buckets, "fused")
        _, nbytes = plan.traffic()
        reps = 10 if nbytes > (4 << 30) else 50

        def run(k):
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record(main_stream)
            for _ in range(k):
                if evs:
                    for e in evs:
                        e.record(main_stream)
                plan.execute(bufs, events=evs, stream=main_stream)
            t1.record(main_stream)
            torch.cuda.synchronize()
            return t0.elapsed_time(t1) / k

        run(3)
        ms = run(reps)
        gbps = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 4), "hbm_GBps": round(gbps, 1),
                     "pct_of_peak": round(100 * gbps / PEAK_HBM_GBPS, 2),
                     "fused_passes": plan.fused_passes(), "bytes": nbytes,
                     "cache_resident": nbytes < (256 << 20)}
        plan.destroy()
        del bufs
        torch.cuda.empty_cache()
    log(f"bench: configs {out}")
    return out


def stepwise_leg(w, bufs, topo, buckets, main_stream, torch, ddl, fused_bytes):
    """The step-by-step schedule on the same buffers: timed without
    per-launch events, replayed from a HIP graph, then one profiled pass for
    the kernel-side figures."""
    plan = ddl.Plan(w.P, w.n, w.dtype, w.op, topo, buckets, "stepwise")
    _, sbytes = plan.traffic()
    evs = [torch.cuda.Event() for _ in buckets] if w.side_stream else None

    def step_once():
        if evs:
            for e in evs:
                e.record(main_stream)
        plan.execute(bufs, events=evs, stream=main_stream)

    step_once()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    steps = 3
    t0.record(main_stream)
    for _ in range(steps):
        step_once()
    t1.record(main_stream)
    torch.cuda.synchronize()
    sms = t0.elapsed_time(t1) / steps
    # the same execution captured once into a HIP graph and replayed: the
    # thousands of step launches are then issued by one graph launch
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(main_stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            if evs:
                for e in evs:
                    e.record(cap)
            plan.execute(bufs, events=evs, stream=cap)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    t0.record(main_stream)
    for _ in range(steps):
        graph.replay()
    t1.record(main_stream)
    torch.cuda.synchronize()
    gms = t0.elapsed_time(t1) / steps
    del graph
    # the per-kernel figures come from one profiled step on a single side
    # stream: overlapping launches would stretch each one's duration
    plan.set_side_streams(1)
    plan.set_profiling(True)
    step_once()
    torch.cuda.synchronize()
    kinds = plan.profile_read_kinds()
    plan.set_side_streams(0)
    launches = sum(v[1] for v in kinds.values())
    kms = sum(v[0] for v in kinds.values())
    # per step kernel: its algorithmic bytes per launch over its average
    # duration (3 L s per reduce-scatter launch, 2 L s per all-gather one)
    kernel_rows = {}
    for kind, share in (("reduce", 3), ("gather", 2)):
        tot, cnt, mx = kinds[kind]
        if cnt:
            nb = share * sbytes / 5 / cnt   # the step bytes split 3 : 2
            kernel_rows[kind + "_step_kernel"] = {
                "launches_per_step": cnt, "avg_launch_us": round(tot / cnt * 1e3, 2),
                "max_launch_us": round(mx * 1e3, 2), "algorithmic_bytes_per_launch": int(nb),
                "GBps": round(nb / (tot / cnt * 1e-3) / 1e9, 1)}
    res = {"ms_per_step": round(sms, 3),
                       "graph_ms_per_step": round(gms, 3),
                       "hbm_GBps": round(sbytes / (sms * 1e-3) / 1e9, 1),
                       "fused_floor_equiv_GBps": round(fused_bytes / (sms * 1e-3) / 1e9, 1),
                       "bytes_per_step": sbytes,
                       "launches_per_step": launches,
                       "avg_launch_us": round(kms / max(launches, 1) * 1e3, 2),
                       **kernel_rows}
    plan.destroy()
    log(f"bench: stepwise {res}")
    return res


def overlap_leg(w, bufs, topo, buckets, main_stream, torch, ddl, synth, fused_bytes, fused_ms):
    """Overlap with a streaming compute kernel standing in for the rest of
    back-propagation: 0.925 x the all-reduce's bytes (the Baidu article's
    ~370 ms compute vs ~400 ms communication), in one slice per bucket;
    bucket b waits for slice b."""
    nb = len(buckets)
    comp_elems = int(0.925 * fused_bytes / 8) // (4 * nb) * (4 * nb)
    free = torch.cuda.mem_get_info()[0]
    if comp_elems * 4 > free * 0.9:
        comp_elems = int(free * 0.9 / 4) // (4 * nb) * (4 * nb)
    scratch = torch.zeros(comp_elems, dtype=torch.float32, device="cuda")
    per = comp_elems // nb
    cs = main_stream.cuda_stream

    def compute_slices(evs):
        for i in range(nb):
            synth.stream_compute(scratch.data_ptr() + 4 * i * per, per, 1.0, 0.0, cs)
            if evs is not None:
                evs[i].record(main_stream)

    plan = ddl.Plan(w.P, w.n, w.dtype, w.op, topo, buckets, "fused")
    evs = [torch.cuda.Event() for _ in buckets]
    compute_slices(None)
    torch.cuda.synchronize()
    reps = 3
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(main_stream)
    for _ in range(reps):
        compute_slices(None)
    t1.record(main_stream)
    torch.cuda.synchronize()
    t_comp = t0.elapsed_time(t1) / reps
    compute_slices(evs)
    plan.execute(bufs, events=evs, stream=main_stream)
    torch.cuda.synchronize()
    t0.record(main_stream)
    for _ in range(reps):
        compute_slices(evs)
        plan.execute(bufs, events=evs, stream=main_stream)
    t1.record(main_stream)
    torch.cuda.synchronize()
    t_both = t0.elapsed_time(t1) / reps
    comp_bytes = 2 * 4 * comp_elems
    res = {
        "t_allreduce_ms": round(fused_ms, 3), "t_compute_ms": round(t_comp, 3),
        "t_both_ms": round(t_both, 3),
        "overlap_efficiency": round((fused_ms + t_comp - t_both) / min(fused_ms, t_comp), 3),
        "combined_hbm_GBps": round((fused_bytes + comp_bytes) / (t_both * 1e-3) / 1e9, 1),
        "compute_bytes": comp_bytes,
    }
    plan.destroy()
    del scratch
    torch.cuda.empty_cache()
    log(f"bench: overlap {res}")
    return res


def per_gpu_step_leg(w, main_stream, torch, ddl):
    """One GPU's share of a real ring step: a chunk of the workload's bucket
    (L / P elements) added into, or copied over, one neighbour's -- timed as
    the step kernels of a two-rank ring over two such chunks (each of its
    steps holds two pairs, one per rank: two GPUs' shares in one launch)."""
    L = (w.bucket_list()[0][1] + w.P - 1) // w.P
    L = (L + 3) // 4 * 4
    tdt = torch.float32 if w.dtype == "f32" else torch.float16
    bufs = [torch.ones(2 * L, dtype=tdt, device="cuda") for _ in range(2)]
    plan = ddl.Plan(2, 2 * L, w.dtype, "sum", ddl.topo("ring"), None, "stepwise")
    plan.execute(bufs, stream=main_stream)
    torch.cuda.synchronize()
    plan.set_profiling(True)
    plan.profile_read_kinds()
    reps = 200
    for _ in range(reps):
        plan.execute(bufs, stream=main_stream)
    torch.cuda.synchronize()
    k = plan.profile_read_kinds()
    plan.destroy()
    esz = 4 if w.dtype == "f32" else 2
    res = {"chunk_elements": L, "chunks_per_launch": 2}
    for kind, nbytes in (("reduce", 2 * 3 * L * esz), ("gather", 2 * 2 * L * esz)):
        tot, cnt, _ = k[kind]
        us = tot / cnt * 1e3
        res[kind] = {"avg_launch_us": round(us, 2), "bytes": nbytes,
                     "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}
    log(f"bench: per-GPU step {res}")
    return res


def typed_leg(main_stream, torch, ddl, synth):
    """Buckets of their own element type: the mixed-precision ResNet-50
    gradient (binary16 weights, binary32 BatchNorm and bias tensors) over 16
    ranks and 4 rings, fused and stepwise."""
    from synth.workloads import resnet50_mixed_typed_buckets
    segs, nbytes = resnet50_mixed_typed_buckets()
    P = 16
    tb = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(P)]
    for r, t in enumerate(tb):
        for b, (off, cnt, dt) in enumerate(segs):
            synth.fill_device(t.data_ptr() + off, cnt, synth.F32 if dt == "f32" else synth.F16,
                              "normal", 40 + b, r, sigma=1e-2)
    torch.cuda.synchronize()
    res = {"ranks": P, "topology": "4 rings", "buckets": len(segs), "bytes_per_rank": nbytes}
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for mode in ("fused", "stepwise"):
        plan = ddl.Plan.typed(P, nbytes, "mean", ddl.topo("multiring", 4), segs, mode)
        _, hbm = plan.traffic()
        plan.execute(tb, stream=main_stream)
        torch.cuda.synchronize()
        reps = 20
        t0.record(main_stream)
        for _ in range(reps):
            plan.execute(tb, stream=main_stream)
        t1.record(main_stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / reps
        res[mode] = {"ms": round(ms, 4), "hbm_GBps": round(hbm / (ms * 1e-3) / 1e9, 1),
                     "bytes": hbm}
        plan.destroy()
    del tb
    torch.cuda.empty_cache()
    log(f"bench: typed {res}")
    return res


def sgd_leg(w, bufs, topo, buckets, main_stream, torch, ddl, synth, fused_ms, passes=0):
    """The SGD step fused into the all-reduce's epilogue, against the
    all-reduce followed by a separate update of every replica."""
    lr = 0.01
    esz = 4 if w.dtype == "f32" else 2
    free = torch.cuda.mem_get_info()[0]
    nrep = w.P if w.P * w.n * 4 < 0.8 * free else 1
    weights = [torch.empty(w.n, dtype=torch.float32, device="cuda") for _ in range(nrep)]
    for t in weights:
        synth.fill_device(t.data_ptr(), w.n, synth.F32, "uniform", 77, 0)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event() for _ in buckets] if w.side_stream else None
    plan = ddl.Plan(w.P, w.n, w.dtype, w.op, topo, buckets, "fused")
    plan.set_fused_passes(passes)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {"replicas": nrep, "lr": lr, "fused_passes": plan.fused_passes()}
    for keep in (True, False):
        def one():
            if evs:
                for e in evs:
                    e.record(main_stream)
            plan.execute_sgd(bufs, weights, lr, keep_grads=keep, events=evs, stream=main_stream)
        one()
        torch.cuda.synchronize()
        reps = 3
        t0.record(main_stream)
        for _ in range(reps):
            one()
        t1.record(main_stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / reps
        nbytes = (2 if keep else 1) * w.P * w.n * esz + 2 * 4 * nrep * w.n
        res["keep_grads" if keep else "drop_grads"] = {
            "ms": round(ms, 3), "hbm_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "bytes": nbytes}
    plan.destroy()
    # the unfused baseline: the all-reduce, then w -= lr * y on every replica
    gview = [b if b.dtype == torch.float32 else b.float() for b in bufs[:1]]
    def separate():
        torch._foreach_add_(weights, [gview[0]] * nrep, alpha=-lr)
    separate()
    torch.cuda.synchronize()
    reps = 3
    t0.record(main_stream)
    for _ in range(reps):
        separate()
    t1.record(main_stream)
    torch.cuda.synchronize()
    upd_ms = t0.elapsed_time(t1) / reps
    res["separate_update_ms"] = round(upd_ms, 3)
    res["allreduce_plus_separate_ms"] = round(fused_ms + upd_ms, 3)
    del weights
    torch.cuda.empty_cache()
    log(f"bench: sgd {res}")
    return res


def lars_leg(w, bufs, topo, buckets, main_stream, torch, ddl, synth, fused_ms, passes=0):
    """The LARS step after the all-reduce (every bucket a layer; the Sony
    article's coefficient 0.01 and eps 1e-6), one weight replica per rank
    (one shared replica when HBM is short): the whole step's time, and each
    LARS kernel's average launch against its algorithmic bytes, from one
    profiled step."""
    lr = 0.01
    esz = 4 if w.dtype == "f32" else 2
    free = torch.cuda.mem_get_info()[0]
    nrep = w.P if w.P * w.n * 4 < 0.8 * free else 1
    weights = [torch.empty(w.n, dtype=torch.float32, device="cuda") for _ in range(nrep)]
    for t in weights:
        synth.fill_device(t.data_ptr(), w.n, synth.F32, "uniform", 77, 0)
    rates = torch.zeros(len(buckets), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    evs = [torch.cuda.Event() for _ in buckets] if w.side_stream else None
    plan = ddl.Plan(w.P, w.n, w.dtype, w.op, topo, buckets, "fused")
    plan.set_fused_passes(passes)
    _, ar_bytes = plan.traffic()

    def one():
        if evs:
            for e in evs:
                e.record(main_stream)
        plan.execute_lars(bufs, weights, lr, rates_out=rates, events=evs, stream=main_stream)

    one()
    torch.cuda.synchronize()
    reps = 3
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(main_stream)
    for _ in range(reps):
        one()
    t1.record(main_stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    # algorithmic bytes: the all-reduce; the norms read y and w_0 (s + 4 per
    # element); the update reads y and reads and writes every replica
    # (s + 8 nrep); the rates read 16 bytes per tile
    norm_b, upd_b = (esz + 4) * w.n, (esz + 8 * nrep) * w.n
    nbytes = ar_bytes + norm_b + upd_b
    plan.set_profiling(True)
    plan.profile_read_kinds()
    one()
    torch.cuda.synchronize()
    kinds = plan.profile_read_kinds()
    plan.destroy()
    res = {"replicas": nrep, "lr": lr, "coeff": ddl.LARS_COEFF, "eps": ddl.LARS_EPS,
           "fused_passes": passes or "auto",
           "layers": len(buckets), "ms": round(ms, 3),
           "hbm_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes": nbytes,
           "over_allreduce_ms": round(ms - fused_ms, 3)}
    for kind, total_b in (("lars_norm", norm_b), ("update", upd_b)):
        tot, cnt, mx = kinds[kind]
        if cnt:
            nb = total_b / cnt
            res[kind + "_kernel"] = {"launches_per_step": cnt,
                                     "avg_launch_us": round(tot / cnt * 1e3, 2),
                                     "max_launch_us": round(mx * 1e3, 2),
                                     "algorithmic_bytes_per_launch": int(nb),
                                     "GBps": round(nb / (tot / cnt * 1e-3) / 1e9, 1)}
    tot, cnt, _ = kinds["lars_rate"]
    if cnt:
        res["lars_rate_kernel"] = {"launches_per_step": cnt,
                                   "avg_launch_us": round(tot / cnt * 1e3, 2)}
    r = rates.cpu()
    res["rate_range"] = [float(r.min()), float(r.max())]
    del weights
    torch.cuda.empty_cache()
    log(f"bench: lars {res}")
    return res


def cpu_baseline(args, w, topo, torch, ddl, synth, np):
    """The CPU oracle as it stands, single-threaded, on the first buckets (in
    issue order) of the same workload; inputs generated on the GPU by the
    same seeded generator and copied to the host.  The GPU result of a fresh
    all-reduce of each sampled bucket is compared with the oracle's."""
    import oracle as orc
    kinds = {"ring": orc.RING, "multiring": orc.MULTIRING, "torus2d": orc.TORUS2D}
    sdt = synth.F32 if w.dtype == "f32" else synth.F16
    tdt = torch.float32 if w.dtype == "f32" else torch.float16
    sample = w.bucket_list()[:max(1, args.cpu_buckets)]
    secs, nbytes, mismatched = 0.0, 0, 0
    for off, cnt in sample:
        dev = [torch.empty(cnt, dtype=tdt, device="cuda") for _ in range(w.P)]
        for r, t in enumerate(dev):
            synth.fill_device(t.data_ptr(), cnt, sdt, w.dist, w.seed, r, first=off,
                              sigma=w.sigma)
        torch.cuda.synchronize()
        host = [t.cpu().numpy() for t in dev]
        plan = ddl.Plan(w.P, cnt, w.dtype, w.op, topo, None, "fused")
        plan.execute(dev)
        torch.cuda.synchronize()
        plan.destroy()
        t0 = time.perf_counter()
        orc.allreduce(host, op=orc.MEAN if w.op == "mean" else orc.SUM, kind=kinds[w.topo],
                      k=w.k, rows=w.rows, cols=w.cols)
        secs += time.perf_counter() - t0
        nbytes += 2 * w.P * cnt * (4 if w.dtype == "f32" else 2)
        got = dev[0].cpu().numpy()
        mismatched += int(np.count_nonzero(got.view(np.uint8) != host[0].view(np.uint8)))
        del dev, host
    log(f"bench: cpu oracle {nbytes / secs / 1e9:.2f} GB/s over {len(sample)} buckets, "
        f"{secs:.1f} s")
    return {"value": round(nbytes / secs / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{len(sample)} of {len(w.bucket_list())} buckets in issue order "
                      f"({w.P} ranks x {sample[0][1]} elements each), single-threaded C, "
                      f"same algorithmic bytes as the GPU figure",
            "seconds": round(secs, 2),
            "host_cpus": os.cpu_count(),
            "host": host_info(),
            "bytes_differing_from_gpu": mismatched}


def host_info():
    """CPU model, usable CPUs and memory of the host the oracle ran on."""
    info = {"usable_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
            else os.cpu_count()}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal"):
                    info["ram_gb"] = round(int(line.split()[1]) / 2**20, 1)
                    break
    except OSError:
        pass
    return info


if __name__ == "__main__":
    main()
