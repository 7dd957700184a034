#!/usr/bin/env python3
"""Benchmark of the gradient all-reduce on one MI355X.

One step = one all-reduce of the workload (default: 40 virtual ranks of 300M
fp32 gradients each, 48 GB, 64 equal buckets issued last-first, each gated
by its own ready event on the library's side stream), inputs resident in HBM.
Prints one JSON line: achieved HBM GB/s (the algorithmic bytes of the fused
pass, every rank's input read once and its result written once, over the
step time); the roofline of the dominant kernel from the kernels' own
durations in the committed rocprofv3 summary of the same form (taken on the
current sources), with the live figure from HIP events around the launches
of every m-th bucket group of a second run of the timed steps beside it (no
fraction when the kernels' time would exceed the steps' wall time); the CPU
oracle
timed on a bounded sample of the same workload; and side measurements (the
other workloads, step-by-step mode in both forms, small buckets with one
ready event each, overlap with a streaming compute kernel, the SGD and LARS
steps, typed buckets, one GPU's real per-step shape).
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
LEGS = ("configs", "ceilings", "stepwise", "latency", "overlap", "sgd", "lars", "typed", "per_gpu_step")
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
    for name in ("fused_kernel.hip", "step_kernels.hip", "device_common.h", "ddl_internal.h",
                 "plan.cpp", "schedule.cpp"):
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


def committed_counted(stem, workload):
    """{kernel: counted HBM bytes per launch (FETCH_SIZE x 2 + WRITE_SIZE)}
    from the committed counter summary profiles/<stem>_<workload>_traffic.json,
    if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{stem}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return {k: v["read_bytes_per_launch"] + v["write_bytes_per_launch"]
            for k, v in rec.get("kernels", {}).items()}


# committed rocprofv3 kernel-trace summaries: the stem of the file by form of
# the hot path, and the kernels whose average durations add up to one unit
TRACE_FILES = {"fused2": ("fused_pass", ("fused_reduce_kernel", "bcast_kernel")),
               "fused1": ("fused_kernel", ("fused_kernel",)),
               "walk": ("walk_kernel", ("walk_kernel",)),
               "steps": ("step_kernel", ("reduce_step_kernel", "gather_step_kernel"))}


def lib_tuning(knob):
    """A kernel knob's current value (ddl_get_tuning)."""
    import sgd_gradient_all_amd as ddl
    return ddl.get_tuning(knob)


def committed_trace(form, workload, bytes_per_unit):
    """The rocprofv3 average kernel durations of this form and workload from
    the committed summary (profiles/<stem>_<workload>_trace.json), the
    roofline fraction they give, and whether they were taken on the current
    kernel sources."""
    stem, names = TRACE_FILES[form]
    path = os.path.join(ROOT, "profiles", f"{stem}_{workload}_trace.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ks = rec.get("kernels", {})
    if not all(n in ks for n in names):
        return None
    # a pass of the two-kernel form is one launch of each; a step-by-step
    # unit is a launch of either kind, reduce and gather launches alternating
    avg_us = sum(ks[n]["avg_us"] for n in names)
    if form == "steps":
        avg_us /= len(names)
    achieved = bytes_per_unit / (avg_us * 1e-6) / 1e9
    return {"file": os.path.relpath(path.replace("_trace.json", ".md"), ROOT),
            "avg_unit_us": round(avg_us, 2),
            "per_kernel_avg_us": {n: ks[n]["avg_us"] for n in names},
            "achieved": round(achieved, 2), "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "source_matches": rec.get("kernel_source_sha256_16") == kernel_source_hash()}


def roofline_of(args, w, passes, hbm_bytes, ms, ms_prof, kinds, per_step):
    """Roofline of the dominant kernel: the algorithmic bytes of one unit (a
    launch; in the fused pass's two-kernel form a reduce + broadcast pair)
    over its average duration.  The duration is the kernels' own, from the
    committed rocprofv3 summary of this form and workload when it was taken
    on the current sources; the live HIP-event figure of the sampled timed
    region stands beside it (and stands in for it otherwise).  A duration
    whose units per step would exceed the step's wall time gives no
    fraction."""
    kernels = {}
    if args.mode == "fused" and passes == 2:
        form = "fused2"
        red, bc = kinds["fused_reduce"], kinds["broadcast"]
        units = per_step["fused_reduce"]
        sampled = red[1]
        avg_ms = red[0] / red[1] + bc[0] / bc[1]
        kmax = red[2] + bc[2]
        bytes_per_unit = hbm_bytes / units
        rk = bytes_per_unit * (w.P + 1) / (2 * w.P)   # P reads + 1 write
        bk = bytes_per_unit / 2                        # 1 read + P-1 writes
        for name, (tot, cnt, mx), nb in (("fused_reduce_kernel", red, rk),
                                          ("bcast_kernel", bc, bk)):
            kernels[name] = {"launches_per_step": per_step[
                                 "fused_reduce" if name.startswith("fused") else "broadcast"],
                             "sampled_launches": cnt,
                             "avg_launch_us": round(tot / cnt * 1e3, 2),
                             "max_launch_us": round(mx * 1e3, 2),
                             "algorithmic_bytes_per_launch": int(nb),
                             "GBps": round(nb / (tot / cnt * 1e-3) / 1e9, 1)}
        # the reduce kernel walks its tiles rank by rank from 16 ranks on
        # (fused_reduce_ranks_kernel), tile by tile below; both fill the
        # fused_reduce_kernel entries here and in the committed summaries
        red_name = ("fused_reduce_ranks_kernel" if w.P >= lib_tuning("reduce_ranks_min_p")
                    else "fused_reduce_kernel")
        kernel_name = f"fused pass: {red_name} + bcast_kernel"
    else:
        if args.mode == "fused":
            form, keys, kernel_name = "fused1", ("fused",), "fused_kernel"
        elif per_step.get("walk"):
            form, keys, kernel_name = "walk", ("walk",), "walk_kernel"
        else:
            form, keys, kernel_name = "steps", ("reduce", "gather"), "step_kernel"
        units = sum(per_step[k] for k in keys)
        sampled = sum(kinds[k][1] for k in keys)
        avg_ms = sum(kinds[k][0] for k in keys) / max(sampled, 1)
        kmax = max(kinds[k][2] for k in keys)
        bytes_per_unit = hbm_bytes / units
    ev_achieved = bytes_per_unit / (avg_ms * 1e-3) / 1e9
    ev_kernel_ms = units * avg_ms
    ev_ok = ev_kernel_ms <= ms and ev_kernel_ms <= ms_prof
    events = {"avg_unit_us": round(avg_ms * 1e3, 2), "max_unit_us": round(kmax * 1e3, 2),
              "achieved": round(ev_achieved, 2), "frac": round(ev_achieved / PEAK_HBM_GBPS, 4),
              "kernel_ms_per_step": round(ev_kernel_ms, 4), "sampled_units": sampled,
              "profiled_ms_per_step": round(ms_prof, 4), "fits_step_wall_time": ev_ok,
              "timing": f"HIP event pairs around the launches of every {args.prof_stride}-th "
                        f"bucket group, on the stream they run on, over {args.steps} timed "
                        f"steps (each pair also holds its launch's dispatch)"}
    rp = committed_trace(form, w.name, bytes_per_unit)
    out = {"bound": "hbm", "kernel": kernel_name, "achieved": None, "peak": PEAK_HBM_GBPS,
           "unit": "GB/s", "frac": None, "traffic": measured_traffic(w.name, args.mode, passes),
           "units_per_step": units, "algorithmic_bytes_per_unit": int(bytes_per_unit)}
    # the kernels' own durations, from the committed rocprofv3 summary of
    # this form and workload taken on the current sources; else the events
    if rp and rp["source_matches"] and units * rp["avg_unit_us"] * 1e-3 <= ms:
        out.update(achieved=rp["achieved"], frac=rp["frac"], source="rocprof",
                   avg_unit_us=rp["avg_unit_us"])
        rp["event_over_rocprof"] = round(avg_ms * 1e3 / rp["avg_unit_us"], 4)
    elif ev_ok:
        out.update(achieved=events["achieved"], frac=events["frac"], source="events",
                   avg_unit_us=events["avg_unit_us"])
    else:
        out["withheld"] = (f"no committed rocprofv3 summary of the current sources, and "
                           f"{units} units x {avg_ms * 1e3:.2f} us (events) = "
                           f"{ev_kernel_ms:.3f} ms exceeds the step's wall time "
                           f"({ms:.3f} ms)")
    if rp:
        out["rocprof"] = rp
    out["events"] = events
    return out, kernels


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
    ap.add_argument("--step-form", type=int, default=0, choices=[0, 1, 2],
                    help="stepwise mode: 0 the plan's choice, 1 one launch per schedule "
                         "step, 2 the persistent step kernel")
    ap.add_argument("--side-streams", type=int, default=0, choices=[0, 1, 2, 3, 4],
                    help="side streams the headline plan's event-gated groups alternate over "
                         "(0: the plan's choice)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip every side measurement (--legs)")
    ap.add_argument("--legs", default=",".join(LEGS),
                    help="comma-separated side measurements to run, of: " + ", ".join(LEGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-buckets", type=int, default=64,
                    help="buckets of the workload the CPU oracle is timed on")
    ap.add_argument("--prof-stride", type=int, default=8,
                    help="the roofline's HIP events bracket the launches of every m-th "
                         "bucket group of the timed steps (default 8)")
    ap.add_argument("--tune", action="append", default=[], metavar="KNOB=VALUE",
                    help="set a library tuning knob (ddl_set_tuning) before the run, "
                         "e.g. bcast_xcd=8; repeatable")
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

    for kv in args.tune:
        knob, _, val = kv.partition("=")
        ddl.set_tuning(knob, int(val))
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
    del b  # the list alone holds the buffers (the configs leg releases them)
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
    else:
        plan.set_step_form(args.step_form)
    if args.coalesce_bytes:
        plan.set_coalesce_bytes(args.coalesce_bytes)
    plan.set_side_streams(args.side_streams)
    passes = plan.fused_passes()
    _, hbm_bytes = plan.traffic()
    evs = make_events()
    for _ in range(args.warmup):
        record_all(evs)
        plan.execute(bufs, events=evs, stream=main_stream)
    torch.cuda.synchronize()
    # timed region 1: the steps alone -> value, ms_per_step
    ms = run_steps(plan, evs, args.steps)
    value = hbm_bytes / (ms * 1e-3) / 1e9
    # launches per step, counted on one step with every launch bracketed
    plan.set_profiling(1)
    plan.profile_read()
    run_steps(plan, evs, 1)
    per_step = {k: v[1] for k, v in plan.profile_read_kinds().items()}
    # timed region 2: the same steps with HIP event pairs around the launches
    # of every prof_stride-th bucket group, on the stream they run on -> each
    # kernel's average launch duration, with the steps barely slowed
    plan.set_profiling(args.prof_stride)
    plan.profile_read()
    ms_prof = run_steps(plan, evs, args.steps)
    kinds = plan.profile_read_kinds()
    plan.set_profiling(0)
    roofline, kernels = roofline_of(args, w, passes, hbm_bytes, ms, ms_prof, kinds, per_step)
    log(f"bench: {ms:.3f} ms/step, {value:.1f} GB/s; roofline {roofline} {kernels or ''}")
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
                   "fused_passes": passes, "step_form": plan.step_form(),
                   "bytes_per_step": hbm_bytes},
        "pct_of_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "bus_bw_GBps": round(bus_bw, 2),
        "roofline": roofline,
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
        # the in-tree streams of known bytes: nel floats read, then written,
        # then copied (read and written)
        sink = torch.zeros(256, dtype=torch.float32, device="cuda")
        cs = main_stream.cuda_stream
        synth.stream_read(a.data_ptr(), nel, sink.data_ptr(), cs)
        synth.stream_write(b.data_ptr(), nel, 2.0, cs)
        synth.stream_copy(a.data_ptr(), b.data_ptr(), nel, cs)
        torch.cuda.synchronize()
        result["calib_stream_bytes"] = nel * 4
        del sink
        del a, b

    if args.legs:
        result.update(extras(args, w, bufs, topo, buckets, main_stream, torch, ddl, synth,
                             hbm_bytes, ms))

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, w, topo, torch, ddl, synth, np)

    print(json.dumps(result), flush=True)


def extras(args, w, bufs, topo, buckets, main_stream, torch, ddl, synth, fused_bytes, fused_ms):
    out = {}
    # the other workloads first, before the large legs below have churned
    # HBM, and with the headline's buffers released for the time (the rate
    # of a pass depends somewhat on the physical pages behind its buffers);
    # the headline's buffers are then made again with the same inputs
    if "configs" in args.legs:
        nbufs = len(bufs)
        bufs.clear()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        out["configs"] = configs_leg(w, main_stream, torch, ddl, synth)
        tdt = torch.float32 if w.dtype == "f32" else torch.float16
        sdt = synth.F32 if w.dtype == "f32" else synth.F16
        bufs.extend(torch.empty(w.n, dtype=tdt, device="cuda") for _ in range(nbufs))
        for r, b in enumerate(bufs):
            synth.fill_device(b.data_ptr(), w.n, sdt, w.dist, w.seed, r, sigma=w.sigma)
        torch.cuda.synchronize()
    if "ceilings" in args.legs:
        out["hbm_ceilings"] = ceilings_leg(main_stream, torch, synth)
        copy = out["hbm_ceilings"]["copy"]["GBps"]
        # each pass moves as many bytes in as out, as a copy does
        rel = {w.name: round(fused_bytes / (fused_ms * 1e-3) / 1e9 / copy, 3)}
        for name, row in out.get("configs", {}).items():
            if not row["cache_resident"]:
                rel[name] = round(row["hbm_GBps"] / copy, 3)
        out["hbm_ceilings"]["fused_pass_over_copy"] = rel
    if "stepwise" in args.legs:
        out["stepwise"] = stepwise_leg(w, bufs, topo, buckets, main_stream, torch, ddl,
                                       fused_bytes)
    if "latency" in args.legs:
        out["latency"] = latency_leg(main_stream, torch, ddl, synth)
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
    if "per_gpu_step" in args.legs:
        out["per_gpu_step"] = per_gpu_step_leg(w, main_stream, torch, ddl)
    return out


def configs_leg(head, main_stream, torch, ddl, synth, allocations=3):
    """The other workloads, each in its plan's default fused form on fresh
    inputs: ms per all-reduce and HBM GB/s over its algorithmic bytes (the
    4-rank 2^20 case fits the caches, so its figure is not an HBM one).  Each
    workload runs on `allocations` successive fresh allocations of its
    buffers (the rate depends somewhat on the physical pages behind them);
    the reported figure is their median, every allocation's is listed.  On
    the first allocation the stepwise mode is timed too, in both forms (the
    persistent step kernel, and one launch per schedule step), over the
    schedule's step bytes."""
    from synth.workloads import WORKLOADS
    out = {}
    for name, w in WORKLOADS.items():
        if name == head.name:
            continue
        tdt = torch.float32 if w.dtype == "f32" else torch.float16
        sdt = synth.F32 if w.dtype == "f32" else synth.F16
        runs = []
        for _ in range(allocations):
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
                t0 = torch.cuda.Event(enable_timing=True)
                t1 = torch.cuda.Event(enable_timing=True)
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
            runs.append(run(reps))
            passes = plan.fused_passes()
            plan.destroy()
            if len(runs) == 1:
                # the stepwise mode on the first allocation, in both forms
                stepwise = {}
                for form, label in ((2, "persistent"), (1, "per_step_launches")):
                    plan = ddl.Plan(w.P, w.n, w.dtype, w.op,
                                    ddl.topo(w.topo, w.k, w.rows, w.cols), buckets, "stepwise")
                    plan.set_step_form(form)
                    _, sbytes = plan.traffic()
                    run(1)
                    sms = run(max(3, reps // 5))
                    stepwise[label] = {"ms": round(sms, 4),
                                       "step_bytes_GBps": round(sbytes / (sms * 1e-3) / 1e9, 1)}
                    plan.destroy()
            del bufs
            torch.cuda.empty_cache()
        ms = sorted(runs)[len(runs) // 2]
        gbps = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 4), "hbm_GBps": round(gbps, 1),
                     "pct_of_peak": round(100 * gbps / PEAK_HBM_GBPS, 2),
                     "ms_per_allocation": [round(x, 4) for x in runs],
                     "fused_passes": passes, "bytes": nbytes,
                     "cache_resident": nbytes < (256 << 20), "stepwise": stepwise}
    log(f"bench: configs {out}")
    return out


def ceilings_leg(main_stream, torch, synth, nbytes=1_200_000_000, reps=7):
    """The rates plain streams reach on this device (in-tree kernels of
    known bytes, non-temporal 16-byte accesses, one 4 KB tile per
    workgroup): a copy of nbytes (nbytes read and nbytes written), a read
    and a write.  The fused pass reads and writes the same number of bytes,
    as a copy does, so the copy's rate is the one to hold it against."""
    n = nbytes // 4
    a = torch.empty(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    sink = torch.zeros(256, dtype=torch.float32, device="cuda")
    cs = main_stream.cuda_stream
    synth.stream_write(a.data_ptr(), n, 1.0, cs)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, moved):
        fn()
        times = []
        for _ in range(reps):
            t0.record(main_stream)
            fn()
            t1.record(main_stream)
            torch.cuda.synchronize()
            times.append(t0.elapsed_time(t1))
        ms = sorted(times)[reps // 2]
        gbps = moved / (ms * 1e-3) / 1e9
        return {"ms": round(ms, 4), "GBps": round(gbps, 1),
                "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4)}

    out = {"bytes_per_stream": n * 4,
           "copy": timed(lambda: synth.stream_copy(a.data_ptr(), b.data_ptr(), n, cs), 8 * n),
           "read": timed(lambda: synth.stream_read(a.data_ptr(), n, sink.data_ptr(), cs), 4 * n),
           "write": timed(lambda: synth.stream_write(b.data_ptr(), n, 2.0, cs), 4 * n)}
    del a, b, sink
    torch.cuda.empty_cache()
    log(f"bench: ceilings {out}")
    return out


def stepwise_leg(w, bufs, topo, buckets, main_stream, torch, ddl, fused_bytes):
    """The step-by-step schedule on the same buffers, in both forms: one
    kernel launch per schedule step (the per-GPU step kernels) and the
    persistent step kernel (one launch per group, each workgroup walking
    every step of its tile).  Each is timed without per-launch events; the
    per-step form is also replayed from a HIP graph; one profiled step of
    each (one side stream, so launches do not overlap) gives the kernel-side
    figures: each kernel's average launch against its algorithmic bytes."""
    plan = ddl.Plan(w.P, w.n, w.dtype, w.op, topo, buckets, "stepwise")
    _, sbytes = plan.traffic()
    evs = [torch.cuda.Event() for _ in buckets] if w.side_stream else None
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def step_once():
        if evs:
            for e in evs:
                e.record(main_stream)
        plan.execute(bufs, events=evs, stream=main_stream)

    def timed(steps):
        t0.record(main_stream)
        for _ in range(steps):
            step_once()
        t1.record(main_stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    res = {"bytes_per_step": sbytes, "default_form": plan.step_form()}
    for form, label in ((1, "per_step_launches"), (2, "persistent")):
        plan.set_step_form(form)
        step_once()
        torch.cuda.synchronize()
        sms = timed(3)
        # the schedule's step bytes over the step time; the persistent form
        # re-reads a tile's step outputs from the caches, so its step-byte
        # rate can exceed what HBM moves: the counted bytes (committed
        # counter summary of the same kernels) give the HBM rate
        row = {"ms_per_step": round(sms, 3),
               "step_bytes_GBps": round(sbytes / (sms * 1e-3) / 1e9, 1),
               "step_bytes_pct_of_peak": round(100 * sbytes / (sms * 1e-3) / 1e9 /
                                               PEAK_HBM_GBPS, 2),
               "fused_floor_equiv_GBps": round(fused_bytes / (sms * 1e-3) / 1e9, 1)}
        if form == 1:
            # captured once into a HIP graph and replayed: the thousands of
            # step launches are then issued by one graph launch
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
            for _ in range(3):
                graph.replay()
            t1.record(main_stream)
            torch.cuda.synchronize()
            row["graph_ms_per_step"] = round(t0.elapsed_time(t1) / 3, 3)
            del graph
            torch.cuda.synchronize()
        # kernel-side figures: one profiled step on a single side stream
        plan.set_side_streams(1)
        plan.set_profiling(1)
        step_once()
        torch.cuda.synchronize()
        kinds = plan.profile_read_kinds()
        plan.set_profiling(0)
        plan.set_side_streams(0)
        row["launches_per_step"] = sum(v[1] for v in kinds.values())
        counted = committed_counted("step_kernel" if form == 1 else "walk_kernel", w.name)
        if counted:
            per_kind = (("reduce", "reduce_step_kernel"), ("gather", "gather_step_kernel")) \
                if form == 1 else (("walk", "walk_kernel"),)
            hbm = sum(kinds[k][1] * counted[name] for k, name in per_kind if name in counted)
            row["counted_hbm_GBps"] = round(hbm / (sms * 1e-3) / 1e9, 1)
            row["counted_pct_of_peak"] = round(100 * hbm / (sms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2)
        shares = (("reduce", 3), ("gather", 2)) if form == 1 else (("walk", 5),)
        for kind, share in shares:
            tot, cnt, mx = kinds[kind]
            if cnt:
                nb = share * sbytes / 5 / cnt   # the step bytes split 3 : 2
                name = "walk_kernel" if kind == "walk" else kind + "_step_kernel"
                row[name] = {
                    "launches_per_step": cnt, "avg_launch_us": round(tot / cnt * 1e3, 2),
                    "max_launch_us": round(mx * 1e3, 2),
                    "algorithmic_bytes_per_launch": int(nb),
                    "GBps": round(nb / (tot / cnt * 1e-3) / 1e9, 1)}
        res[label] = row
    plan.destroy()
    log(f"bench: stepwise {res}")
    return res


def latency_leg(main_stream, torch, ddl, synth, calls=4):
    """Small buckets (IBM's latency/bandwidth trade-off): the ResNet-50
    gradient over 16 ranks and 4 rings, binary32, each of its 161 tensors its
    own bucket with its own ready event, recorded in list order on the
    caller's stream as back-propagation would record them, output layer
    first.  For the fused pass and both step forms, at grouping thresholds 0
    and 16 MB (with and without the ordered-events promise):
      - device_ms: device time of one call with the host ahead of the device
        (a streaming kernel on the caller's stream holds the device while the
        call is enqueued): from the end of that kernel, through the caller's
        161 event records, to the end of the all-reduce;
      - after_events_ms: the same call from the moment the last ready event
        has been recorded (every gradient ready) to the end of the
        all-reduce -- what back-propagation would be left waiting for;
      - graph_ms: the call, event records included, captured once into a HIP
        graph and replayed back to back (the records become graph edges);
      - eager_ms: back-to-back eager calls, event records included (host-
        bound when the host is slower than the device);
      - host_ms: the host time of the library call itself.
    Against the same all-reduce with no events (one group).  The
    `..._group_events` variants record one event per group that
    ddl_plan_event_groups reports (after the group's last tensor) and pass it
    for each of the group's tensors: the same groups and launches, with one
    record per group instead of one per tensor.  The `..._nofence`
    variants record the per-tensor events as the binding's ReadyEvent makes
    them, without the system-scope fence of a default record."""
    from synth.workloads import WORKLOADS
    w = WORKLOADS["multiring_k4_p16_resnet50"]
    bufs = [torch.empty(w.n, dtype=torch.float32, device="cuda") for _ in range(w.P)]
    for r, b in enumerate(bufs):
        synth.fill_device(b.data_ptr(), w.n, synth.F32, w.dist, w.seed, r, sigma=w.sigma)
    buckets = w.bucket_list()
    topo = ddl.topo(w.topo, w.k, w.rows, w.cols)
    events = [torch.cuda.Event() for _ in buckets]
    nofence_events = [ddl.ReadyEvent() for _ in buckets]
    gate = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
    cs = main_stream.cuda_stream
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    tm = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()

    def hold(n):
        for _ in range(n):
            synth.stream_compute(gate.data_ptr(), gate.numel(), 1.0, 0.0, cs)

    t0.record(main_stream)
    hold(4)
    t1.record(main_stream)
    torch.cuda.synchronize()
    hold_ms = t0.elapsed_time(t1) / 4

    # the events recorded (in list order) and those passed, one per bucket
    rec, passed = events, events

    def record_events(stream):
        for e in rec:
            e.record(stream)

    def run(plan, gated):
        if gated:
            record_events(main_stream)
        plan.execute(bufs, events=passed if gated else None, stream=main_stream)

    def measure(plan, gated, graph_too):
        run(plan, gated)
        torch.cuda.synchronize()
        # the library's own host time per call
        host = []
        for _ in range(calls):
            if gated:
                record_events(main_stream)
            h0 = time.perf_counter()
            plan.execute(bufs, events=passed if gated else None, stream=main_stream)
            host.append(time.perf_counter() - h0)
        torch.cuda.synchronize()
        host_ms = sorted(host)[len(host) // 2] * 1e3
        # back to back
        t0.record(main_stream)
        for _ in range(calls):
            run(plan, gated)
        t1.record(main_stream)
        torch.cuda.synchronize()
        eager = t0.elapsed_time(t1) / calls
        # one call at a time behind a streaming kernel that covers its host
        # time: device time from the kernel's end, and from the last record
        nhold = int((eager * 1.5 + 1.0) / max(hold_ms, 1e-3)) + 1
        dev, after, ahead = [], [], True
        for _ in range(calls):
            hold(nhold)
            h0 = time.perf_counter()
            t0.record(main_stream)
            if gated:
                record_events(main_stream)
            tm.record(main_stream)
            plan.execute(bufs, events=passed if gated else None, stream=main_stream)
            t1.record(main_stream)
            ahead = ahead and (time.perf_counter() - h0) * 1e3 < nhold * hold_ms
            torch.cuda.synchronize()
            dev.append(t0.elapsed_time(t1))
            after.append(tm.elapsed_time(t1))
        row = {"device_ms": round(sum(dev) / calls, 4),
               "after_events_ms": round(sum(after) / calls, 4),
               "eager_ms": round(eager, 4), "host_ms": round(host_ms, 4),
               "host_ahead": bool(ahead)}
        if graph_too:
            graph = torch.cuda.CUDAGraph()
            cap = torch.cuda.Stream()
            cap.wait_stream(main_stream)
            with torch.cuda.stream(cap):
                with torch.cuda.graph(graph, stream=cap):
                    if gated:
                        record_events(cap)
                    plan.execute(bufs, events=passed if gated else None, stream=cap)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            t0.record(main_stream)
            for _ in range(calls):
                graph.replay()
            t1.record(main_stream)
            torch.cuda.synchronize()
            row["graph_ms"] = round(t0.elapsed_time(t1) / calls, 4)
            del graph
            torch.cuda.synchronize()
        return row

    res = {"workload": w.name, "ranks": w.P, "tensors": len(buckets), "events": len(buckets),
           "hold_kernel_ms": round(hold_ms, 3)}
    plan = ddl.Plan(w.P, w.n, w.dtype, w.op, topo, buckets, "fused")
    res["no_events_fused"] = measure(plan, False, True)
    plan.destroy()
    variants = [("fused", 0, 0, False, False, False), ("fused", 0, 16, False, False, False),
                ("fused", 0, 16, True, False, False), ("fused", 0, 16, True, True, False),
                ("fused", 0, 16, True, False, True),
                ("stepwise", 2, 0, False, False, False), ("stepwise", 2, 16, True, False, False),
                ("stepwise", 2, 16, True, True, False), ("stepwise", 2, 16, True, False, True),
                ("stepwise", 1, 0, False, False, False), ("stepwise", 1, 16, True, False, False)]
    for mode, form, thr_mb, ordered, grouped, nofence in variants:
        plan = ddl.Plan(w.P, w.n, w.dtype, w.op, topo, buckets, mode)
        if mode == "stepwise":
            plan.set_step_form(form)
        plan.set_coalesce_bytes(thr_mb << 20)
        # the events are recorded in list order on one stream, as
        # back-propagation records them: the promise may be made
        plan.set_ordered_events(ordered)
        if grouped:
            last = plan.event_groups()
            rec = [torch.cuda.Event() for _ in last]
            passed = [rec[sum(1 for x in last if x < b)] for b in range(len(buckets))]
        elif nofence:
            rec, passed = nofence_events, nofence_events
        else:
            rec, passed = events, events
        plan.set_profiling(1)
        run(plan, True)
        torch.cuda.synchronize()
        launches = sum(v[1] for v in plan.profile_read_kinds().values())
        plan.set_profiling(0)
        key = (f"{mode}{'' if mode == 'fused' else '_form%d' % form}_coalesce_{thr_mb}mb"
               f"{'_ordered' if ordered else ''}{'_group_events' if grouped else ''}"
               f"{'_nofence' if nofence else ''}")
        row = measure(plan, True, True)
        row["launches"] = launches
        row["events_recorded"] = len(rec)
        res[key] = row
        # captured plans must outlive the graph, which is gone by now
        plan.destroy()
    base = res["no_events_fused"]
    res["fused_event_gated_over_no_events"] = {
        k: {m: round(res[k][m] / base[m], 3) for m in ("device_ms", "graph_ms")}
        for k in ("fused_coalesce_0mb", "fused_coalesce_16mb", "fused_coalesce_16mb_ordered",
                  "fused_coalesce_16mb_ordered_nofence",
                  "fused_coalesce_16mb_ordered_group_events")}
    del bufs, gate, nofence_events
    torch.cuda.empty_cache()
    log(f"bench: latency {res}")
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
    plan.set_step_form(1)   # the per-step kernels, one launch per step
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
        # the stepwise figure is over the schedule's step bytes, which the
        # persistent form partly re-reads from the caches
        key = "hbm_GBps" if mode == "fused" else "step_bytes_GBps"
        res[mode] = {"ms": round(ms, 4), key: round(hbm / (ms * 1e-3) / 1e9, 1), "bytes": hbm}
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
