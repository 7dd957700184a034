"""The benchmark's host logic, without a GPU: the roofline figure of the
bench line follows from the committed rocprofv3 summaries (and only while
they were taken on the current kernel sources), and a duration that the
step's wall time contradicts gives no fraction."""
import json
import os
import types

import pytest

import bench
from synth.workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEAD = WORKLOADS["ring_p40_300m_64b"]


def committed(stem):
    with open(os.path.join(ROOT, "profiles", f"{stem}_{HEAD.name}_trace.json")) as f:
        return json.load(f)


def args(mode="fused"):
    return types.SimpleNamespace(mode=mode, prof_stride=8, steps=20)


def kinds(red_us, bc_us, launches=8):
    """profile_read_kinds-shaped figures: (total ms, launches, longest ms)."""
    return {"fused_reduce": (red_us * launches * 1e-3, launches, red_us * 1e-3),
            "broadcast": (bc_us * launches * 1e-3, launches, bc_us * 1e-3)}


def test_roofline_is_the_committed_trace_of_the_current_sources():
    rec = committed("fused_pass")
    if rec["kernel_source_sha256_16"] != bench.kernel_source_hash():
        pytest.skip("the committed trace predates the current kernel sources")
    red = rec["kernels"]["fused_reduce_kernel"]["avg_us"]
    bc = rec["kernels"]["bcast_kernel"]["avg_us"]
    hbm = 2 * HEAD.P * HEAD.n * 4                      # 96 GB per step
    out, per_kernel = bench.roofline_of(args(), HEAD, 2, hbm, ms=17.0, ms_prof=17.1,
                                        kinds=kinds(140.0, 128.0),
                                        per_step={"fused_reduce": 64, "broadcast": 64})
    assert out["source"] == "rocprof"
    # by hand: one pass moves every rank's bucket in and out, 1.5 GB
    per_pass = 2 * HEAD.P * (HEAD.n // 64) * 4
    assert out["algorithmic_bytes_per_unit"] == per_pass
    want = per_pass / ((red + bc) * 1e-6) / 1e9
    assert out["achieved"] == pytest.approx(want, rel=1e-4)
    assert out["frac"] == pytest.approx(want / 8000.0, abs=1e-4)
    # the live figure stands beside it
    assert out["events"]["avg_unit_us"] == pytest.approx(268.0)
    assert set(per_kernel) == {"fused_reduce_kernel", "bcast_kernel"}
    # and the traffic is the committed counters' figure per pass
    assert out["traffic"] == bench.measured_traffic(HEAD.name, "fused", 2)


def test_stale_trace_falls_back_to_events(monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "not-the-sources")
    hbm = 2 * HEAD.P * HEAD.n * 4
    out, _ = bench.roofline_of(args(), HEAD, 2, hbm, ms=17.5, ms_prof=17.6,
                               kinds=kinds(135.0, 125.0),
                               per_step={"fused_reduce": 64, "broadcast": 64})
    assert out["source"] == "events"
    assert out["avg_unit_us"] == pytest.approx(260.0)
    assert out["traffic"] is None             # counters of other sources are not used
    assert out["rocprof"]["source_matches"] is False


def test_contradicted_duration_gives_no_fraction(monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "not-the-sources")
    hbm = 2 * HEAD.P * HEAD.n * 4
    # 64 units of 280 us = 17.9 ms > the 16.7 ms step
    out, _ = bench.roofline_of(args(), HEAD, 2, hbm, ms=16.7, ms_prof=16.8,
                               kinds=kinds(150.0, 130.0),
                               per_step={"fused_reduce": 64, "broadcast": 64})
    assert out["frac"] is None and out["achieved"] is None
    assert "exceeds the step's wall time" in out["withheld"]
    assert out["events"]["fits_step_wall_time"] is False


def test_committed_trace_wall_time_check():
    """A committed duration whose units would exceed the step time is not
    used either: the line then falls back to (or withholds) the events."""
    rec = committed("fused_pass")
    if rec["kernel_source_sha256_16"] != bench.kernel_source_hash():
        pytest.skip("the committed trace predates the current kernel sources")
    hbm = 2 * HEAD.P * HEAD.n * 4
    out, _ = bench.roofline_of(args(), HEAD, 2, hbm, ms=10.0, ms_prof=10.0,
                               kinds=kinds(135.0, 125.0),
                               per_step={"fused_reduce": 64, "broadcast": 64})
    assert out.get("source") != "rocprof" and out["frac"] is None


def test_counted_rates_need_current_counters(monkeypatch):
    got = bench.committed_counted("walk_kernel", HEAD.name)
    rec_path = os.path.join(ROOT, "profiles", f"walk_kernel_{HEAD.name}_traffic.json")
    with open(rec_path) as f:
        rec = json.load(f)
    if rec["kernel_source_sha256_16"] == bench.kernel_source_hash():
        k = rec["kernels"]["walk_kernel"]
        assert got == {"walk_kernel": k["read_bytes_per_launch"] + k["write_bytes_per_launch"]}
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "not-the-sources")
    assert bench.committed_counted("walk_kernel", HEAD.name) is None
    assert bench.measured_traffic(HEAD.name, "fused", 2) is None


def test_more_than_one_gpu_is_refused():
    """One GPU only: --gpus 2 exits with a message before touching torch."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "measures one GPU" in r.stdout
