"""Host-side checks of libddl.so (no GPU calls).

- the library loads and exports every function include/ddl.h declares;
- argument validation returns the documented codes;
- the schedule generator's tables, replayed on the host by a small table
  interpreter written here, reproduce the oracle bit for bit (step tables and
  fused chains), and move the traffic the oracle counts.
"""
import os
import re
import subprocess

import numpy as np
import pytest

import oracle as orc
import sgd_gradient_all_amd as ddl
from sgd_gradient_all_amd import _ddl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    with open(os.path.join(ROOT, "include", "ddl.h")) as f:
        text = f.read()
    declared = set(re.findall(r"^\s*(?:int|const char \*)\s*(ddl_\w+)\s*\(", text, re.M))
    assert {"ddl_plan_create", "ddl_plan_execute", "ddl_allreduce", "ddl_plan_traffic",
            "ddl_plan_destroy", "ddl_strerror"} <= declared
    out = subprocess.run(["nm", "-D", "--defined-only", _ddl._LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ddl_\w+)", out))
    assert declared <= exported, declared - exported
    lib = ddl.lib()
    for name in declared:
        assert hasattr(lib, name)


def test_strerror_covers_every_code():
    for code in range(0, -11, -1):
        assert ddl.ddl_strerror(code) != "unknown error"
    assert ddl.ddl_strerror(-99) == "unknown error"


def _create_rc(P, n, dtype=0, op=0, kind=0, k=1, rows=0, cols=0, order=None, buckets=None,
               mode=1):
    import ctypes
    t = _ddl.topo(kind, k, rows, cols, order)
    barr, nb = _ddl._buckets(buckets)
    h = ctypes.c_void_p()
    rc = ddl.lib().ddl_plan_create(ctypes.byref(h), P, n, dtype, op, ctypes.byref(t), barr, nb,
                                   mode)
    if rc == 0:
        ddl.lib().ddl_plan_destroy(h)
    return rc


def test_stale_and_foreign_handles_are_argument_errors():
    """Every entry point looks its handle up among the live plans first: a
    second destroy, a call on a destroyed plan and a pointer that never was
    a plan return DDL_E_ARG instead of touching freed memory (no GPU is
    needed: each fails before any device work)."""
    import ctypes
    L = ddl.lib()
    plan = ddl.Plan(4, 1000, "f32", "sum", ddl.topo("ring"))
    h = plan.handle
    assert L.ddl_plan_destroy(h) == 0
    plan.handle = None
    bufs = (ctypes.c_void_p * 4)(*[256 * (r + 1) for r in range(4)])
    n = ctypes.c_int()
    hbm = ctypes.c_size_t()
    assert L.ddl_plan_destroy(h) == -2
    assert L.ddl_plan_execute(h, bufs, None, None, None) == -2
    assert L.ddl_plan_execute_sgd(h, bufs, bufs, 4, 0.1, 1, None, None, None) == -2
    assert L.ddl_plan_execute_lars(h, bufs, bufs, 4, 0.1, 0.01, 1e-6, None, None, None,
                                   None) == -2
    assert L.ddl_plan_traffic(h, None, ctypes.byref(hbm)) == -2
    assert L.ddl_plan_num_steps(h, ctypes.byref(n)) == -2
    assert L.ddl_plan_set_coalesce_bytes(h, 1) == -2
    assert L.ddl_plan_set_profiling(h, 1) == -2
    junk = (ctypes.c_char * 512)()
    foreign = ctypes.cast(junk, ctypes.c_void_p)
    assert L.ddl_plan_destroy(foreign) == -2
    assert L.ddl_plan_execute(foreign, bufs, None, None, None) == -2
    assert L.ddl_plan_destroy(None) == -1


def test_noalloc_lars_rejections_need_no_device():
    """The allocation-free LARS entry point rejects, before any device work,
    a plan too large for its fixed scratch (DDL_E_SCRATCH) and a plan that
    has not yet run on the device (DDL_E_UNBOUND); typed plans are
    argument errors as for the allocating entry point."""
    big = ddl.Plan(2, (1 << 29) + 4096, "f32", "mean", ddl.topo("ring"))
    with pytest.raises(ddl.DDLError) as ei:
        big.execute_lars_noalloc([0x1000, 0x2000], [0x3000], 0.1)
    assert ei.value.code == -10
    big.destroy()
    many = ddl.Plan(2, 70_000, "f32", "mean", ddl.topo("ring"), [(i, 1) for i in range(70_000)])
    with pytest.raises(ddl.DDLError) as ei:
        many.execute_lars_noalloc([0x1000, 0x2000], [0x3000], 0.1)
    assert ei.value.code == -10
    many.destroy()
    fits = ddl.Plan(4, (1 << 29) - 8192, "f32", "mean", ddl.topo("ring"))
    with pytest.raises(ddl.DDLError) as ei:
        fits.execute_lars_noalloc([0x1000 * (r + 1) for r in range(4)], [0x9000], 0.1)
    assert ei.value.code == -9
    fits.destroy()
    typed = ddl.Plan.typed(2, 64, "mean", ddl.topo("ring"), [(0, 16, "f32")])
    with pytest.raises(ddl.DDLError) as ei:
        typed.execute_lars_noalloc([0x1000, 0x2000], [0x3000], 0.1)
    assert ei.value.code == -2
    typed.destroy()


def test_argument_validation():
    assert _create_rc(4, 100) == 0
    assert _create_rc(0, 100) == -2
    assert _create_rc(129, 100) == -2
    assert _create_rc(4, 100, dtype=7) == -2
    assert _create_rc(4, 100, op=3) == -2
    assert _create_rc(4, 100, mode=5) == -2
    assert _create_rc(4, 100, kind=2, rows=3, cols=2) == -2
    assert _create_rc(4, 100, kind=2, rows=2, cols=2, order=[0, 1, 2, 3]) == -2
    assert _create_rc(4, 100, kind=1, k=0) == -2
    assert _create_rc(4, 100, order=[0, 1, 1, 3]) == -2
    assert _create_rc(4, 100, order=[0, 1, 2, 4]) == -2
    assert _create_rc(4, 100, buckets=[(0, 50), (40, 60)]) == -3
    assert _create_rc(4, 100, buckets=[(0, 50), (60, 40)]) == -3
    assert _create_rc(4, 100, buckets=[(0, 50), (50, 60)]) == -3
    assert _create_rc(4, 100, buckets=[(50, 50), (0, 50), (10, 0)]) == 0
    assert _create_rc(4, 0) == 0
    assert _create_rc(128, 10) == 0


# ---------------------------------------------------------------------------
# a table interpreter: replays the plan's tables on host arrays with numpy
# arithmetic (binary32 add / divide; binary16 through binary32, rounded)
# ---------------------------------------------------------------------------
def _add(a, b, dtype):
    if dtype == np.float32:
        return a + b
    return (a.astype(np.float32) + b.astype(np.float32)).astype(np.float16)


def _div(a, P, dtype):
    if dtype == np.float32:
        return a / np.float32(P)
    return (a.astype(np.float32) / np.float32(P)).astype(np.float16)


def interpret_steps(plan, bufs, nbuckets, dtype, which=None):
    steps = plan.num_steps()
    for b in (range(nbuckets) if which is None else which):
        for s in range(steps):
            kind = plan.step_kind(s)
            items = plan.step_items(s, b)
            # all items of a step read before any writes land (they are
            # race-free, this keeps the replay honest either way)
            staged = [(src, dst, div, off, cnt, bufs[src][off:off + cnt].copy())
                      for src, dst, div, off, cnt in items]
            for src, dst, div, off, cnt, data in staged:
                if kind == ddl.DDL_K_REDUCE:
                    r = _add(bufs[dst][off:off + cnt], data, dtype)
                    if div:
                        r = _div(r, len(bufs), dtype)
                    bufs[dst][off:off + cnt] = r
                else:
                    bufs[dst][off:off + cnt] = data


def interpret_fused(plan, bufs, nbuckets, dtype, mean, which=None):
    P = len(bufs)
    for b in (range(nbuckets) if which is None else which):
        spans, group = plan.fused_spans(b)
        for off, cnt, chain in spans:
            acc = None
            for g in range(0, P, group):
                gacc = bufs[chain[g]][off:off + cnt].copy()
                for r in chain[g + 1:g + group]:
                    gacc = _add(gacc, bufs[r][off:off + cnt], dtype)
                acc = gacc if acc is None else _add(acc, gacc, dtype)
            if mean:
                acc = _div(acc, P, dtype)
            for r in range(P):
                bufs[r][off:off + cnt] = acc


def interpret_walk(plan, bufs, nbuckets, dtype, mean, which=None):
    """The persistent step kernel's rule, on host arrays: every fused span
    (chain c in groups of C) goes through the row reduce-scatter of each
    group, the reduce-scatter and all-gather over the groups' last entries,
    and the row all-gather of each group, each step reading and writing the
    ranks' arrays.  Returns the element accesses made (reads + writes)."""
    P = len(bufs)
    moved = 0
    for b in (range(nbuckets) if which is None else which):
        spans, C = plan.fused_spans(b)
        G = P // C
        for off, cnt, c in spans:
            sl = slice(off, off + cnt)

            def reduce(src, dst, last):
                r = _add(bufs[c[dst]][sl], bufs[c[src]][sl], dtype)
                bufs[c[dst]][sl] = _div(r, P, dtype) if last else r
                return 3 * cnt

            def copy(src, dst):
                bufs[c[dst]][sl] = bufs[c[src]][sl]
                return 2 * cnt

            for g in range(G):
                for t in range(C - 1):
                    moved += reduce(g * C + t, g * C + t + 1, mean and G == 1 and t == C - 2)
            for t in range(G - 1):
                moved += reduce(t * C + C - 1, (t + 1) * C + C - 1, mean and t == G - 2)
            for t in range(G - 1):
                moved += copy(((t - 1) % G) * C + C - 1, t * C + C - 1)
            for g in range(G):
                for t in range(C - 1):
                    moved += copy(g * C + (t - 1) % C, g * C + t)
    return moved


def _cases():
    rng = np.random.default_rng(21)
    cases = []
    for P in (1, 2, 3, 4, 5, 8, 12, 16):
        for kind in ("ring", "multiring", "torus2d"):
            for dtype in (np.float32, np.float16):
                n = int(rng.integers(1, 400))
                k, rows, cols, order = 1, 0, 0, None
                if kind == "multiring":
                    k = int(rng.integers(1, 5))
                    order = np.concatenate([rng.permutation(P) for _ in range(k)]).tolist()
                elif kind == "torus2d":
                    divs = [d for d in range(1, P + 1) if P % d == 0]
                    rows = int(rng.choice(divs))
                    cols = P // rows
                elif rng.random() < 0.5:
                    order = rng.permutation(P).tolist()
                nb = int(rng.integers(1, 4))
                cuts = sorted(set(int(c) for c in rng.integers(0, n, nb - 1))) if nb > 1 else []
                edges = [0] + cuts + [n]
                buckets = [(edges[i], edges[i + 1] - edges[i]) for i in range(len(edges) - 1)]
                buckets = buckets[::-1]
                cases.append((P, n, kind, k, rows, cols, order, dtype, buckets))
    return cases


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"P{c[0]}-n{c[1]}-{c[2]}-{c[7].__name__}")
@pytest.mark.parametrize("op", ["sum", "mean"])
def test_tables_replay_to_the_oracle(case, op):
    P, n, kind, k, rows, cols, order, dtype, buckets = case
    rng = np.random.default_rng(P * 1000 + n)
    g = [rng.standard_normal(n).astype(dtype) for _ in range(P)]
    kinds = {"ring": orc.RING, "multiring": orc.MULTIRING, "torus2d": orc.TORUS2D}
    ref = [x.copy() for x in g]
    sent_ref = orc.allreduce(ref, op=orc.MEAN if op == "mean" else orc.SUM, kind=kinds[kind],
                             k=k, rows=rows, cols=cols, ring_order=order, buckets=buckets)
    t = ddl.topo(kind, k, rows, cols, order)
    dt = "f32" if dtype == np.float32 else "f16"
    for mode in ("stepwise", "fused", "walk"):
        plan = ddl.Plan(P, n, dt, op, t, buckets, "stepwise" if mode == "walk" else mode)
        bufs = [x.copy() for x in g]
        if mode == "stepwise":
            interpret_steps(plan, bufs, len(buckets), dtype)
        elif mode == "walk":
            # the persistent step kernel's rule moves the stepwise bytes
            moved = interpret_walk(plan, bufs, len(buckets), dtype, op == "mean")
            assert moved == 5 * (P - 1) * n
        else:
            interpret_fused(plan, bufs, len(buckets), dtype, op == "mean")
        for r in range(P):
            assert bufs[r].tobytes() == ref[r].tobytes(), (mode, r)
        sent, hbm = plan.traffic()
        assert sent == [int(v) for v in sent_ref]
        esz = np.dtype(dtype).itemsize
        if mode == "fused":
            assert hbm == 2 * P * n * esz
        else:
            assert hbm == 5 * (P - 1) * n * esz
        plan.destroy()


def test_typed_tables_replay_to_the_oracle():
    """A plan with typed buckets: each bucket's tables, replayed on the
    dtype's view of the byte buffers, give the oracle's walk of that bucket
    alone (binary32 and binary16 buckets interleaved, ragged)."""
    rng = np.random.default_rng(5)
    for P, kind, k, rows, cols in ((5, "ring", 1, 0, 0), (8, "multiring", 3, 0, 0),
                                   (6, "torus2d", 1, 2, 3)):
        layout, at = [], 0
        for _ in range(7):
            dt = "f16" if rng.random() < 0.5 else "f32"
            esz = 4 if dt == "f32" else 2
            if at % esz:
                off, cnt, pdt = layout[-1]
                layout[-1] = (off, cnt + 1, pdt)
                at += 2
            cnt = int(rng.integers(1, 300))
            layout.append((at, cnt, dt))
            at += cnt * esz
        layout = layout[::-1]
        nbytes = at
        pad = (nbytes + 3) // 4 * 4
        g = [rng.integers(0, 256, pad, dtype=np.uint8) for _ in range(P)]
        # finite values: random bytes can make NaNs, whose payloads may differ
        for off, cnt, dt in layout:
            npdt = np.float32 if dt == "f32" else np.float16
            for r in range(P):
                g[r][off:off + cnt * np.dtype(npdt).itemsize] = \
                    rng.standard_normal(cnt).astype(npdt).view(np.uint8)
        t = ddl.topo(kind, k, rows, cols)
        for mode in ("stepwise", "fused"):
            plan = ddl.Plan.typed(P, nbytes, "mean", t, layout, mode)
            bufs = [x.copy() for x in g]
            for b, (off, cnt, dt) in enumerate(layout):
                npdt = np.float32 if dt == "f32" else np.float16
                views = [x[:pad // np.dtype(npdt).itemsize * np.dtype(npdt).itemsize]
                         .view(npdt) for x in bufs]
                if mode == "stepwise":
                    interpret_steps(plan, views, len(layout), npdt, which=[b])
                else:
                    interpret_fused(plan, views, len(layout), npdt, True, which=[b])
            plan.destroy()
            for off, cnt, dt in layout:
                npdt = np.float32 if dt == "f32" else np.float16
                nb = cnt * np.dtype(npdt).itemsize
                seg = [x[off:off + nb].view(npdt).copy() for x in g]
                kinds = {"ring": orc.RING, "multiring": orc.MULTIRING, "torus2d": orc.TORUS2D}
                orc.allreduce(seg, op=orc.MEAN, kind=kinds[kind], k=k, rows=rows, cols=cols)
                for r in range(P):
                    assert bufs[r][off:off + nb].tobytes() == seg[r].view(np.uint8).tobytes(), \
                        (kind, mode, off, dt, r)


def test_step_counts_and_kinds():
    for P, kind, rows, cols, want in ((8, "ring", 0, 0, 14), (16, "multiring", 0, 0, 30),
                                      (16, "torus2d", 4, 4, 12), (6, "torus2d", 2, 3, 6),
                                      (1, "ring", 0, 0, 0)):
        plan = ddl.Plan(P, 1000, "f32", "mean", ddl.topo(kind, 4, rows, cols))
        assert plan.num_steps() == want
        kinds = [plan.step_kind(s) for s in range(want)]
        assert kinds == [ddl.DDL_K_REDUCE] * (want // 2) + [ddl.DDL_K_GATHER] * (want // 2)
        plan.destroy()


def test_headline_table_sizes():
    # 40 ranks, 64 buckets of 4,687,500 fp32: 78 steps of 40 pairs each per
    # bucket, 40 fused spans per bucket with chunks of 117,184 or 117,188
    n = 300_000_000
    buckets = [(i * 4_687_500, 4_687_500) for i in reversed(range(64))]
    plan = ddl.Plan(40, n, "f32", "mean", ddl.topo("ring"), buckets, "fused")
    assert plan.num_steps() == 78
    assert len(plan.step_items(0, 0)) == 40
    spans, group = plan.fused_spans(0)
    assert len(spans) == 40 and group == 40
    assert {c for _, c, _ in spans} == {117_184, 117_188}
    assert spans[0][0] == 63 * 4_687_500
    sent, hbm = plan.traffic()
    # 40 * 4 does not divide 4,687,500, so chunks differ by 4 elements: the
    # total is exact, each rank is within 2 chunk-size steps per bucket of
    # the even share 2 (P-1)/P n
    assert sum(sent) == 2 * 39 * n
    assert all(abs(s - 2 * 39 * n // 40) <= 64 * 2 * 4 for s in sent)
    assert hbm == 2 * 40 * n * 4
    plan.destroy()


def test_plan_create_needs_no_gpu():
    # plan creation and inspection are host-only; no HIP call is made
    plan = ddl.Plan(16, 25_557_032, "f16", "mean", ddl.topo("torus2d", rows=4, cols=4))
    spans, group = plan.fused_spans(0)
    assert group == 4 and len(spans) == 16
    plan.destroy()


def test_fused_pass_form_setting():
    # host-only: the automatic form is two kernels from 16 ranks on for
    # groups of at least 200 MB over all ranks (400 MB for binary16), one
    # kernel otherwise (fused plans only); explicit 1 and 2 stick; anything
    # else is rejected.  Thresholds: 16 ranks binary32 3,276,800 elements per
    # rank, 40 ranks 1,310,720, 16 ranks binary16 13,107,200.
    big32, big16 = 200 << 20, 400 << 20
    for P, n, dt, mode, want in ((8, 1 << 26, "f32", "fused", 1),
                                 (15, 1 << 26, "f32", "fused", 1),
                                 (16, big32 // 64, "f32", "fused", 2),
                                 (16, big32 // 64 - 1, "f32", "fused", 1),
                                 (40, big32 // 160, "f32", "fused", 2),
                                 (40, big32 // 160 - 1, "f32", "fused", 1),
                                 (40, 4096, "f32", "fused", 1),
                                 (15, 1 << 26, "f16", "fused", 1),
                                 (16, big16 // 32, "f16", "fused", 2),
                                 (16, big16 // 32 - 1, "f16", "fused", 1),
                                 (1, 4096, "f32", "fused", 1),
                                 (40, 4096, "f32", "stepwise", 0)):
        plan = ddl.Plan(P, n, dt, "mean", ddl.topo("ring"), None, mode)
        assert plan.fused_passes() == want, (P, n, dt, mode)
        if mode == "fused" and P > 1:
            for v in (1, 2):
                plan.set_fused_passes(v)
                assert plan.fused_passes() == v
            plan.set_fused_passes(0)
            assert plan.fused_passes() == want
        for bad in (-1, 3):
            with pytest.raises(ddl.DDLError):
                plan.set_fused_passes(bad)
        plan.destroy()


def test_tuning_knobs():
    defaults = {"bcast_ranks": 0, "reduce_nt_load": 1, "fused_nt_load_max_p": 24, "anchor": 0,
                "fused_batch": 1, "reduce_batch": 4, "bcast_tiles": 1, "bcast_xcd": 0,
                "update_reps": 2, "update_batch": 4, "reduce_ranks_min_p": 16, "bcast_store_wait": 2,
                "fused_store_wait": 2}
    for k, v in defaults.items():
        assert ddl.get_tuning(k) == v, k
    for k in defaults:
        ddl.set_tuning(k, 5)
        assert ddl.get_tuning(k) == 5
        ddl.set_tuning(k, -1)
        assert ddl.get_tuning(k) == defaults[k]
    for bad in (-1, len(defaults)):
        with pytest.raises(ddl.DDLError):
            ddl.set_tuning(bad, 1)
        with pytest.raises(ddl.DDLError):
            ddl.get_tuning(bad)


def test_sgd_argument_validation_before_any_gpu_call():
    import ctypes
    P = 4
    for mode, nweights, keep, want in (("fused", 2, 1, -2), ("fused", 0, 1, -2),
                                       ("stepwise", 4, 0, -2), ("stepwise", 1, 0, -2)):
        plan = ddl.Plan(P, 1000, "f32", "mean", ddl.topo("ring"), None, mode)
        bufs = (ctypes.c_void_p * P)(*[16 * (r + 1) for r in range(P)])
        w = (ctypes.c_void_p * max(1, nweights))(*[4096 * (r + 1) for r in range(max(1, nweights))])
        rc = ddl.lib().ddl_plan_execute_sgd(plan.handle, bufs, w, nweights, 0.1, keep, None, None,
                                            None)
        assert rc == want, (mode, nweights, keep, rc)
        plan.destroy()


def test_lars_argument_validation_before_any_gpu_call():
    import ctypes
    P = 4
    nan, inf = float("nan"), float("inf")
    plan = ddl.Plan(P, 1000, "f32", "mean", ddl.topo("ring"), None, "fused")
    bufs = (ctypes.c_void_p * P)(*[16 * (r + 1) for r in range(P)])
    for nweights, coeff, eps, wofs, want in ((2, 0.01, 1e-6, 0, -2), (0, 0.01, 1e-6, 0, -2),
                                             (1, -0.01, 1e-6, 0, -2), (1, 0.01, -1e-6, 0, -2),
                                             (1, nan, 1e-6, 0, -2), (1, 0.01, nan, 0, -2),
                                             (1, inf, 1e-6, 0, -2), (P, 0.01, inf, 0, -2),
                                             (P, 0.01, 1e-6, 4, -4), (1, 0.01, 1e-6, 8, -4)):
        w = (ctypes.c_void_p * max(1, nweights))(
            *[4096 * (r + 1) + wofs for r in range(max(1, nweights))])
        rc = ddl.lib().ddl_plan_execute_lars(plan.handle, bufs, w, nweights, 0.1, coeff, eps,
                                             None, None, None, None)
        assert rc == want, (nweights, coeff, eps, wofs, rc)
    w = (ctypes.c_void_p * 1)(4096)
    assert ddl.lib().ddl_plan_execute_lars(plan.handle, bufs, None, 1, 0.1, 0.01, 1e-6, None,
                                           None, None, None) == -1
    assert ddl.lib().ddl_plan_execute_lars(None, bufs, w, 1, 0.1, 0.01, 1e-6, None, None, None,
                                           None) == -1
    plan.destroy()
    # no LARS on typed plans
    plan = ddl.Plan.typed(P, 4000, "sum", ddl.topo("ring"), [(0, 1000, "f32")])
    assert ddl.lib().ddl_plan_execute_lars(plan.handle, bufs, w, 1, 0.1, 0.01, 1e-6, None,
                                           None, None, None) == -2
    plan.destroy()


def test_schedule_generator_under_sanitizers(tmp_path):
    """The host schedule generator, built with AddressSanitizer and
    UndefinedBehaviorSanitizer (g++, host code only), through random
    configurations with an independent coverage/race/traffic check."""
    exe = tmp_path / "schedule_asan"
    src = os.path.join(ROOT, "tests", "schedule_asan_driver.cpp")
    lib_src = os.path.join(ROOT, "sgd_gradient_all_amd", "csrc", "schedule.cpp")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"),
                    src, lib_src, "-o", str(exe)], check=True)
    out = subprocess.run([str(exe), "400"], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "ok 400 cases" in out.stdout


def test_typed_plan_validation_and_tables():
    """Plans with typed buckets (byte offsets, a dtype per bucket): argument
    checks, and each bucket's tables equal a plain plan's of its dtype."""
    P = 6
    layout = [(0, 1000, "f32"), (4000, 2048, "f16"), (8096, 7, "f32"), (8124, 3, "f16"),
              (8130, 500, "f16")]
    nbytes = 8130 + 1000
    plan = ddl.Plan.typed(P, nbytes, "mean", ddl.topo("ring"), layout)
    for b, (off, cnt, dt) in enumerate(layout):
        esz = 4 if dt == "f32" else 2
        spans, group = plan.fused_spans(b)
        ref = ddl.Plan(P, off // esz + cnt, dt, "mean", ddl.topo("ring"),
                       [(0, off // esz), (off // esz, cnt)] if off else [(0, cnt)])
        want, _ = ref.fused_spans(1 if off else 0)
        assert spans == want, b
        items = plan.step_items(3, b)
        assert items == ref.step_items(3, 1 if off else 0), b
        ref.destroy()
    sent, hbm = plan.traffic()
    assert hbm == 2 * P * nbytes
    assert sum(sent) == 2 * (P - 1) * sum(c for _, c, _ in layout)
    plan.destroy()
    bad = [
        [(0, 1000, "f32"), (4002, 2047, "f16")],     # gap
        [(0, 1001, "f32"), (4000, 2048, "f16")],     # overlap
        [(2, 1000, "f32"), (4002, 2048, "f16")],     # f32 offset not a multiple of 4
        [(0, 1000, "f32"), (4000, 2049, "f16")],     # past the end
    ]
    for bl in bad:
        with pytest.raises(ddl.DDLError) as e:
            ddl.Plan.typed(P, 8096, "sum", ddl.topo("ring"), bl)
        assert e.value.code == -3, bl
    with pytest.raises(ddl.DDLError) as e:
        ddl.Plan.typed(P, 8, "sum", ddl.topo("ring"), [(0, 2, 7)])
    assert e.value.code == -2
    # no SGD on typed plans
    import ctypes
    plan = ddl.Plan.typed(P, 4000, "sum", ddl.topo("ring"), [(0, 1000, "f32")])
    bufs = (ctypes.c_void_p * P)(*[16 * (r + 1) for r in range(P)])
    w = (ctypes.c_void_p * 1)(4096)
    assert ddl.lib().ddl_plan_execute_sgd(plan.handle, bufs, w, 1, 0.1, 1, None, None,
                                          None) == -2
    plan.destroy()


def test_oneshot_rejects_bad_rank_counts_before_reading_ring_orders():
    """ddl_allreduce range-checks P (and k) before it reads the ring order
    into its cache key: a negative or too-large P with a ring order is
    DDL_E_ARG, not a read far past the caller's array."""
    import ctypes
    order = (ctypes.c_int * 4)(0, 1, 2, 3)
    bufs = (ctypes.c_void_p * 4)(*[16 * (r + 1) for r in range(4)])
    for P, kind, k in ((-1, 0, 1), (0, 0, 1), (ddl.DDL_MAX_RANKS + 1, 0, 1), (4, 1, 0), (4, 1, -3)):
        t = ddl.topo("ring") if kind == 0 else ddl.topo("multiring", 1)
        t.kind, t.k = kind, k
        t.ring_order = ctypes.cast(order, ctypes.POINTER(ctypes.c_int))
        rc = ddl.lib().ddl_allreduce(bufs, P, 100, 0, 0, ctypes.byref(t), None, 0, 1, None, None)
        assert rc == -2, (P, kind, k, rc)
    n = ctypes.c_size_t(99)
    assert ddl.lib().ddl_cache_count(ctypes.byref(n)) == 0 and n.value == 0


def test_plan_layer_under_sanitizers(tmp_path):
    """The plan layer's host code (plan.cpp with schedule.cpp), built with
    AddressSanitizer and UndefinedBehaviorSanitizer (g++, host code only),
    against a fake device whose memory is host memory: random plain and typed
    plans through every entry point, each kernel launch's tile ranges checked
    against the tables it indexes, and every allocation, stream and event
    released."""
    exe = tmp_path / "plan_asan"
    csrc = os.path.join(ROOT, "sgd_gradient_all_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__",
                    "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "plan_asan_driver.cpp"),
                    os.path.join(csrc, "plan.cpp"), os.path.join(csrc, "schedule.cpp"),
                    "-o", str(exe)], check=True)
    out = subprocess.run([str(exe), "150"], capture_output=True, text=True, timeout=600,
                         env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert out.returncode == 0, out.stdout[-3000:] + out.stderr[-3000:]
    assert "ok 150 cases" in out.stdout
