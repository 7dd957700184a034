"""ctypes binding of include/ddl.h.  Argument marshalling only."""
import atexit
import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libddl.so")

DDL_MAX_RANKS = 128
DDL_F32, DDL_F16 = 0, 1
DDL_SUM, DDL_MEAN = 0, 1
DDL_RING, DDL_MULTIRING, DDL_TORUS2D = 0, 1, 2
DDL_STEPWISE, DDL_FUSED = 0, 1
DDL_K_REDUCE, DDL_K_GATHER, DDL_K_FUSED, DDL_K_FUSED_REDUCE, DDL_K_BROADCAST = 0, 1, 2, 3, 4
DDL_K_LARS_NORM, DDL_K_LARS_RATE, DDL_K_UPDATE, DDL_K_WALK = 5, 6, 7, 8
DDL_K_COUNT = 9
LAUNCH_KINDS = ("reduce", "gather", "fused", "fused_reduce", "broadcast", "lars_norm",
                "lars_rate", "update", "walk")
# LARS as the Sony ResNet-50 article trains with it: coefficient and eps
LARS_COEFF, LARS_EPS = 0.01, 1e-6

_DTYPES = {"f32": DDL_F32, "f16": DDL_F16, "float32": DDL_F32, "float16": DDL_F16}
_OPS = {"sum": DDL_SUM, "mean": DDL_MEAN}
_MODES = {"stepwise": DDL_STEPWISE, "fused": DDL_FUSED}
_KINDS = {"ring": DDL_RING, "multiring": DDL_MULTIRING, "torus2d": DDL_TORUS2D}


class ddl_topo(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("k", ctypes.c_int), ("rows", ctypes.c_int),
                ("cols", ctypes.c_int), ("ring_order", ctypes.POINTER(ctypes.c_int))]


class ddl_bucket(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_size_t), ("count", ctypes.c_size_t),
                ("ready_event", ctypes.c_void_p)]


class ddl_typed_bucket(ctypes.Structure):
    _fields_ = [("byte_offset", ctypes.c_size_t), ("count", ctypes.c_size_t),
                ("dtype", ctypes.c_int)]


class ddl_step_item(ctypes.Structure):
    _fields_ = [("src", ctypes.c_int), ("dst", ctypes.c_int), ("divide", ctypes.c_int),
                ("step", ctypes.c_int), ("offset", ctypes.c_size_t),
                ("count", ctypes.c_size_t)]


class DDLError(RuntimeError):
    def __init__(self, code, what=""):
        self.code = code
        super().__init__(f"{what}: {ddl_strerror(code)} ({code})" if what else
                         f"{ddl_strerror(code)} ({code})")


_lib = None


def lib():
    """Load libddl.so.  There is no fallback: without the library, fail."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(
                f"{_LIB_PATH} is not built; run sgd_gradient_all_amd/_build.py "
                "(or __graft_entry__.build())")
        L = ctypes.CDLL(_LIB_PATH)
        i32, vp, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        P_topo, P_bucket = ctypes.POINTER(ddl_topo), ctypes.POINTER(ddl_bucket)
        sig = {
            "ddl_plan_create": ([ctypes.POINTER(vp), i32, sz, i32, i32, P_topo, P_bucket,
                                 i32, i32], i32),
            "ddl_plan_create_typed": ([ctypes.POINTER(vp), i32, sz, i32, P_topo,
                                       ctypes.POINTER(ddl_typed_bucket), i32, i32], i32),
            "ddl_plan_execute": ([vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp], i32),
            "ddl_allreduce": ([ctypes.POINTER(vp), i32, sz, i32, i32, P_topo, P_bucket, i32,
                               i32, vp, vp], i32),
            "ddl_plan_execute_sgd": ([vp, ctypes.POINTER(vp), ctypes.POINTER(vp), i32,
                                      ctypes.c_float, i32, ctypes.POINTER(vp), vp, vp], i32),
            "ddl_plan_execute_lars": ([vp, ctypes.POINTER(vp), ctypes.POINTER(vp), i32,
                                       ctypes.c_float, ctypes.c_double, ctypes.c_double,
                                       vp, ctypes.POINTER(vp), vp, vp], i32),
            "ddl_plan_execute_lars_noalloc": ([vp, ctypes.POINTER(vp), ctypes.POINTER(vp), i32,
                                               ctypes.c_float, ctypes.c_double, ctypes.c_double,
                                               vp, ctypes.POINTER(vp), vp, vp], i32),
            "ddl_plan_traffic": ([vp, ctypes.POINTER(sz), ctypes.POINTER(sz)], i32),
            "ddl_plan_destroy": ([vp], i32),
            "ddl_cache_clear": ([], i32),
            "ddl_cache_count": ([ctypes.POINTER(sz)], i32),
            "ddl_strerror": ([i32], ctypes.c_char_p),
            "ddl_plan_set_coalesce_bytes": ([vp, sz], i32),
            "ddl_plan_set_side_streams": ([vp, i32], i32),
            "ddl_plan_set_ordered_events": ([vp, i32], i32),
            "ddl_plan_event_groups": ([vp, ctypes.POINTER(i32), i32], i32),
            "ddl_plan_set_fused_passes": ([vp, i32], i32),
            "ddl_set_tuning": ([i32, i32], i32),
            "ddl_get_tuning": ([i32, ctypes.POINTER(i32)], i32),
            "ddl_plan_get_fused_passes": ([vp, ctypes.POINTER(i32)], i32),
            "ddl_plan_set_step_form": ([vp, i32], i32),
            "ddl_plan_get_step_form": ([vp, ctypes.POINTER(i32)], i32),
            "ddl_plan_profile_read_kinds": ([vp, ctypes.POINTER(ctypes.c_double),
                                             ctypes.POINTER(i32),
                                             ctypes.POINTER(ctypes.c_double)], i32),
            "ddl_plan_set_profiling": ([vp, i32], i32),
            "ddl_plan_profile_read": ([vp, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_double)],
                                      i32),
            "ddl_plan_num_steps": ([vp, ctypes.POINTER(i32)], i32),
            "ddl_plan_step_kind": ([vp, i32, ctypes.POINTER(i32)], i32),
            "ddl_plan_step_items": ([vp, i32, i32, ctypes.POINTER(ddl_step_item), i32,
                                     ctypes.POINTER(i32)], i32),
            "ddl_plan_fused_spans": ([vp, i32, ctypes.POINTER(sz), ctypes.POINTER(sz),
                                      ctypes.POINTER(i32), i32, ctypes.POINTER(i32),
                                      ctypes.POINTER(i32)], i32),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def ddl_strerror(code):
    return lib().ddl_strerror(code).decode()


def _check(rc, what):
    if rc != 0:
        raise DDLError(rc, what)


def _code(table, v):
    return table[v] if isinstance(v, str) else int(v)


def _ptr(x):
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    for attr in ("cuda_stream", "cuda_event"):
        if hasattr(x, attr):
            return getattr(x, attr)
    return int(x)


_hip = None


def _hip_lib():
    global _hip
    if _hip is None:
        h = ctypes.CDLL("libamdhip64.so")
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        h.hipEventCreateWithFlags.restype = ctypes.c_int
        h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventRecord.restype = ctypes.c_int
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipEventDestroy.restype = ctypes.c_int
        _hip = h
    return _hip


class ReadyEvent:
    """A HIP event for a bucket's readiness, made through the HIP runtime
    (hipEventCreateWithFlags), with timing disabled and, by default, without
    the system-scope fence an event record otherwise performs: the library
    only makes its streams wait for ready events, which orders the device
    work on either side, and never inspects them from the host.  A record
    then costs the device less, and does not write back and invalidate the
    caches under the kernels running beside it.  Pass it wherever an event
    goes (it has cuda_event); record(stream) records it on a stream (a torch
    stream or a raw handle; None = the null stream)."""

    DISABLE_TIMING = 0x2
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, system_fence=False):
        flags = self.DISABLE_TIMING | (0 if system_fence else self.DISABLE_SYSTEM_FENCE)
        h = ctypes.c_void_p()
        rc = _hip_lib().hipEventCreateWithFlags(ctypes.byref(h), flags)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.cuda_event = h.value

    def record(self, stream=None):
        rc = _hip_lib().hipEventRecord(self.cuda_event, _ptr(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def __del__(self):
        if getattr(self, "cuda_event", None) and _hip is not None:
            _hip.hipEventDestroy(self.cuda_event)
            self.cuda_event = None


def topo(kind="ring", k=1, rows=0, cols=0, ring_order=None):
    """A ddl_topo (the ring order array is kept alive on the object)."""
    t = ddl_topo()
    t.kind = _code(_KINDS, kind)
    t.k, t.rows, t.cols = k, rows, cols
    if ring_order is not None:
        flat = [int(v) for v in ring_order]
        t._order = (ctypes.c_int * len(flat))(*flat)
        t.ring_order = t._order
    return t


def _buckets(buckets, events=None):
    if buckets is None:
        return None, 0
    arr = (ddl_bucket * max(1, len(buckets)))()
    for i, (off, cnt) in enumerate(buckets):
        arr[i].offset, arr[i].count = off, cnt
        arr[i].ready_event = _ptr(events[i]) if events is not None else None
    return arr, len(buckets)


def _bufs(bufs):
    return (ctypes.c_void_p * len(bufs))(*[_ptr(b) for b in bufs])


def ddl_allreduce(bufs, n, dtype="f32", op="sum", topology=None, buckets=None,
                  mode="fused", stream=None, done_event=None, events=None):
    """One-shot all-reduce with a cached plan (see ddl_allreduce in ddl.h)."""
    t = topology if topology is not None else topo()
    barr, nb = _buckets(buckets, events)
    rc = lib().ddl_allreduce(_bufs(bufs), len(bufs), n, _code(_DTYPES, dtype),
                             _code(_OPS, op), ctypes.byref(t), barr, nb, _code(_MODES, mode),
                             _ptr(stream), _ptr(done_event))
    _check(rc, "ddl_allreduce")


def ddl_cache_clear():
    _check(lib().ddl_cache_clear(), "ddl_cache_clear")


def ddl_cache_count():
    """Plans ddl_allreduce holds in its cache (at most 64)."""
    n = ctypes.c_size_t(0)
    _check(lib().ddl_cache_count(ctypes.byref(n)), "ddl_cache_count")
    return n.value


TUNE = {"bcast_ranks": 0, "reduce_nt_load": 1, "fused_nt_load_max_p": 2, "anchor": 3,
        "fused_batch": 4, "reduce_batch": 5, "bcast_tiles": 6, "bcast_xcd": 7,
        "update_reps": 8, "update_batch": 9, "reduce_ranks_min_p": 10,
        "bcast_store_wait": 11, "fused_store_wait": 12}


def set_tuning(knob, value):
    """Process-wide kernel knob (ddl_set_tuning); value < 0 restores the default."""
    _check(lib().ddl_set_tuning(_code(TUNE, knob), int(value)), "ddl_set_tuning")


def get_tuning(knob):
    v = ctypes.c_int()
    _check(lib().ddl_get_tuning(_code(TUNE, knob), ctypes.byref(v)), "ddl_get_tuning")
    return v.value


# Handles of Plans garbage-collected while their work was still in flight
# (ddl_plan_destroy answered DDL_E_BUSY): destroyed later, when the next
# Plan is made or executed, or at exit, instead of being leaked.
_pending = []
_pending_lock = threading.RLock()  # __del__ may run inside _reap


def _reap():
    """Destroy the pending handles whose work has completed; returns how many
    are still pending."""
    with _pending_lock:
        if not _pending:
            return 0
        keep = []
        for h in _pending:
            rc = lib().ddl_plan_destroy(h)
            if rc == -7:  # DDL_E_BUSY: still in flight
                keep.append(h)
        _pending[:] = keep
        return len(keep)


atexit.register(_reap)


class Plan:
    """Owner of a ddl_plan (ddl_plan_create / execute / traffic / destroy)."""

    def __init__(self, P, n, dtype="f32", op="sum", topology=None, buckets=None,
                 mode="fused"):
        _reap()
        self.P, self.n = P, n
        self.nbuckets = len(buckets) if buckets is not None else (1 if n else 0)
        t = topology if topology is not None else topo()
        barr, nb = _buckets(buckets)
        h = ctypes.c_void_p()
        _check(lib().ddl_plan_create(ctypes.byref(h), P, n, _code(_DTYPES, dtype),
                                     _code(_OPS, op), ctypes.byref(t), barr, nb,
                                     _code(_MODES, mode)), "ddl_plan_create")
        self.handle = h

    @classmethod
    def typed(cls, P, nbytes, op="sum", topology=None, buckets=(), mode="fused"):
        """A plan whose buckets carry their own dtype: buckets is a list of
        (byte_offset, count, dtype) in issue order (ddl_plan_create_typed)."""
        _reap()
        self = cls.__new__(cls)
        self.P, self.n, self.nbuckets = P, nbytes, len(buckets)
        self.handle = None
        t = topology if topology is not None else topo()
        arr = (ddl_typed_bucket * max(1, len(buckets)))()
        for i, (off, cnt, dt) in enumerate(buckets):
            arr[i].byte_offset, arr[i].count, arr[i].dtype = off, cnt, _code(_DTYPES, dt)
        h = ctypes.c_void_p()
        _check(lib().ddl_plan_create_typed(ctypes.byref(h), P, nbytes, _code(_OPS, op),
                                           ctypes.byref(t), arr, len(buckets),
                                           _code(_MODES, mode)), "ddl_plan_create_typed")
        self.handle = h
        return self

    def execute(self, bufs, events=None, stream=None, done_event=None):
        if _pending:
            _reap()
        if len(bufs) != self.P:
            raise ValueError(f"expected {self.P} buffers, got {len(bufs)}")
        ev = None
        if events is not None:
            ev = (ctypes.c_void_p * max(1, len(events)))(*[_ptr(e) for e in events])
        _check(lib().ddl_plan_execute(self.handle, _bufs(bufs), ev, _ptr(stream),
                                      _ptr(done_event)), "ddl_plan_execute")

    def execute_sgd(self, bufs, weights, lr, keep_grads=True, events=None, stream=None,
                    done_event=None):
        """All-reduce, then w = w - lr * y on every weight replica (one per rank,
        or a single shared one), fused into the reduction's epilogue."""
        if len(bufs) != self.P:
            raise ValueError(f"expected {self.P} buffers, got {len(bufs)}")
        ev = None
        if events is not None:
            ev = (ctypes.c_void_p * max(1, len(events)))(*[_ptr(e) for e in events])
        _check(lib().ddl_plan_execute_sgd(self.handle, _bufs(bufs), _bufs(weights), len(weights),
                                          float(lr), 1 if keep_grads else 0, ev, _ptr(stream),
                                          _ptr(done_event)), "ddl_plan_execute_sgd")

    def execute_lars(self, bufs, weights, lr, coeff=LARS_COEFF, eps=LARS_EPS, rates_out=None,
                     events=None, stream=None, done_event=None):
        """All-reduce, then the LARS step of every bucket (a layer): rate =
        lr * coeff * ||w|| / (||y|| + eps), w = w - rate * y on every replica.
        rates_out: None or device memory (pointer or tensor) for one float32
        per bucket."""
        if len(bufs) != self.P:
            raise ValueError(f"expected {self.P} buffers, got {len(bufs)}")
        ev = None
        if events is not None:
            ev = (ctypes.c_void_p * max(1, len(events)))(*[_ptr(e) for e in events])
        _check(lib().ddl_plan_execute_lars(self.handle, _bufs(bufs), _bufs(weights),
                                           len(weights), float(lr), float(coeff), float(eps),
                                           _ptr(rates_out), ev, _ptr(stream),
                                           _ptr(done_event)), "ddl_plan_execute_lars")

    def execute_lars_noalloc(self, bufs, weights, lr, coeff=LARS_COEFF, eps=LARS_EPS,
                             rates_out=None, events=None, stream=None, done_event=None):
        """execute_lars without any device allocation: the partial sums and
        rates live in the library's fixed per-device scratch (the plan must
        have run on the device before; ddl_plan_execute_lars_noalloc)."""
        if len(bufs) != self.P:
            raise ValueError(f"expected {self.P} buffers, got {len(bufs)}")
        ev = None
        if events is not None:
            ev = (ctypes.c_void_p * max(1, len(events)))(*[_ptr(e) for e in events])
        _check(lib().ddl_plan_execute_lars_noalloc(self.handle, _bufs(bufs), _bufs(weights),
                                                   len(weights), float(lr), float(coeff),
                                                   float(eps), _ptr(rates_out), ev,
                                                   _ptr(stream), _ptr(done_event)),
               "ddl_plan_execute_lars_noalloc")

    def traffic(self):
        sent = (ctypes.c_size_t * self.P)()
        hbm = ctypes.c_size_t()
        _check(lib().ddl_plan_traffic(self.handle, sent, ctypes.byref(hbm)), "ddl_plan_traffic")
        return list(sent), hbm.value

    def set_coalesce_bytes(self, nbytes):
        _check(lib().ddl_plan_set_coalesce_bytes(self.handle, nbytes), "set_coalesce_bytes")

    def event_groups(self):
        """List index of the last bucket of each group a call forms at the
        current threshold when every bucket has its own ready event; one
        event per group, shared by the group's buckets, gives the same
        groups with one record and one wait per group."""
        n = lib().ddl_plan_event_groups(self.handle, None, 0)
        if n < 0:
            _check(n, "ddl_plan_event_groups")
        last = (ctypes.c_int * max(1, n))()
        _check(min(0, lib().ddl_plan_event_groups(self.handle, last, n)), "ddl_plan_event_groups")
        return list(last[:n])

    def set_ordered_events(self, ordered=True):
        """Promise that the ready events are recorded in bucket list order on
        one stream: a group then waits for its last event only."""
        _check(lib().ddl_plan_set_ordered_events(self.handle, 1 if ordered else 0),
               "set_ordered_events")

    def set_side_streams(self, n):
        _check(lib().ddl_plan_set_side_streams(self.handle, n), "set_side_streams")

    def set_fused_passes(self, passes):
        """0 automatic, 1 one kernel, 2 reduce kernel + broadcast kernel."""
        _check(lib().ddl_plan_set_fused_passes(self.handle, int(passes)), "set_fused_passes")

    def fused_passes(self):
        v = ctypes.c_int()
        _check(lib().ddl_plan_get_fused_passes(self.handle, ctypes.byref(v)), "fused_passes")
        return v.value

    def set_step_form(self, form):
        """Stepwise plans: 0 automatic, 1 one launch per schedule step, 2 one
        persistent launch per group (each workgroup walks every step of a tile)."""
        _check(lib().ddl_plan_set_step_form(self.handle, int(form)), "set_step_form")

    def step_form(self):
        v = ctypes.c_int()
        _check(lib().ddl_plan_get_step_form(self.handle, ctypes.byref(v)), "step_form")
        return v.value

    def set_profiling(self, on=True):
        """True/1: bracket every launch with HIP events; an int m > 1: the
        launches of every m-th bucket group; False/0: off."""
        v = int(on) if not isinstance(on, bool) else (1 if on else 0)
        _check(lib().ddl_plan_set_profiling(self.handle, v), "set_profiling")

    def profile_read(self):
        tot, mx = ctypes.c_double(), ctypes.c_double()
        cnt = ctypes.c_int()
        _check(lib().ddl_plan_profile_read(self.handle, ctypes.byref(tot), ctypes.byref(cnt),
                                           ctypes.byref(mx)), "profile_read")
        return tot.value, cnt.value, mx.value

    def profile_read_kinds(self):
        """{kind name: (total ms, launches, longest ms)} since the last read."""
        tot = (ctypes.c_double * DDL_K_COUNT)()
        mx = (ctypes.c_double * DDL_K_COUNT)()
        cnt = (ctypes.c_int * DDL_K_COUNT)()
        _check(lib().ddl_plan_profile_read_kinds(self.handle, tot, cnt, mx),
               "profile_read_kinds")
        return {LAUNCH_KINDS[k]: (tot[k], cnt[k], mx[k]) for k in range(DDL_K_COUNT)}

    def num_steps(self):
        s = ctypes.c_int()
        _check(lib().ddl_plan_num_steps(self.handle, ctypes.byref(s)), "num_steps")
        return s.value

    def step_kind(self, step):
        k = ctypes.c_int()
        _check(lib().ddl_plan_step_kind(self.handle, step, ctypes.byref(k)), "step_kind")
        return k.value

    def step_items(self, step, bucket):
        cnt = ctypes.c_int()
        _check(lib().ddl_plan_step_items(self.handle, step, bucket, None, 0, ctypes.byref(cnt)),
               "step_items")
        arr = (ddl_step_item * max(1, cnt.value))()
        _check(lib().ddl_plan_step_items(self.handle, step, bucket, arr, cnt.value,
                                         ctypes.byref(cnt)), "step_items")
        return [(a.src, a.dst, a.divide, a.offset, a.count) for a in arr[:cnt.value]]

    def fused_spans(self, bucket):
        ns, grp = ctypes.c_int(), ctypes.c_int()
        _check(lib().ddl_plan_fused_spans(self.handle, bucket, None, None, None, 0,
                                          ctypes.byref(ns), ctypes.byref(grp)), "fused_spans")
        m = max(1, ns.value)
        off, cnt = (ctypes.c_size_t * m)(), (ctypes.c_size_t * m)()
        chain = (ctypes.c_int * (m * self.P))()
        _check(lib().ddl_plan_fused_spans(self.handle, bucket, off, cnt, chain, ns.value,
                                          ctypes.byref(ns), ctypes.byref(grp)), "fused_spans")
        spans = [(off[i], cnt[i], list(chain[i * self.P:(i + 1) * self.P]))
                 for i in range(ns.value)]
        return spans, grp.value

    def destroy(self):
        if self.handle:
            _check(lib().ddl_plan_destroy(self.handle), "ddl_plan_destroy")
            self.handle = None

    def try_destroy(self):
        """ddl_plan_destroy that reports work in flight instead of raising:
        returns 0 once the plan is freed, DDL_E_BUSY (-7) while it is not."""
        if not self.handle:
            return 0
        rc = lib().ddl_plan_destroy(self.handle)
        if rc == 0:
            self.handle = None
        elif rc != -7:
            _check(rc, "ddl_plan_destroy")
        return rc

    def __del__(self):
        try:
            h = getattr(self, "handle", None)
            if h:
                self.handle = None
                if lib().ddl_plan_destroy(h) == -7:  # busy: destroy it later
                    with _pending_lock:
                        _pending.append(h)
        except Exception:
            pass


def ddl_plan_create(*args, **kw):
    return Plan(*args, **kw)
