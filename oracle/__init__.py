"""ctypes wrapper of the CPU oracle (ddl_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  Everything here is
argument marshalling; the arithmetic is in ddl_oracle.c.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ddl_oracle.c")
# DDL_ORACLE_LIB: load another build of ddl_oracle.c (the mutation tests plant
# mistakes in scratch copies and check that the pins catch them)
_LIB_PATH = os.environ.get("DDL_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

F32, F16 = 0, 1
SUM, MEAN = 0, 1
RING, MULTIRING, TORUS2D = 0, 1, 2

CFLAGS = ["-O2", "-std=c11", "-Wall", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared"]


def build():
    """Compile liboracle.so with gcc (plain C, no fast-math, no contraction)."""
    subprocess.check_call(["gcc", *CFLAGS, "-o", _LIB_PATH, _SRC, "-lm"])


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        u64, i32, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p
        L.ddl_oracle_allreduce.argtypes = [
            ctypes.POINTER(vp), i32, u64, i32, i32, i32, i32, i32, i32,
            ctypes.POINTER(i32), ctypes.POINTER(u64), ctypes.POINTER(u64), i32,
            u64, u64, u64, ctypes.POINTER(u64)]
        L.ddl_oracle_allreduce.restype = i32
        L.ddl_oracle_sum_f64.argtypes = [ctypes.POINTER(vp), i32, u64, i32, i32, vp]
        L.ddl_oracle_sum_f64.restype = i32
        L.ddl_oracle_sgd.argtypes = [ctypes.POINTER(vp), i32, vp, u64, i32, ctypes.c_float]
        L.ddl_oracle_sgd.restype = i32
        L.ddl_oracle_lars.argtypes = [ctypes.POINTER(vp), i32, vp, ctypes.POINTER(u64),
                                      ctypes.POINTER(u64), i32, i32, ctypes.c_float,
                                      ctypes.c_double, ctypes.c_double, vp]
        L.ddl_oracle_lars.restype = i32
        L.ddl_oracle_split.argtypes = [u64, i32, u64, ctypes.POINTER(u64)]
        L.ddl_oracle_split.restype = None
        for name in ("ddl_oracle_f16_to_f32", "ddl_oracle_f32_to_f16"):
            getattr(L, name).argtypes = [vp, vp, u64]
            getattr(L, name).restype = None
        L.ddl_oracle_f16_add.argtypes = [vp, vp, vp, u64]
        L.ddl_oracle_f16_add.restype = None
        L.ddl_oracle_f16_div.argtypes = [vp, i32, vp, u64]
        L.ddl_oracle_f16_div.restype = None
        _lib = L
    return _lib


def _dtype_code(arr_dtype):
    if arr_dtype == np.float32:
        return F32
    if arr_dtype == np.float16:
        return F16
    raise TypeError(f"unsupported dtype {arr_dtype}")


def _u64(seq):
    seq = list(seq)
    return (ctypes.c_uint64 * max(1, len(seq)))(*seq)


def allreduce(bufs, op=SUM, kind=RING, k=1, rows=0, cols=0, ring_order=None,
              buckets=None, q=None, window=None, count_only_n=None):
    """Run the oracle in place on a list of P numpy arrays (one per rank).

    buckets: list of (offset, count) in issue order; default one bucket.
    q: split quantum in elements; default 16 bytes / element size.
    window: (lo, hi) when the arrays hold only elements [lo, hi) of the n
            elements per rank; then count_only_n gives n.
    Returns the per-rank sent-element counters (numpy uint64 array).
    """
    L = lib()
    P = len(bufs)
    dt = _dtype_code(bufs[0].dtype)
    for b in bufs:
        assert b.dtype == bufs[0].dtype and b.flags.c_contiguous and b.ndim == 1
    if window is None:
        n = bufs[0].shape[0]
        lo, hi = 0, n
    else:
        lo, hi = window
        n = count_only_n
        assert n is not None and bufs[0].shape[0] == hi - lo
    if q is None:
        q = 16 // bufs[0].itemsize
    if buckets is None:
        buckets = [(0, n)]
    ptrs = (ctypes.c_void_p * P)(*[b.ctypes.data for b in bufs])
    order = None
    if ring_order is not None:
        flat = [int(v) for v in np.asarray(ring_order).reshape(-1)]
        order = (ctypes.c_int * len(flat))(*flat)
    sent = (ctypes.c_uint64 * P)()
    rc = L.ddl_oracle_allreduce(
        ptrs, P, n, dt, op, kind, k, rows, cols, order,
        _u64(b[0] for b in buckets), _u64(b[1] for b in buckets), len(buckets),
        q, lo, hi, sent)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return np.array(list(sent), dtype=np.uint64)


def traffic(P, n, dtype=F32, kind=RING, k=1, rows=0, cols=0, ring_order=None,
            buckets=None, q=None):
    """Per-rank sent elements of the schedule, walked without buffers."""
    L = lib()
    if q is None:
        q = 4 if dtype == F32 else 8
    if buckets is None:
        buckets = [(0, n)]
    order = None
    if ring_order is not None:
        flat = [int(v) for v in np.asarray(ring_order).reshape(-1)]
        order = (ctypes.c_int * len(flat))(*flat)
    sent = (ctypes.c_uint64 * P)()
    rc = L.ddl_oracle_allreduce(
        None, P, n, dtype, SUM, kind, k, rows, cols, order,
        _u64(b[0] for b in buckets), _u64(b[1] for b in buckets), len(buckets),
        q, 0, n, sent)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return np.array(list(sent), dtype=np.uint64)


def sum_f64(bufs, op=SUM):
    """The plain definition in binary64: sum (or mean) over ranks."""
    L = lib()
    P = len(bufs)
    n = bufs[0].shape[0]
    out = np.empty(n, dtype=np.float64)
    ptrs = (ctypes.c_void_p * P)(*[b.ctypes.data for b in bufs])
    rc = L.ddl_oracle_sum_f64(ptrs, P, n, _dtype_code(bufs[0].dtype), op,
                              out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out


def sgd(weights, y, lr):
    """In place: every float32 array in weights takes w - lr * y (binary32,
    product then difference), y the all-reduced gradient."""
    L = lib()
    for w in weights:
        assert w.dtype == np.float32 and w.flags.c_contiguous and w.shape == y.shape
    ptrs = (ctypes.c_void_p * len(weights))(*[w.ctypes.data for w in weights])
    rc = L.ddl_oracle_sgd(ptrs, len(weights), y.ctypes.data, y.size, _dtype_code(y.dtype),
                          float(lr))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")


def lars(weights, y, layers, lr, coeff=0.01, eps=1e-6):
    """In place: the LARS step of every layer (offset, count) on every float32
    array in weights; returns the per-layer rates lr * trust (float32)."""
    L = lib()
    for w in weights:
        assert w.dtype == np.float32 and w.flags.c_contiguous and w.shape == y.shape
    ptrs = (ctypes.c_void_p * len(weights))(*[w.ctypes.data for w in weights])
    rates = np.zeros(max(1, len(layers)), dtype=np.float32)
    rc = L.ddl_oracle_lars(ptrs, len(weights), y.ctypes.data, _u64(o for o, _ in layers),
                           _u64(c for _, c in layers), len(layers), _dtype_code(y.dtype),
                           float(lr), float(coeff), float(eps), rates.ctypes.data)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return rates[:len(layers)]


def split(L_, m, q):
    out = (ctypes.c_uint64 * (m + 1))()
    lib().ddl_oracle_split(L_, m, q, out)
    return [int(v) for v in out]


def f16_to_f32(bits):
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float32)
    lib().ddl_oracle_f16_to_f32(bits.ctypes.data, out.ctypes.data, bits.size)
    return out


def f32_to_f16(vals):
    vals = np.ascontiguousarray(vals, dtype=np.float32)
    out = np.empty(vals.shape, dtype=np.uint16)
    lib().ddl_oracle_f32_to_f16(vals.ctypes.data, out.ctypes.data, vals.size)
    return out


def f16_add(a, b):
    a = np.ascontiguousarray(a, dtype=np.uint16)
    b = np.ascontiguousarray(b, dtype=np.uint16)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().ddl_oracle_f16_add(a.ctypes.data, b.ctypes.data, out.ctypes.data, a.size)
    return out


def f16_div(a, P):
    a = np.ascontiguousarray(a, dtype=np.uint16)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().ddl_oracle_f16_div(a.ctypes.data, P, out.ctypes.data, a.size)
    return out
