"""Seeded synthetic gradients and the workload table.

Definitions of the values are in synth.h.  Host generation is synth.c
(libsynth_host.so, gcc); device generation is synth_fill.hip
(libsynth_dev.so, hipcc), which also holds the streaming compute kernel the
overlap measurement runs beside the all-reduce and plain streams of known
bytes (copy, read, write) for counter calibration and the rate a plain
stream reaches.  Neither holds any of the all-reduce's arithmetic.
"""
import ctypes
import os
import subprocess

import numpy as np

from .workloads import WORKLOADS, Workload, resnet50_param_sizes  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_HOST_SO = os.path.join(_HERE, "libsynth_host.so")
_DEV_SO = os.path.join(_HERE, "libsynth_dev.so")

F32, F16 = 0, 1
UNIFORM, NORMAL, RANKCONST, SMALLINT = 0, 1, 2, 3
DIST_CODES = {"uniform": UNIFORM, "normal": NORMAL, "rankconst": RANKCONST,
              "smallint": SMALLINT}

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build_host():
    subprocess.check_call(
        ["gcc", "-O2", "-std=c11", "-Wall", "-fopenmp", "-ffp-contract=off",
         "-fno-fast-math", "-fPIC", "-shared", "-o", _HOST_SO,
         os.path.join(_HERE, "synth.c")])


def build_dev():
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    subprocess.check_call(
        [hipcc, *HIP_FLAGS, "-o", _DEV_SO, os.path.join(_HERE, "synth_fill.hip")])


def build():
    build_host()
    build_dev()


_host = None
_dev = None


def host_lib():
    global _host
    if _host is None:
        if not os.path.exists(_HOST_SO):
            build_host()
        L = ctypes.CDLL(_HOST_SO)
        u64, i32, vp, dbl = ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p, ctypes.c_double
        L.synth_mix64.argtypes = [u64]
        L.synth_mix64.restype = u64
        L.synth_word.argtypes = [u64, i32, u64]
        L.synth_word.restype = u64
        L.synth_fill_host.argtypes = [vp, i32, i32, u64, i32, u64, u64, dbl]
        L.synth_fill_host.restype = None
        L.synth_gather_host.argtypes = [vp, i32, i32, u64, i32, vp, u64, dbl]
        L.synth_gather_host.restype = None
        L.synth_f32_to_f16.argtypes = [ctypes.c_float]
        L.synth_f32_to_f16.restype = ctypes.c_uint16
        _host = L
    return _host


def dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(_DEV_SO):
            build_dev()
        L = ctypes.CDLL(_DEV_SO)
        u64, i32, vp, dbl, f32 = (ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_double, ctypes.c_float)
        L.synth_fill_device.argtypes = [vp, i32, i32, u64, i32, u64, u64, dbl, vp]
        L.synth_fill_device.restype = i32
        L.synth_stream_compute.argtypes = [vp, u64, f32, f32, vp]
        L.synth_stream_compute.restype = i32
        L.synth_stream_copy.argtypes = [vp, vp, u64, vp]
        L.synth_stream_copy.restype = i32
        L.synth_stream_read.argtypes = [vp, u64, vp, vp]
        L.synth_stream_read.restype = i32
        L.synth_stream_write.argtypes = [vp, u64, f32, vp]
        L.synth_stream_write.restype = i32
        _dev = L
    return _dev


def np_dtype(code):
    return np.float32 if code == F32 else np.float16


def fill_host(n, dtype, dist, seed, rank, first=0, sigma=1.0):
    """Rank `rank`'s elements [first, first+n) as a numpy array."""
    out = np.empty(n, dtype=np_dtype(dtype))
    host_lib().synth_fill_host(out.ctypes.data, dtype, DIST_CODES.get(dist, dist),
                               seed, rank, first, n, sigma)
    return out


def gather_host(idx, dtype, dist, seed, rank, sigma=1.0):
    """Rank `rank`'s elements at the indices idx, as a numpy array."""
    idx = np.ascontiguousarray(idx, dtype=np.uint64)
    out = np.empty(idx.size, dtype=np_dtype(dtype))
    host_lib().synth_gather_host(out.ctypes.data, dtype, DIST_CODES.get(dist, dist),
                                 seed, rank, idx.ctypes.data, idx.size, sigma)
    return out


def fill_device(ptr, n, dtype, dist, seed, rank, first=0, sigma=1.0, stream=0):
    """Generate rank `rank`'s elements [first, first+n) into device memory."""
    rc = dev_lib().synth_fill_device(ptr, dtype, DIST_CODES.get(dist, dist), seed,
                                     rank, first, n, sigma, stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill_device failed ({rc})")


def stream_compute(ptr, n, alpha, beta, stream=0):
    """In-place a = alpha*a + beta over n fp32 elements (overlap workload)."""
    rc = dev_lib().synth_stream_compute(ptr, n, alpha, beta, stream)
    if rc != 0:
        raise RuntimeError(f"synth_stream_compute failed ({rc})")


def stream_copy(src, dst, n, stream=0):
    """dst = src over n fp32 elements, non-temporal (a stream of known bytes)."""
    rc = dev_lib().synth_stream_copy(src, dst, n, stream)
    if rc != 0:
        raise RuntimeError(f"synth_stream_copy failed ({rc})")


def stream_read(src, n, sink, stream=0):
    """Reads n fp32 elements (sink: 256 floats, written only in a case that
    does not arise)."""
    rc = dev_lib().synth_stream_read(src, n, sink, stream)
    if rc != 0:
        raise RuntimeError(f"synth_stream_read failed ({rc})")


def stream_write(dst, n, value, stream=0):
    """dst = value over n fp32 elements, non-temporal."""
    rc = dev_lib().synth_stream_write(dst, n, value, stream)
    if rc != 0:
        raise RuntimeError(f"synth_stream_write failed ({rc})")
