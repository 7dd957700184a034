"""Pins of the oracle's binary16 arithmetic against numpy's IEEE conversions.

numpy converts binary16 <-> binary32 / binary64 with round to nearest even and
keeps subnormals; it is a library routine independent of the oracle's own code.
The per-step rule fp16(f32(a) + f32(b)) must equal the correctly rounded
binary16 sum, computed here as the exact binary64 sum rounded once by numpy
(double rounding through binary32 is harmless since 24 >= 2*11 + 2).
"""
import numpy as np
import pytest

import oracle as orc


def _same_half(a, b):
    fa, fb = a.view(np.float16), b.view(np.float16)
    return (a == b) | (np.isnan(fa) & np.isnan(fb))


def test_f16_to_f32_exhaustive():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_to_f32(h)
    want = h.view(np.float16).astype(np.float32)
    same = (got.view(np.uint32) == want.view(np.uint32)) | (np.isnan(got) & np.isnan(want))
    assert same.all()


def _near_half_boundaries():
    """binary32 patterns within 2 ulps of every midpoint between adjacent
    binary16 values, and of every binary16 value itself."""
    h = np.arange(0, 0x7c00, dtype=np.uint16)          # non-negative finite
    v = h.view(np.float16).astype(np.float64)
    nxt = np.append(v[1:], 65536.0)
    mids = ((v + nxt) / 2).astype(np.float32)          # exact in binary32
    pts = np.concatenate([mids, v.astype(np.float32)]).view(np.uint32).astype(np.int64)
    out = [pts + d for d in (-2, -1, 0, 1, 2)]
    pts = np.clip(np.concatenate(out), 0, 0x7f7fffff).astype(np.uint32)
    return np.concatenate([pts, pts | np.uint32(0x80000000)])


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_f32_to_f16_boundaries_and_stride():
    pats = np.concatenate([
        _near_half_boundaries(),
        np.arange(0, 1 << 32, 251, dtype=np.uint64).astype(np.uint32),
        np.array([0x7f800000, 0xff800000, 0x7fc00000, 0x00000001, 0x80000001,
                  0x477fefff, 0x477ff000, 0x477ff001, 0x33000000, 0x33000001], np.uint32),
    ])
    x = pats.view(np.float32)
    got = orc.f32_to_f16(x)
    want = x.astype(np.float16).view(np.uint16)
    assert _same_half(got, want).all()


@pytest.mark.slow
@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_f32_to_f16_exhaustive():
    for hi in range(256):
        pats = (np.arange(1 << 24, dtype=np.uint32) | np.uint32(hi << 24))
        x = pats.view(np.float32)
        assert _same_half(orc.f32_to_f16(x), x.astype(np.float16).view(np.uint16)).all(), hi


def _add_reference(a, b):
    return (a.view(np.float16).astype(np.float64)
            + b.view(np.float16).astype(np.float64)).astype(np.float16).view(np.uint16)


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_f16_add_all_a_against_strided_b():
    a = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    for b0 in list(range(0, 1 << 16, 127)) + [0x0001, 0x8001, 0x03ff, 0x0400, 0x7bff,
                                                0xfbff, 0x7c00, 0xfc00, 0x3c00, 0xbc00]:
        b = np.full(a.shape, b0, dtype=np.uint16)
        assert _same_half(orc.f16_add(a, b), _add_reference(a, b)).all(), hex(b0)


@pytest.mark.slow
@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_f16_add_exhaustive():
    a = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    for b0 in range(1 << 16):
        b = np.full(a.shape, b0, dtype=np.uint16)
        assert _same_half(orc.f16_add(a, b), _add_reference(a, b)).all(), hex(b0)


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_f16_add_subnormals_kept():
    # the smallest subnormal plus itself is 2 x 2^-24, not zero
    one = np.array([1], np.uint16)
    assert orc.f16_add(one, one).tolist() == [2]
    # 2^-14 - 2^-24 (largest subnormal) + 2^-24 -> smallest normal
    assert orc.f16_add(np.array([0x3ff], np.uint16), one).tolist() == [0x400]
