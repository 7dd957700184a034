"""Pins of the oracle's LARS step (Sony ResNet-50 article, "训练设置": LARS
with coefficient 0.01 and eps 1e-6; the trust ratio of You, Gitman and
Ginsburg's layer-wise adaptive rate scaling).

Expected values come from exact rational arithmetic (fractions, or decimal at
60 digits for square roots), closed forms chosen so the norms are exact,
invariants of the definition, and the reduction to the plain SGD step, which
has pins of its own.  A dropped eps, eps added to the squared norm, the two
norms swapped, a missing coefficient or learning rate, a norm taken from the
wrong replica or a rate shared across layers each fail one of them.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle as orc

getcontext().prec = 60
F32_EPS = Fraction(1, 2 ** 23)


def round_f32(x):
    """Nearest binary32 to the exact rational x (ties to even), and the
    relative distance from x to the nearest rounding boundary."""
    f = np.float32(float(x))
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(c)) - x)
        key = (d, int(np.frombuffer(c.tobytes(), np.uint32)[0]) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    c = best[1]
    lo = Fraction(float(np.nextafter(c, np.float32(-np.inf))))
    hi = Fraction(float(np.nextafter(c, np.float32(np.inf))))
    mid_lo, mid_hi = (lo + Fraction(float(c))) / 2, (hi + Fraction(float(c))) / 2
    margin = min(abs(x - mid_lo), abs(mid_hi - x)) / abs(x) if x else Fraction(1)
    return c, margin


def dsqrt(fr):
    return Decimal(fr.numerator) / Decimal(fr.denominator) if fr == 0 else \
        (Decimal(fr.numerator) / Decimal(fr.denominator)).sqrt()


def exact_rate(w0, y, lr, coeff, eps):
    """lr * trust at 60 digits, from the exact sums of squares."""
    W = sum(Fraction(float(v)) ** 2 for v in w0.astype(np.float64))
    G = sum(Fraction(float(v)) ** 2 for v in y.astype(np.float64))
    if W == 0 or G == 0:
        return Fraction(float(np.float32(lr)))
    t = Decimal(float(coeff)) * dsqrt(W) / (dsqrt(G) + Decimal(float(eps)))
    return Fraction(float(np.float32(lr))) * Fraction(t)


def f32_step(w, y, rate):
    """w - rate * y in binary32, product rounded first (numpy float32)."""
    prod = (np.float32(rate) * y.astype(np.float32)).astype(np.float32)
    return (w - prod).astype(np.float32)


# ---------------------------------------------------------------------------
# closed forms with exact norms
# ---------------------------------------------------------------------------
def test_closed_form_powers_of_two_eps_zero():
    # 16 elements of w = 2, y = 0.5: ||w|| = 8, ||y|| = 2, trust = 0.5 * 8 / 2
    # = 2, rate = 0.25 * 2 = 0.5, w' = 2 - 0.5 * 0.5 = 1.75, all exact
    w = np.full(16, 2.0, np.float32)
    y = np.full(16, 0.5, np.float32)
    rates = orc.lars([w], y, [(0, 16)], 0.25, coeff=0.5, eps=0.0)
    assert rates[0] == np.float32(0.5)
    assert np.all(w == np.float32(1.75))


def test_closed_form_page_constants_eps_matters():
    # 64 elements of w = 1.5, y = 2^-10: ||w|| = 12, ||y|| = 2^-7 exactly, so
    # lr * trust = lr * c * 12 / (2^-7 + e) with c, e the binary64 values of
    # 0.01 and 1e-6; eps shifts it by 1.3e-4 relative, a thousand binary32 ulps
    n = 64
    w = np.full(n, 1.5, np.float32)
    y = np.full(n, 2.0 ** -10, np.float32)
    lr = np.float32(0.1)
    x = Fraction(float(lr)) * Fraction(0.01) * 12 / (Fraction(1, 128) + Fraction(1e-6))
    want, margin = round_f32(x)
    assert margin > Fraction(1, 10 ** 12)  # far from a tie: binary64 steps cannot flip it
    w0 = w.copy()
    rates = orc.lars([w], y, [(0, n)], lr, coeff=0.01, eps=1e-6)
    assert rates[0] == want
    assert np.array_equal(w, f32_step(w0, y, want))
    # and eps really is in the denominator next to ||y||, not dropped and not
    # added to the squared norm
    no_eps, _ = round_f32(Fraction(float(lr)) * Fraction(0.01) * 12 * 128)
    sq_eps, _ = round_f32(Fraction(float(lr)) * Fraction(0.01) * 12 /
                          Fraction(Decimal(2.0 ** -14 + 1e-6).sqrt()))
    assert rates[0] != no_eps and rates[0] != sq_eps


def test_closed_form_f16_gradient():
    # binary16 gradient widened exactly: y = -0.25 (16 elements), w = 3 (16):
    # ||w|| = 12, ||y|| = 1, trust = 0.5 * 12 / 1 = 6, rate = 0.125 * 6 = 0.75,
    # w' = 3 - 0.75 * (-0.25) = 3.1875
    w = np.full(16, 3.0, np.float32)
    y = np.full(16, -0.25, np.float16)
    rates = orc.lars([w], y, [(0, 16)], 0.125, coeff=0.5, eps=0.0)
    assert rates[0] == np.float32(0.75)
    assert np.all(w == np.float32(3.1875))


# ---------------------------------------------------------------------------
# exact rational norms on small random layers
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(6))
def test_rates_against_exact_arithmetic(seed):
    rng = np.random.default_rng(seed)
    sizes = [1, 3, 7, 16, 33, 100]
    n = sum(sizes)
    w = (rng.standard_normal(n) * 0.05).astype(np.float32)
    y = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    layers, at = [], 0
    for c in sizes:
        layers.append((at, c))
        at += c
    lr = 0.1 * (seed + 1)
    w0 = w.copy()
    rates = orc.lars([w], y, layers, lr)
    for l, (o, c) in enumerate(layers):
        want, margin = round_f32(exact_rate(w0[o:o + c], y[o:o + c], lr, 0.01, 1e-6))
        if margin > Fraction(1, 10 ** 12):
            assert rates[l] == want, (l, rates[l], want)
        else:
            assert abs(Fraction(float(rates[l])) - Fraction(float(want))) <= \
                abs(Fraction(float(want))) * F32_EPS
        # the update itself: numpy float32 with the exactly derived rate
        assert np.array_equal(w[o:o + c], f32_step(w0[o:o + c], y[o:o + c], want))


# ---------------------------------------------------------------------------
# invariants and special cases
# ---------------------------------------------------------------------------
def test_gradient_scale_invariance_without_eps():
    # with eps = 0 the trust ratio is inversely proportional to ||y||: a
    # gradient scaled by 4 gets a rate scaled by 1/4 exactly (powers of two),
    # and the update rate * y is unchanged bit for bit
    rng = np.random.default_rng(7)
    n = 500
    layers = [(0, 120), (120, 200), (320, 180)]
    w = rng.standard_normal(n).astype(np.float32)
    y = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    a, b = w.copy(), w.copy()
    ra = orc.lars([a], y, layers, 0.3, coeff=0.01, eps=0.0)
    rb = orc.lars([b], (y * 4).astype(np.float32), layers, 0.3, coeff=0.01, eps=0.0)
    assert np.array_equal(rb * 4, ra)
    assert np.array_equal(a, b)


def test_weight_scale_scales_rate():
    # with eps = 0, weights scaled by 2 double the rate exactly
    rng = np.random.default_rng(8)
    w = rng.standard_normal(64).astype(np.float32)
    y = rng.standard_normal(64).astype(np.float32)
    r1 = orc.lars([w.copy()], y, [(0, 64)], 0.5, eps=0.0)
    r2 = orc.lars([(w * 2).astype(np.float32)], y, [(0, 64)], 0.5, eps=0.0)
    assert r2[0] == r1[0] * 2


def test_zero_layer_falls_back_to_sgd():
    # a layer of zero weights (or zero gradient) keeps trust 1: the plain SGD
    # step with lr, as orc.sgd computes it
    rng = np.random.default_rng(9)
    y = rng.standard_normal(40).astype(np.float32)
    w = np.zeros(40, np.float32)
    ref = w.copy()
    rates = orc.lars([w], y, [(0, 40)], 0.07)
    orc.sgd([ref], y, 0.07)
    assert rates[0] == np.float32(0.07)
    assert np.array_equal(w, ref)
    w = rng.standard_normal(40).astype(np.float32)
    w0 = w.copy()
    rates = orc.lars([w], np.zeros(40, np.float32), [(0, 40)], 0.07)
    assert rates[0] == np.float32(0.07)
    assert np.array_equal(w, w0)


def test_layers_independent_and_norms_from_replica_zero():
    rng = np.random.default_rng(10)
    n = 300
    layers = [(0, 100), (100, 150), (250, 50)]
    w = rng.standard_normal(n).astype(np.float32)
    other = rng.standard_normal(n).astype(np.float32)   # replica 1 differs
    y = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    a, b = w.copy(), other.copy()
    rates = orc.lars([a, b], y, layers, 0.2)
    # each layer alone gives the same rate and update (order of layers and
    # the other layers' contents do not matter)
    for l, (o, c) in enumerate(layers[::-1]):
        solo = w[o:o + c].copy()
        r = orc.lars([solo], y[o:o + c].copy(), [(0, c)], 0.2)
        assert r[0] == rates[len(layers) - 1 - l]
        assert np.array_equal(solo, a[o:o + c])
    # replica 1 is stepped with replica 0's rates
    for l, (o, c) in enumerate(layers):
        assert np.array_equal(b[o:o + c], f32_step(other[o:o + c], y[o:o + c], rates[l]))
    # distinct layers really get distinct rates here
    assert len(set(rates.tolist())) == len(layers)


def test_empty_layers_and_bad_arguments():
    w = np.ones(8, np.float32)
    y = np.ones(8, np.float32)
    rates = orc.lars([w], y, [(0, 0), (0, 8), (8, 0)], 0.5, coeff=1.0, eps=0.0)
    assert rates[0] == np.float32(0.5) and rates[2] == np.float32(0.5)
    assert rates[1] == np.float32(0.5)  # ||w|| / ||y|| = 1
    for coeff, eps in ((-0.01, 1e-6), (0.01, -1e-6), (float("nan"), 1e-6),
                       (0.01, float("inf"))):
        with pytest.raises(ValueError):
            orc.lars([w], y, [(0, 8)], 0.5, coeff=coeff, eps=eps)
