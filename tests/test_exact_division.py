"""The flush kernel divides x / s (quantization: x an fp16 value or a difference of two, s a
group scale) by a reciprocal-and-remainder sequence instead of IEEE division:
    y = RN(1/s),  q = RN(x y),  r = RN(x - q s) (one fused multiply-add),  RN(q + r y) (another).
Markstein's theorem says the last value is RN(x / s) when y is the correctly rounded reciprocal
and nothing overflows or underflows.  This pin checks that claim, independently of the theorem,
on every positive finite fp16 x (and on random fp32 dividends, as the fp16-metadata path's
x - m) for scales spread over the range a group of fp16 data can have:
the sequence is emulated with exactly the kernel's roundings (the fused steps in exact rational
arithmetic, one rounding each) and compared with numpy's correctly rounded fp32 division."""
from fractions import Fraction

import numpy as np
import pytest

X = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)   # every positive finite fp16


def _rn32(v: Fraction) -> np.float32:
    """Round a rational to the nearest fp32, ties to even."""
    f = np.float32(float(v))
    best, bd = f, abs(v - Fraction(float(f)))
    for nb in (np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))):
        d = abs(v - Fraction(float(nb)))
        if d < bd or (d == bd and (np.float32(nb).view(np.uint32) & 1) == 0):
            best, bd = np.float32(nb), d
    return best


@pytest.mark.parametrize("s", [2.0**-32 * 3, 1.0 / 255, 0.0731, 1.0 / 3, 7.777, 257.0 / 15, 21834.666])
def test_reciprocal_remainder_division_is_correctly_rounded(s):
    s = np.float32(s)
    y = np.float32(1.0) / s                              # correctly rounded reciprocal
    q = (X * y).astype(np.float32)                       # RN(x y)
    r64 = X.astype(np.float64) - q.astype(np.float64) * np.float64(s)   # exact (q s has 48 bits)
    r = r64.astype(np.float32)                           # the fused step's single rounding
    want = X / s                                         # numpy: correctly rounded fp32 division
    fy = Fraction(float(y))
    for i in range(X.size):
        got = _rn32(Fraction(float(q[i])) + Fraction(float(r[i])) * fy)
        assert got == want[i], (float(X[i]), float(s))


@pytest.mark.parametrize("s", [1.0 / 255, 7.777, 0.5001])
def test_fp32_dividends(s):
    """Dividends x - m of the fp16-metadata path are fp32 differences of two fp16 values, not
    fp16 values themselves: random fp32 magnitudes between 2^-24 and 2^17, both signs."""
    s = np.float32(s)
    rng = np.random.default_rng(11)
    x = (rng.choice([-1.0, 1.0], 8000) * np.exp2(rng.uniform(-24, 17, 8000))).astype(np.float32)
    y = np.float32(1.0) / s
    q = (x * y).astype(np.float32)
    r = (x.astype(np.float64) - q.astype(np.float64) * np.float64(s)).astype(np.float32)
    want = x / s
    fy = Fraction(float(y))
    for i in range(x.size):
        assert _rn32(Fraction(float(q[i])) + Fraction(float(r[i])) * fy) == want[i], (float(x[i]), float(s))


def test_zero_and_scale_one():
    """0 / s is 0 and a constant group's scale 1 returns x itself."""
    for s in (np.float32(1.0), np.float32(0.37)):
        y = np.float32(1.0) / s
        for x in (np.float32(0.0), np.float32(-0.0), np.float32(3.25)):
            q = np.float32(x * y)
            r = np.float32(np.float64(x) - np.float64(q) * np.float64(s))
            got = _rn32(Fraction(float(q)) + Fraction(float(r)) * Fraction(float(y)))
            assert got == np.float32(x / s)


def _fast_fp8_quotient(x: np.float32, s: np.float32, y: np.float32) -> np.float32:
    """The FP8 encoder's division with the kernel's roundings: q = RN(x y), r = RN(x - q s)
    (fused), then q itself when r is 0 or NaN, else RN(q + r y) (fused)."""
    q = np.float32(x * y)
    with np.errstate(invalid="ignore"):
        r = np.float32(np.float64(x) - np.float64(q) * np.float64(s))
    if not abs(r) > 0:
        return q
    return _rn32(Fraction(float(q)) + Fraction(float(r)) * Fraction(float(y)))


@pytest.mark.parametrize("s", [2.0**-60, 2.0**-60 * 1.3711, 3.1 / 448, 11.3 / 57344,
                               float(np.nextafter(np.float32(2.0**60), np.float32(0)))])
def test_fp8_division_every_fp16_value(s):
    """FP8 per-tensor scales inside [2^-60, 2^60] take the reciprocal-and-remainder division:
    every positive finite fp16 x gives the correctly rounded fp32 quotient at the range's ends
    and at calibrated scales; -0, +-inf and negative values give exactly x / s, sign included
    (an FP8 code keeps the sign of zero)."""
    s = np.float32(s)
    y = np.float32(1.0) / s
    q = (X * y).astype(np.float32)
    r = (X.astype(np.float64) - q.astype(np.float64) * np.float64(s)).astype(np.float32)
    want = X / s
    fy = Fraction(float(y))
    for i in range(X.size):
        got = q[i] if not abs(r[i]) > 0 else _rn32(Fraction(float(q[i])) + Fraction(float(r[i])) * fy)
        assert got == want[i], (float(X[i]), float(s))
    special = np.array([0.0, -0.0, np.inf, -np.inf, -65504.0, -2.0**-24, -1.5, -3.0e-5], np.float32)
    for x in special:
        got, ref = _fast_fp8_quotient(x, s, y), np.float32(x / s)
        assert got.view(np.uint32) == ref.view(np.uint32), (float(x), float(s))
