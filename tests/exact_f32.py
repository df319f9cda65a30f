"""Exact IEEE binary32 arithmetic for the oracle's pins (test helper).

Values are Python floats holding binary32 values (or +-inf, NaN).  Each
operation is evaluated exactly on ``fractions.Fraction`` and rounded once to
binary32 (nearest, ties to even, subnormals and overflow included) by the
integer procedure ``rn32``; signed zeros, infinities and NaN follow the IEEE 754
rules.  e^-g is evaluated with Python's ``decimal`` to 60 digits and rounded
only when the value is provably clear of a rounding boundary.  Nothing here
comes from the GPU library or its table generator.
"""
import decimal
import math
from fractions import Fraction

import numpy as np

decimal.getcontext().prec = 60
TWO = Fraction(2)
F32_OVERFLOW = TWO ** 128 - TWO ** 103      # at or above: rounds to infinity
INF, NAN = math.inf, math.nan


def rn32(x: Fraction) -> float:
    """x rounded once to the nearest binary32 (ties to even), as a Python float."""
    if x == 0:
        return 0.0
    neg = x < 0
    a = -x if neg else x
    if a >= F32_OVERFLOW:
        return -INF if neg else INF
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if a < TWO ** e:
        e -= 1                                   # now 2^e <= a < 2^(e+1)
    q = max(e, -126) - 23                        # the binary32 quantum at a (subnormals: 2^-149)
    m = a / TWO ** q
    n = m.numerator // m.denominator
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = float(n * TWO ** q)                      # exact in binary64
    return -v if neg else v


def _sign(x: float) -> float:
    return math.copysign(1.0, x)


def add(a: float, b: float) -> float:
    if math.isnan(a) or math.isnan(b):
        return NAN
    if math.isinf(a) or math.isinf(b):
        if math.isinf(a) and math.isinf(b) and _sign(a) != _sign(b):
            return NAN
        return a if math.isinf(a) else b
    s = Fraction(a) + Fraction(b)
    if s == 0:
        # an exact zero sum is +0 in round-to-nearest, except -0 + -0
        return -0.0 if (a == 0 and b == 0 and _sign(a) < 0 and _sign(b) < 0) else 0.0
    return rn32(s)


def sub(a: float, b: float) -> float:
    return add(a, -b)


def mul(a: float, b: float) -> float:
    if math.isnan(a) or math.isnan(b):
        return NAN
    sgn = _sign(a) * _sign(b)
    if math.isinf(a) or math.isinf(b):
        if a == 0 or b == 0:
            return NAN
        return math.copysign(INF, sgn)
    if a == 0 or b == 0:
        return math.copysign(0.0, sgn)
    return rn32(Fraction(a) * Fraction(b))


def div(a: float, b: float) -> float:
    if math.isnan(a) or math.isnan(b) or (math.isinf(a) and math.isinf(b)) or (a == 0 and b == 0):
        return NAN
    sgn = _sign(a) * _sign(b)
    if math.isinf(b) or a == 0:
        return math.copysign(0.0, sgn)
    if math.isinf(a) or b == 0:
        return math.copysign(INF, sgn)
    return rn32(Fraction(a) / Fraction(b))


def exp_neg_rn32(g: float) -> float:
    """RN32(e^-g), the decision checked to lie clear of the rounding boundary."""
    if g < -100.0:            # e^100 > FLT_MAX (ln FLT_MAX = 88.72): rounds to infinity
        return INF
    if g > 110.0:             # e^-110 < 2^-151, below half the smallest subnormal
        return 0.0
    d = (-decimal.Decimal(g)).exp()
    if d >= decimal.Decimal(2 ** 128 - 2 ** 103):
        return INF
    f = np.float32(float(d))
    cands = {float(c) for c in (np.nextafter(f, np.float32(0)), f, np.nextafter(f, np.float32(np.inf)))
             if np.isfinite(c)}
    dist = sorted((abs(decimal.Decimal(c) - d), c) for c in cands)
    # the nearest candidate must win by far more than the 60-digit evaluation error
    assert dist[1][0] - dist[0][0] > d * decimal.Decimal(10) ** -50, g
    return dist[0][1]


def f32_bits(v) -> np.ndarray:
    return np.asarray(v, np.float32).view(np.uint32)


def bf16_value(bits: int) -> float:
    return float(np.uint32(int(bits) << 16).view(np.float32))


def finite_bf16_patterns() -> np.ndarray:
    b = np.arange(65536, dtype=np.uint32)
    return b[(b & 0x7F80) != 0x7F80].astype(np.uint16)
