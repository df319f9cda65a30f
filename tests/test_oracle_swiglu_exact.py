"""The oracle's SwiGLU evaluated exactly, one rounding at a time, on rationals.

The SwiGLU reading takes h = silu(g) * u as four IEEE binary32 operations in a
fixed order ("LLMQ: Efficient Lower-Precision Pretraining for Consumer GPUs",
section 3.1, requantisation fused with the nonlinearity; the pages print no
formula, so the textbook silu(g) = g / (1 + e^-g) is used):

    E   = RN32(e^-g)          (correctly rounded)
    t   = RN32(1 + E)
    s_g = RN32(g / t)
    h   = RN32(s_g * u)

Here every step is recomputed from its definition (``exact_f32``, the tests'
exact binary32 helpers): e^-g from Python's ``decimal`` (60 digits, and the
rounding decision is made only when the value is provably away from a rounding
boundary), the sum, quotient and product exactly on ``fractions.Fraction``, and
each result rounded once to binary32 (nearest, ties to even, subnormals and
overflow included) by an integer procedure.  Nothing is imported from the GPU library or
its table generator.  The oracle's h must equal it bit for bit for every
finite bf16 gate value (u = 1, so h = s_g), and for a seeded sample of gate
values times several up values (the last rounding).  A plausible slip -- g
multiplied by RN32(1 / t) instead of divided by t, an FMA contraction of any
two steps, a float exponential that is not correctly rounded, or the halves
of [gate | up] swapped -- changes some of these bits.
"""
from fractions import Fraction

import numpy as np

from exact_f32 import F32_OVERFLOW, TWO, exp_neg_rn32, f32_bits, finite_bf16_patterns, rn32


def swiglu_exact(gbits: int, ubits: int) -> float:
    g = float(np.uint32(gbits << 16).view(np.float32))
    u = float(np.uint32(ubits << 16).view(np.float32))
    E = exp_neg_rn32(g)
    if np.isinf(E):
        s = -0.0 if g < 0 else np.nan            # g / inf for finite negative g
    else:
        t = rn32(1 + Fraction(E))
        s = rn32(Fraction(g) / Fraction(t))
        if s == 0.0:
            s = -0.0 if g < 0 or (g == 0 and np.signbit(g)) else 0.0
    if s == 0.0:
        return float(np.float32(s) * np.float32(u))      # a signed zero times u: exact
    if u == 0.0:
        return float(np.float32(s) * np.float32(u))
    return rn32(Fraction(s) * Fraction(u))


def test_exact_rounding_helper():
    """rn32 against numpy's binary64 -> binary32 conversion (itself a single
    RNE rounding) on values that binary64 holds exactly, ties included."""
    rng = np.random.default_rng(3)
    for _ in range(2000):
        m = int(rng.integers(1, 1 << 40))
        e = int(rng.integers(-170, 130))
        x = Fraction(m) * TWO ** e
        with np.errstate(over="ignore"):
            ref = np.float32(float(x))
        assert f32_bits(rn32(x)) == f32_bits(ref), (m, e)
    for k in (0, 1, 3):                           # exact ties: 1 + (2k + 1) 2^-24
        x = 1 + Fraction(2 * k + 1, 1 << 24)
        assert rn32(x) == float(np.float32(float(x)))
    assert rn32(F32_OVERFLOW) == np.inf and rn32(F32_OVERFLOW - TWO ** 80) == float(np.finfo(np.float32).max)
    assert rn32(TWO ** -150) == 0.0 and rn32(TWO ** -150 + TWO ** -200) == 2.0 ** -149


def test_every_gate_value(orc):
    """h = s_g (u = 1) for every finite bf16 gate value, bit for bit."""
    g = finite_bf16_patterns()
    ones = np.full_like(g, 0x3F80)
    h = orc.swiglu_h(np.concatenate([g, ones])[None, :]).ravel()
    want = np.array([swiglu_exact(int(b), 0x3F80) for b in g], np.float32)
    bad = f32_bits(h) != f32_bits(want)
    assert not bad.any(), [(hex(int(b)), float(x), float(y)) for b, x, y in zip(g[bad], h[bad], want[bad])][:5]


def test_sampled_gate_and_up_values(orc):
    """The last rounding, RN32(s_g * u), on a seeded sample of gate values times
    up values of several magnitudes (subnormal and overflowing products included)."""
    rng = np.random.default_rng(11)
    g = rng.choice(finite_bf16_patterns(), 3000)
    for ub in (0xBFC0, 0x3FAB, 0x0075, 0x4B37, 0x7E80, 0xC2F7):   # -1.5, 1.336, subnormal, 1.2e7, 8.5e37, -123.5
        u = np.full_like(g, ub)
        h = orc.swiglu_h(np.concatenate([g, u])[None, :]).ravel()
        want = np.array([swiglu_exact(int(b), ub) for b in g], np.float32)
        bad = f32_bits(h) != f32_bits(want)
        assert not bad.any(), (hex(ub), [(hex(int(b)), float(x), float(y)) for b, x, y in
                                         zip(g[bad], h[bad], want[bad])][:5])


def test_a_planted_reordering_is_caught():
    """The pin is sensitive to the order of roundings: multiplying g by RN32(1 / t)
    instead of dividing by t changes s_g for some bf16 gate values."""
    diffs = 0
    for b in finite_bf16_patterns()[::7]:
        g = float(np.uint32(int(b) << 16).view(np.float32))
        E = exp_neg_rn32(g)
        if np.isinf(E) or g == 0.0:
            continue
        t = rn32(1 + Fraction(E))
        diffs += rn32(Fraction(g) / Fraction(t)) != rn32(Fraction(g) * Fraction(rn32(1 / Fraction(t))))
    assert diffs > 0
