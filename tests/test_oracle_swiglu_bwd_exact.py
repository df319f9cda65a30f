"""The oracle's SwiGLU backward evaluated exactly, one rounding at a time.

The backward reading takes the textbook derivative of h = silu(g) * u with
sigma = 1 / (1 + e^-g) and silu'(g) = sigma * (1 + g * (1 - sigma)) as single
binary32 operations in a fixed order ("LLMQ: Efficient Lower-Precision
Pretraining for Consumer GPUs", section 3.1, the SwiGLU block and its
recomputation; section 5 / Figure 2, E5M2 gradients):

    E = RN32(e^-g),  t = RN32(1 + E),  sig = RN32(1 / t),  s = RN32(g / t)
    c = RN32(1 - sig),  p = RN32(g * c),  q = RN32(1 + p),  ds = RN32(sig * q)
    du = RN32(d * s),   dg = RN32(RN32(d * u) * ds)

Every step is recomputed here from its definition with the tests' exact
binary32 helpers (``exact_f32``: rationals, one rounding per operation, IEEE
signed zeros and infinities), and the oracle's gradient must equal it bit for
bit: for every finite bf16 gate value with u = d = 1 (so dg = silu'(g) and
du = silu(g)), and for a seeded sample of gate values under several (u, d)
pairs (the last two roundings).  The float64 pins elsewhere bound the same
function only within a few ulps; these catch a changed rounding order
(sig + sig * p for sig * q, d * (u * ds) for (d * u) * ds, g * RN32(1 / t) for
g / t), which stays inside such a bound.
"""
import numpy as np

import oracle
from exact_f32 import add, bf16_value, div, exp_neg_rn32, f32_bits, finite_bf16_patterns, mul, sub


def grad_exact(g: float, u: float, d: float):
    E = exp_neg_rn32(g)
    t = add(1.0, E)
    sig = div(1.0, t)
    s = div(g, t)
    c = sub(1.0, sig)
    p = mul(g, c)
    q = add(1.0, p)
    ds = mul(sig, q)
    return mul(mul(d, u), ds), mul(d, s)


def oracle_grad(gbits, ubits, dbits):
    n = len(gbits)
    gu = np.empty((n, 2), np.uint16)
    gu[:, 0] = gbits
    gu[:, 1] = ubits
    dh = np.asarray(dbits, np.uint16).reshape(n, 1)
    out = oracle.swiglu_grad(gu, dh)
    return out[:, 0], out[:, 1]


def check(gbits, ubits, dbits, what):
    dg, du = oracle_grad(gbits, ubits, dbits)
    want = [grad_exact(bf16_value(g), bf16_value(u), bf16_value(d)) for g, u, d in zip(gbits, ubits, dbits)]
    wdg = np.array([w[0] for w in want], np.float32)
    wdu = np.array([w[1] for w in want], np.float32)
    for got, exp, name in ((dg, wdg, "dg"), (du, wdu, "du")):
        bad = (f32_bits(got) != f32_bits(exp)) & ~(np.isnan(got) & np.isnan(exp))
        assert not bad.any(), (what, name, [(hex(int(g)), float(x), float(y))
                                            for g, x, y in zip(np.asarray(gbits)[bad], got[bad], exp[bad])][:5])


def test_every_gate_value():
    """dg = silu'(g) and du = silu(g) (u = d = 1) for every finite bf16 gate value."""
    g = finite_bf16_patterns()
    ones = np.full_like(g, 0x3F80)
    check(g, ones, ones, "u = d = 1")


def test_sampled_gate_values_with_up_and_gradient():
    """The last two roundings, on a seeded sample of gate values under (u, d)
    pairs of several magnitudes (subnormal and overflowing products included)."""
    rng = np.random.default_rng(23)
    g = rng.choice(finite_bf16_patterns(), 2000)
    for ub, db in ((0xBFC0, 0x3A83), (0x3FAB, 0xC2F7), (0x0075, 0x4B37), (0x7E80, 0x3F81), (0xC3A1, 0x0101)):
        check(g, np.full_like(g, ub), np.full_like(g, db), f"u {hex(ub)} d {hex(db)}")


def test_the_pin_sees_a_changed_rounding_order():
    """Three plausible slips change some of these bits: silu' as sig + sig * p,
    dg as d * (u * ds), and s as g * RN32(1 / t)."""
    gs = [bf16_value(b) for b in finite_bf16_patterns()[::5]]
    n1 = n2 = n3 = 0
    for g in gs:
        E = exp_neg_rn32(g)
        t = add(1.0, E)
        sig = div(1.0, t)
        c = sub(1.0, sig)
        p = mul(g, c)
        ds = mul(sig, add(1.0, p))
        n1 += f32_bits(ds) != f32_bits(add(sig, mul(sig, p)))
        n3 += f32_bits(div(g, t)) != f32_bits(mul(g, div(1.0, t)))
    u, d = bf16_value(0x3FAB), bf16_value(0xBF9D)
    for g in gs[::4]:
        E = exp_neg_rn32(g)
        t = add(1.0, E)
        sig = div(1.0, t)
        ds = mul(sig, add(1.0, mul(g, sub(1.0, sig))))
        n2 += f32_bits(mul(mul(d, u), ds)) != f32_bits(mul(d, mul(u, ds)))
    assert n1 > 0 and n2 > 0 and n3 > 0, (n1, n2, n3)
