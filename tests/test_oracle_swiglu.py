"""Pins of the oracle's SwiGLU requantisation.

* e^-g, exhaustively over every finite bf16 g, against Python ``decimal`` at 60
  digits rounded to the nearest fp32 (a correctly rounded exponential);
* h = silu(g) * u against a float64 evaluation of g / (1 + e^-g) * u, within a
  few fp32 ulps (catches a wrong sign, operand or term);
* closed forms at g = 0, large positive g (silu(g) = g) and large negative g;
* the [gate | up] layout;
* absmax_h = max |h| and hq = torch's float8 cast of RN32(h * s_h);
* the recomputation invariant of "LLMQ: Efficient Lower-Precision Pretraining
  for Consumer GPUs", section 3.1: with the retained absmax statistic the
  requantised bytes equal the forward's, with no second reduction.
"""
import decimal

import numpy as np
import pytest
import torch

from oracle import E4M3

decimal.getcontext().prec = 60


def bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


def correctly_rounded_f32(d: decimal.Decimal) -> np.float32:
    """Nearest fp32 to the (irrational) value d > 0, found by exact comparison."""
    top = decimal.Decimal(2) ** 128 - decimal.Decimal(2) ** 103   # rounds to inf at/above
    if d >= top:
        return np.float32(np.inf)
    f = np.float32(float(d))
    best, bestd = None, None
    for c in (np.nextafter(f, np.float32(0)), f, np.nextafter(f, np.float32(np.inf))):
        if not np.isfinite(c):
            continue
        dist = abs(decimal.Decimal(float(c)) - d)
        if bestd is None or dist < bestd:
            best, bestd = c, dist
    return np.float32(best)


@pytest.mark.slow
def test_exp_neg_exhaustive_vs_decimal(orc):
    g = bits_to_f32(np.arange(65536, dtype=np.uint32).astype(np.uint16))
    g = g[np.isfinite(g)]
    got = orc.exp_neg(g)
    for gi, e in zip(g, got):
        # outside [-100, 110] the result is far beyond fp32 range: e^100 > FLT_MAX
        # (ln FLT_MAX = 88.72) and e^-110 < 2^-151 (half the smallest subnormal)
        if gi < -100:
            want = np.float32(np.inf)
        elif gi > 110:
            want = np.float32(0.0)
        else:
            want = correctly_rounded_f32((-decimal.Decimal(float(gi))).exp())
        assert e == want, (float(gi), float(e), float(want))


def test_silu_times_u_near_float64(orc):
    rng = np.random.default_rng(5)
    M, F = 64, 512
    gate = rng.standard_normal((M, F)) * 4
    up = rng.standard_normal((M, F))
    gu = bf16_bits(np.concatenate([gate, up], axis=1))
    h = orc.swiglu_h(gu)
    g64 = bits_to_f32(gu[:, :F]).astype(np.float64)
    u64 = bits_to_f32(gu[:, F:]).astype(np.float64)
    ref = g64 / (1.0 + np.exp(-g64)) * u64
    err = np.abs(h.astype(np.float64) - ref)
    tol = 4 * 2.0 ** -24 * np.abs(ref) + 1e-44
    assert np.all(err <= tol)


def test_closed_forms_and_layout(orc):
    F = 16
    gate = np.zeros((4, F), np.float32)
    up = np.zeros((4, F), np.float32)
    gate[0], up[0] = 0.0, 3.0                  # silu(0) = 0
    gate[1], up[1] = 40.0, np.arange(F)        # e^-40 < 2^-24: 1 + E = 1, silu = g
    gate[2], up[2] = -200.0, 1.0               # e^200 overflows: silu = g / inf = -0
    gate[3], up[3] = 2.0 ** -40, 1.0           # tiny g: 1 + E = 2, silu = g / 2
    h = orc.swiglu_h(bf16_bits(np.concatenate([gate, up], axis=1)))
    assert np.all(h[0] == 0.0)
    assert np.array_equal(h[1], (40.0 * np.arange(F)).astype(np.float32))
    assert np.all(h[2] == 0.0) and np.all(np.signbit(h[2]))
    assert np.all(h[3] == np.float32(2.0 ** -41))
    # swapping the halves changes the result: gate really is the first half
    h_sw = orc.swiglu_h(bf16_bits(np.concatenate([up, gate], axis=1)))
    assert not np.array_equal(h_sw[1], h[1])


@pytest.mark.parametrize("M,F", [(1, 16), (32, 48), (100, 256)])
def test_requant_forward_and_recompute(orc, M, F):
    rng = np.random.default_rng(M * 1000 + F)
    gu = bf16_bits(rng.standard_normal((M, 2 * F)) * 3)
    h = orc.swiglu_h(gu)
    hq, hqt, am, inv = orc.swiglu_requant(gu, want_hqt=True)
    assert am == np.max(np.abs(h))
    s, inv2 = orc.scale(am, E4M3)
    assert inv == inv2
    ref = torch.from_numpy((h * s).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(hq, ref)
    assert np.array_equal(hqt, hq.T)
    # recomputation with the retained statistic: identical bytes
    hq2, hqt2, am2, inv3 = orc.swiglu_requant(gu, absmax_h=am, want_hqt=True)
    assert am2 == am and inv3 == inv
    assert np.array_equal(hq2, hq) and np.array_equal(hqt2, hqt)


def test_requant_with_stale_statistic_saturates(orc):
    rng = np.random.default_rng(9)
    gu = bf16_bits(rng.standard_normal((8, 64)) * 3)
    h = orc.swiglu_h(gu)
    stale = np.float32(np.max(np.abs(h)) / 4)
    hq, _, _, _ = orc.swiglu_requant(gu, absmax_h=stale)
    big = np.abs(h) * orc.scale(stale, E4M3)[0] > 448
    assert big.any()
    assert np.all((hq[big] & 0x7F) == 0x7E)


def test_tiny_gate_rule_holds_through_exponent_102(orc):
    """For every bf16 gate value whose biased exponent is at most 102 (both
    signs, every mantissa, zeros and subnormals), 1 + e^-g rounds to exactly 2
    and s_g = g / 2; at exponent 103 it does not for every value.  The GEMM
    epilogue that takes the SwiGLU statistic relies on the first fact to hold
    its s_g table in 31 KB (exponents 103..133).  Why: for |g| < 2^-24,
    RN32(e^-g) is 1 (g < 0, or 0 <= g <= 2^-25) or 1 - 2^-24 (2^-25 < g <
    2^-24); 1 + 1 = 2, and 2 - 2^-24 is the midpoint of 2 - 2^-23 and 2,
    which rounds to the even 2.  The check below is exhaustive."""
    bits = np.array([(s << 15) | (e << 7) | m for s in (0, 1) for e in range(0, 103) for m in range(128)],
                    np.uint16)
    one = np.full_like(bits, 0x3F80)                                  # u = 1: h = s_g
    h = orc.swiglu_h(np.concatenate([bits, one])[None, :]).ravel()
    g = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(h.view(np.uint32), (g * np.float32(0.5)).astype(np.float32).view(np.uint32))
    b103 = np.array([(s << 15) | (103 << 7) | m for s in (0, 1) for m in range(128)], np.uint16)
    h103 = orc.swiglu_h(np.concatenate([b103, np.full_like(b103, 0x3F80)])[None, :]).ravel()
    g103 = (b103.astype(np.uint32) << 16).view(np.float32)
    assert not np.array_equal(h103.view(np.uint32), (g103 * np.float32(0.5)).view(np.uint32))
