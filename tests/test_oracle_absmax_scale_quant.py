"""Pins of the oracle's absmax, scale and quantise steps.

* absmax: numpy's max(|x|) on random data with a planted maximum; NaN and
  infinity surface; all-zero input.
* scale: exhaustive over every positive finite bf16 absmax, the fp32 division
  equals the float64 quotient rounded once to fp32 (a correctly rounded
  quotient); the zero and overflow rules.
* the FastML report's "no value clipping" property of just-in-time absmax
  scaling: with a fresh absmax the element that holds it encodes to exactly
  +-max, for every bf16 absmax whose scale does not overflow, in both formats.
* quantise: torch's CPU float8 cast of the fp32 product (an independent
  encoder) and the transposed copy.
"""
import numpy as np
import pytest
import torch

from oracle import E4M3, E5M2

TORCH_DT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}
MAXV = {E4M3: 448.0, E5M2: 57344.0}
MAXCODE = {E4M3: 0x7E, E5M2: 0x7B}


def bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


def test_absmax_planted(orc):
    rng = np.random.default_rng(0)
    for n in [1, 7, 1000, 123457]:
        x = bf16_bits(rng.standard_normal(n))
        pos = rng.integers(n)
        x[pos] = bf16_bits(np.array([-1234.0]))[0]
        got = orc.absmax_bf16(x)
        assert got == np.float32(1232.0) or got == np.float32(1234.0)
        assert got == np.max(np.abs(bits_to_f32(x)))


def test_absmax_special(orc):
    x = bf16_bits(np.zeros(100))
    assert orc.absmax_bf16(x) == 0.0
    x[3] = 0x8000  # -0
    assert orc.absmax_bf16(x) == 0.0
    x[5] = 0xFF80  # -inf
    assert np.isposinf(orc.absmax_bf16(x))
    x[7] = 0x7FC1  # NaN
    assert np.isnan(orc.absmax_bf16(x))
    f = np.array([1.0, -3.0, 2.5e-40, -7.0], np.float32)
    assert orc.absmax_f32(f) == 7.0
    f[1] = np.nan
    assert np.isnan(orc.absmax_f32(f))
    with pytest.raises(ValueError):
        orc.absmax_bf16(np.zeros(0, np.uint16))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_scale_exhaustive_over_bf16(orc, fmt):
    bits = np.arange(1, 0x7F80, dtype=np.uint16)        # every positive finite bf16
    a = bits_to_f32(bits)
    s = np.empty_like(a)
    inv = np.empty_like(a)
    for i, v in enumerate(a):
        s[i], inv[i] = orc.scale(v, fmt)
    with np.errstate(over="ignore"):
        want = (MAXV[fmt] / a.astype(np.float64)).astype(np.float32)
    want[np.isinf(want)] = np.finfo(np.float32).max
    assert np.array_equal(s, want)
    want_inv = (1.0 / s.astype(np.float64)).astype(np.float32)
    assert np.array_equal(inv, want_inv)


def test_scale_special(orc):
    assert orc.scale(0.0, E4M3) == (1.0, 1.0)
    s, inv = orc.scale(1e-38, E4M3)
    assert s == np.finfo(np.float32).max
    s, inv = orc.scale(np.inf, E4M3)
    assert s == 0.0 and np.isposinf(inv)
    s, inv = orc.scale(np.nan, E5M2)
    assert np.isnan(s) and np.isnan(inv)
    assert orc.scale(448.0, E4M3) == (1.0, 1.0)
    assert orc.scale(2.0, E5M2) == (28672.0, np.float32(1.0 / 28672.0))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_no_clipping_with_fresh_absmax(orc, fmt):
    """The absmax element lands on +-max and nothing saturates (FastML report)."""
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    a = bits_to_f32(bits)
    codes = np.empty(a.size, np.uint8)
    clamped = np.zeros(a.size, bool)
    prods = np.empty(a.size, np.float32)
    for i, v in enumerate(a):
        s, _ = orc.scale(v, fmt)
        clamped[i] = s == np.finfo(np.float32).max
        prods[i] = v * s
        codes[i] = orc.encode(np.array([prods[i]], np.float32), fmt)[0]
    assert np.all(codes[~clamped] == MAXCODE[fmt])
    # absmax below ~1e-36 overflows the scale, which is then held at FLT_MAX (the
    # reading taken for that unspecified case): the product stays below max, so
    # nothing is clipped there either.
    assert clamped.sum() < 2000 and np.all(prods[clamped] < MAXV[fmt])
    assert np.all(orc.decode(codes[clamped], fmt) <= MAXV[fmt])


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("shape", [(1, 16), (5, 48), (64, 64), (130, 272)])
def test_quantize_matches_torch_cast(orc, fmt, shape):
    rng = np.random.default_rng(sum(shape) + fmt)
    x = bf16_bits(rng.standard_normal(shape) * (0.02 if fmt == E4M3 else 1e-3))
    am = orc.absmax_bf16(x)
    s, inv = orc.scale(am, fmt)
    q, qt = orc.quantize(x, fmt, s, want_q=True, want_qt=True)
    prod = (bits_to_f32(x) * s).astype(np.float32)
    ref = torch.from_numpy(prod).to(TORCH_DT[fmt]).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)
    assert np.array_equal(qt, q.T)
    assert q.max() <= 0xFE
    # the absmax element maps to +-max
    flat = np.abs(bits_to_f32(x)).reshape(-1)
    i = int(np.argmax(flat))
    assert (q.reshape(-1)[i] & 0x7F) == MAXCODE[fmt]


def test_quantize_optional_outputs(orc):
    x = bf16_bits(np.linspace(-3, 3, 32 * 16).reshape(32, 16))
    q, qt = orc.quantize(x, E4M3, np.float32(10.0), want_q=False, want_qt=True)
    assert q is None and qt.shape == (16, 32)
    q2, _ = orc.quantize(x, E4M3, np.float32(10.0))
    assert np.array_equal(qt, q2.T)
