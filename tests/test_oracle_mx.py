"""Pins of the oracle's block (MX) scaling against things other than itself.

The reading (OCP Microscaling formats v1.0, section 6.3; the LLMQ summary's
section 2 only names block scaling as the alternative that needs hardware
support): blocks of 32 consecutive elements of a row, scale 2^e with
e = floor(log2 max|x|) - emax (8 for E4M3, 15 for E5M2) clamped to [-127, 127]
and stored as the E8M0 byte e + 127, elements x / 2^e encoded nearest-even
with saturation.

* quantise: closed forms for e at every power of two and just below it; a
  round trip of codes and scales built from random codes (a wrong emax, floor,
  sign or block index breaks it); saturation of the block maximum; zero, tiny,
  NaN and infinite blocks; a brute-force nearest-code search over the torch
  decoder's values for random blocks;
* GEMM: with uniform scales it equals the per-tensor GEMM (itself pinned) with
  the descale 2^(ea + eb), bit for bit; with per-block scales it stays within
  the fp32 summation bound of a float64 product of the torch-decoded,
  scaled operands; a swapped block scale is caught; a NaN scale poisons
  exactly the outputs that use it.
"""
import math

import numpy as np
import pytest
import torch

from oracle import E4M3, E5M2

TORCH_DT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}
EMAX = {E4M3: 8, E5M2: 15}
MAXV = {E4M3: 448.0, E5M2: 57344.0}
MAXCODE = {E4M3: 0x7E, E5M2: 0x7B}


def tdecode(c, fmt):
    return torch.from_numpy(np.ascontiguousarray(c)).view(TORCH_DT[fmt]).to(torch.float32).numpy()


def bf16_bits(x):
    """float values exactly representable in bf16 -> bf16 bit patterns."""
    b = np.asarray(x, np.float32).view(np.uint32)
    assert np.all(b & 0xFFFF == 0), "value not representable in bf16"
    return (b >> 16).astype(np.uint16)


def bits_f32(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_scale_closed_form(orc, fmt):
    """max |x| = 2^k and (2 - 2^-7) 2^k give e = k - emax; 2^k - ulp gives k - 1 - emax."""
    ks = list(range(-110, 120, 7))
    rows = []
    for k in ks:
        for top in (2.0 ** k, (2.0 - 2.0 ** -7) * 2.0 ** k, (1.0 - 2.0 ** -8) * 2.0 ** k):
            row = np.full(32, 2.0 ** (k - 3), np.float64)
            row[5] = -top                     # the maximum magnitude, negative
            rows.append(row)
    x = bf16_bits(np.array(rows))
    q, s = orc.mx_quantize(x, fmt)
    for i, k in enumerate(ks):
        want = [k - EMAX[fmt], k - EMAX[fmt], k - 1 - EMAX[fmt]]
        for j in range(3):
            e = max(-127, min(127, want[j]))
            assert int(s[3 * i + j, 0]) == e + 127, (k, j, int(s[3 * i + j, 0]), e)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_round_trip_codes_and_scales(orc, fmt):
    """Blocks built as dec(c) * 2^e with one code in the top binade come back exactly."""
    rng = np.random.default_rng(7 + fmt)
    rows, nb = 64, 6
    vals = tdecode(np.arange(256, dtype=np.uint8), fmt).astype(np.float64)
    finite = [c for c in range(256) if np.isfinite(vals[c])]
    top = [c for c in finite if 2.0 ** EMAX[fmt] <= abs(vals[c]) <= MAXV[fmt]]
    codes = rng.choice(finite, size=(rows, nb * 32)).astype(np.uint8)
    e = rng.integers(-100, 100, size=(rows, nb))
    for i in range(rows):
        for b in range(nb):
            codes[i, b * 32 + rng.integers(0, 32)] = rng.choice(top)
    x = np.empty(codes.shape, np.float64)
    for b in range(nb):
        x[:, b * 32:(b + 1) * 32] = vals[codes[:, b * 32:(b + 1) * 32]] * np.exp2(e[:, b:b + 1].astype(np.float64))
    q, s = orc.mx_quantize(bf16_bits(x), fmt)
    assert np.array_equal(s.astype(np.int64), e + 127)
    # +0 and -0 both round-trip (the codes 0x00 and 0x80 are distinct values' signs)
    assert np.array_equal(q, codes)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_saturation_of_the_block_maximum(orc, fmt):
    """max = 1.9375 * 2^k scales to 1.9375 * 2^emax > max normal: saturates, sign kept."""
    k = 3
    row = np.full(32, 0.5, np.float64)
    row[0], row[1] = 1.9375 * 2.0 ** k, -1.9375 * 2.0 ** k
    q, s = orc.mx_quantize(bf16_bits(row[None, :]), fmt)
    assert int(s[0, 0]) == k - EMAX[fmt] + 127
    assert q[0, 0] == MAXCODE[fmt] and q[0, 1] == 0x80 | MAXCODE[fmt]
    # 0.5 / 2^(k - emax) = 2^(emax - 4): exact, a power of two
    assert tdecode(q[0, 2:3], fmt)[0] == 2.0 ** (EMAX[fmt] - 4)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_special_blocks(orc, fmt):
    z = np.zeros((1, 32), np.float64)
    z[0, 3] = -0.0
    q, s = orc.mx_quantize(bf16_bits(z), fmt)
    assert s[0, 0] == 0 and q[0, 3] == 0x80 and np.all(np.delete(q[0], 3) == 0)
    # a tiny block: e clamps at -127, the elements scale by 2^127 exactly
    t = np.full((1, 32), 2.0 ** -130, np.float64)
    q, s = orc.mx_quantize(bf16_bits(t), fmt)
    assert s[0, 0] == 0 and np.all(tdecode(q[0], fmt) == 2.0 ** -3)
    for bad in (np.nan, np.inf, -np.inf):
        r = np.full((2, 64), 1.5, np.float32)
        r[1, 40] = bad                         # second block of row 1 only
        q, s = orc.mx_quantize(bf16_bits(r), fmt)
        assert s[1, 1] == 255 and s[0, 0] == s[0, 1] == s[1, 0] == 127 - EMAX[fmt]
        dec = tdecode(q[1, 32:], fmt)
        assert dec[0] == 1.5                   # the unscaled encoding
        if bad != bad:
            assert np.isnan(dec[8])
        else:
            assert abs(dec[8]) == MAXV[fmt] and np.sign(dec[8]) == np.sign(bad)


def brute_force_code(v, fmt, vals):
    """Nearest finite code to v (ties to the even mantissa), saturating, sign of v."""
    mag = abs(v)
    best, bd = None, None
    for c in range(128):
        cv = vals[c]
        if not np.isfinite(cv):
            continue
        d = abs(cv - min(mag, MAXV[fmt]))
        if bd is None or d < bd or (d == bd and c % 2 == 0):
            best, bd = c, d
    return best | (0x80 if math.copysign(1.0, v) < 0 else 0)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_brute_force_blocks(orc, fmt):
    rng = np.random.default_rng(11 + fmt)
    vals = tdecode(np.arange(256, dtype=np.uint8), fmt).astype(np.float64)
    x = (rng.standard_normal((6, 64)) * np.exp2(rng.integers(-20, 20, (6, 1)))).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)          # truncation: any bf16 values will do
    xf = bits_f32(xb).astype(np.float64)
    q, s = orc.mx_quantize(xb, fmt)
    for i in range(6):
        for b in range(2):
            blk = xf[i, b * 32:(b + 1) * 32]
            m = np.max(np.abs(blk))
            e = max(-127, min(127, math.frexp(m)[1] - 1 - EMAX[fmt]))
            assert int(s[i, b]) == e + 127
            for k in range(32):
                assert q[i, b * 32 + k] == brute_force_code(blk[k] / 2.0 ** e, fmt, vals), (i, b, k)


def random_codes(rng, shape, fmt, sigma):
    x = (rng.standard_normal(shape) * sigma).astype(np.float32)
    return torch.from_numpy(x).to(TORCH_DT[fmt]).view(torch.uint8).numpy()


@pytest.mark.parametrize("fa", [E4M3, E5M2])
def test_gemm_uniform_scales_equal_per_tensor_gemm(orc, fa):
    rng = np.random.default_rng(3 + fa)
    M, N, K = 24, 40, 256
    a, b = random_codes(rng, (M, K), fa, 20.0), random_codes(rng, (N, K), E4M3, 20.0)
    for ea, eb in ((0, 0), (-9, -4), (5, -20), (13, 2)):
        sa = np.full((M, K // 32), ea + 127, np.uint8)
        sb = np.full((N, K // 32), eb + 127, np.uint8)
        y = orc.mx_gemm(a, sa, fa, b, sb, E4M3)
        ref = orc.gemm(a, fa, b, E4M3, np.float32(2.0 ** ea), np.float32(2.0 ** eb))
        assert np.array_equal(y, ref), (ea, eb)


def test_gemm_block_scales_within_bound(orc):
    rng = np.random.default_rng(5)
    M, N, K = 20, 36, 384
    a, b = random_codes(rng, (M, K), E4M3, 30.0), random_codes(rng, (N, K), E4M3, 30.0)
    sa = rng.integers(117, 137, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(117, 137, (N, K // 32)).astype(np.uint8)
    y = bits_f32(orc.mx_gemm(a, sa, E4M3, b, sb, E4M3)).astype(np.float64)
    ad = tdecode(a, E4M3).astype(np.float64) * np.exp2(np.repeat(sa.astype(np.float64) - 127, 32, axis=1))
    bd = tdecode(b, E4M3).astype(np.float64) * np.exp2(np.repeat(sb.astype(np.float64) - 127, 32, axis=1))
    ref = ad @ bd.T
    bound = np.abs(ad) @ np.abs(bd).T * K * 2.0 ** -24 + np.abs(ref) * 2.0 ** -8 + 1e-30
    assert np.all(np.abs(y - ref) <= bound)
    # a transposed block-scale layout (scales of the wrong K block) is caught
    swapped = sa.copy()
    swapped[:, [0, 1]] = swapped[:, [1, 0]]
    if not np.array_equal(swapped, sa):
        y2 = bits_f32(orc.mx_gemm(a, swapped, E4M3, b, sb, E4M3)).astype(np.float64)
        assert np.linalg.norm(y2 - ref) / np.linalg.norm(ref) > 1e-2


def test_gemm_nan_scale(orc):
    rng = np.random.default_rng(9)
    M, N, K = 8, 16, 128
    a, b = random_codes(rng, (M, K), E4M3, 10.0), random_codes(rng, (N, K), E4M3, 10.0)
    sa = np.full((M, 4), 127, np.uint8)
    sb = np.full((N, 4), 127, np.uint8)
    sa[2, 1] = 255
    sb[5, 3] = 255
    y = bits_f32(orc.mx_gemm(a, sa, E4M3, b, sb, E4M3))
    nan = np.isnan(y)
    want = np.zeros((M, N), bool)
    want[2, :] = True
    want[:, 5] = True
    assert np.array_equal(nan, want)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_f32_blocks_equal_bf16_blocks_on_bf16_values(orc, fmt):
    """The fp32 form of the rule gives the bf16 form's codes and scales on bf16 values."""
    rng = np.random.default_rng(21 + fmt)
    x = (rng.standard_normal((16, 256)) * np.exp2(rng.integers(-30, 30, (16, 1)))).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    q1, s1 = orc.mx_quantize(xb, fmt)
    q2, s2 = orc.mx_quantize_f32(bits_f32(xb).astype(np.float32), fmt)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_f32_blocks_brute_force(orc, fmt):
    """fp32 values with full 24-bit significands, maxima just below powers of two
    (2^k (1 - 2^-24): e = k - 1 - emax) and fp32 subnormal maxima (clamped scale)."""
    rng = np.random.default_rng(33 + fmt)
    vals = tdecode(np.arange(256, dtype=np.uint8), fmt).astype(np.float64)
    x = (rng.standard_normal((6, 64)) * np.exp2(rng.integers(-20, 20, (6, 1)))).astype(np.float32)
    x[0, 3] = np.float32(2.0 ** 5 * (1 - 2.0 ** -24))
    x[1, :32] = np.float32(2.0 ** -140) * np.arange(1, 33, dtype=np.float32)
    q, s = orc.mx_quantize_f32(x, fmt)
    for i in range(6):
        for b in range(2):
            blk = x[i, b * 32:(b + 1) * 32].astype(np.float64)
            m = np.max(np.abs(blk))
            e = -127 if m == 0 else max(-127, min(127, math.frexp(m)[1] - 1 - EMAX[fmt]))
            assert int(s[i, b]) == e + 127, (i, b)
            for k in range(32):
                scaled = float(np.float32(blk[k] * 2.0 ** -e))       # RN32 of the exact quotient
                assert q[i, b * 32 + k] == brute_force_code(scaled, fmt, vals), (i, b, k)
    assert int(s[0, 0]) == 4 - EMAX[fmt] + 127


def test_mx_swiglu_is_mx_of_swiglu_h(orc):
    """The MX SwiGLU requant is the (pinned) SwiGLU output h put through the (pinned)
    fp32 block rule, for drawn and for hand-picked gate/up values."""
    rng = np.random.default_rng(41)
    M, F = 8, 128
    g = (rng.standard_normal((M, F)) * 3).astype(np.float32)
    u = (rng.standard_normal((M, F)) * np.exp2(rng.integers(-8, 8, (M, 1)))).astype(np.float32)
    g[0, :4] = [0.0, -np.inf, 200.0, -200.0]
    u[1, 5] = np.inf
    gu = np.concatenate([(g.view(np.uint32) >> 16), (u.view(np.uint32) >> 16)], axis=1).astype(np.uint16)
    hq, sc = orc.mx_swiglu(gu)
    h = orc.swiglu_h(gu)
    q2, s2 = orc.mx_quantize_f32(np.ascontiguousarray(h, dtype=np.float32), E4M3)
    assert np.array_equal(hq, q2) and np.array_equal(sc, s2)
    assert sc[0, 0] == 255 and sc[1, 0] == 255            # the -inf gate (NaN h) and the infinite up
