"""Pins of the oracle's OFP8 encoder/decoder against things other than itself.

* decode: torch's CPU float8 dtypes (an independent implementation) for all 256
  codes, and the special values tabulated by the OFP8 specification
  (tests/golden/ofp8_special_values.txt);
* encode: brute-force nearest-code search over all 256 torch-decoded values,
  for every bf16 input and for fp32 products x*s at several scales, with ties
  to the even code and saturation beyond max; hand-worked rounding cases
  (tests/golden/ofp8_rounding_cases.txt); round trip; the saturation bound;
  torch's (non-saturating, RNE) cast inside the range where it does not
  overflow.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import E4M3, E5M2

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TORCH_DT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}
MAXV = {E4M3: 448.0, E5M2: 57344.0}
FMT_NAME = {"e4m3": E4M3, "e5m2": E5M2}


def torch_decode_all(fmt):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(TORCH_DT[fmt]).to(torch.float32).numpy()


def all_bf16_as_f32():
    return (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)


def parse_value(tok):
    tok = tok.strip()
    if tok in ("nan", "inf", "-inf"):
        return float(tok)
    if "2^" in tok:
        sign = -1.0 if tok.startswith("-") else 1.0
        tok = tok.lstrip("-")
        if "*" in tok:
            mul, p = tok.split("*")
            return sign * float(mul) * 2.0 ** int(p.split("^")[1])
        return sign * 2.0 ** int(tok.split("^")[1])
    return float(tok)


def brute_force_encode(v, fmt):
    """Nearest code by exhaustive search over the 128 non-negative codes.

    Ties go to the even code (even mantissa LSB), |v| > max saturates to max,
    NaN maps to the format's NaN code with v's sign, the sign bit is v's.
    Distances are float64; for the two neighbours of v they are exact.
    """
    vals = torch_decode_all(fmt)[:128].astype(np.float64)
    finite = np.isfinite(vals) & (vals <= MAXV[fmt])
    cand_codes = np.nonzero(finite)[0]
    cand = vals[cand_codes]
    v = np.asarray(v, np.float32)
    sign = ((v.view(np.uint32) >> 24) & 0x80).astype(np.uint8)
    a = np.abs(v.astype(np.float64))
    out = np.empty(v.shape, np.uint8)
    chunk = 1 << 16
    for s in range(0, v.size, chunk):
        aa = a.reshape(-1)[s:s + chunk]
        d = np.abs(aa[:, None] - cand[None, :])
        dmin = d.min(axis=1, keepdims=True)
        is_min = d == dmin
        # among the nearest, prefer the even code
        even = (cand_codes[None, :] & 1) == 0
        pick_even = is_min & even
        has_even = pick_even.any(axis=1)
        idx = np.where(has_even, pick_even.argmax(axis=1), is_min.argmax(axis=1))
        code = cand_codes[idx].astype(np.uint8)
        big = aa > MAXV[fmt]
        code[big] = np.uint8(0x7E if fmt == E4M3 else 0x7B)
        code[np.isnan(aa)] = np.uint8(0x7F)
        out.reshape(-1)[s:s + chunk] = code
    return out | sign


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_decode_matches_torch_all_codes(orc, fmt):
    codes = np.arange(256, dtype=np.uint8)
    mine = orc.decode(codes, fmt)
    ref = torch_decode_all(fmt)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    # signed zeros too
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def test_decode_special_values_from_spec_table(orc):
    n = 0
    for line in open(os.path.join(GOLDEN, "ofp8_special_values.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        name, code, value = line.split()
        fmt = FMT_NAME[name]
        got = float(orc.decode(np.array([int(code, 16)], np.uint8), fmt)[0])
        want = parse_value(value)
        if math.isnan(want):
            assert math.isnan(got), (name, code)
        else:
            assert got == want, (name, code, got, want)
            neg = float(orc.decode(np.array([int(code, 16) | 0x80], np.uint8), fmt)[0])
            assert neg == -want
        n += 1
    assert n >= 15


def test_encode_hand_worked_cases(orc):
    n = 0
    for line in open(os.path.join(GOLDEN, "ofp8_rounding_cases.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        name, value, code = line.split()[:3]
        fmt = FMT_NAME[name]
        got = int(orc.encode(np.array([parse_value(value)], np.float32), fmt)[0])
        assert got == int(code, 16), (name, value, hex(got), code)
        n += 1
    assert n >= 20


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_brute_force_all_bf16(orc, fmt):
    v = all_bf16_as_f32()
    got = orc.encode(v, fmt)
    want = brute_force_encode(v, fmt)
    nan = np.isnan(v)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all((got[nan] & 0x7F) == 0x7F)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_brute_force_scaled_products(orc, fmt):
    """Every finite bf16 x times assorted fp32 scales, product rounded to fp32 first."""
    x = all_bf16_as_f32()
    x = x[np.isfinite(x)]
    rng = np.random.default_rng(123)
    scales = [np.float32(1.0), np.float32(448.0 / 3.1875), np.float32(57344.0 / 0.0078125),
              np.float32(rng.uniform(0.5, 2.0)), np.float32(rng.uniform(1e3, 1e5)),
              np.float32(3.0e-3)]
    for s in scales:
        p = (x * s).astype(np.float32)   # IEEE fp32 multiply
        with np.errstate(invalid="ignore"):
            sel = np.isfinite(p)
        p = p[sel]
        got = orc.encode(p, fmt)
        want = brute_force_encode(p, fmt)
        assert np.array_equal(got, want), float(s)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_round_trip_identity(orc, fmt):
    codes = np.arange(256, dtype=np.uint8)
    vals = orc.decode(codes, fmt)
    keep = ~np.isnan(vals) & ~np.isinf(vals)
    back = orc.encode(vals[keep], fmt)
    assert np.array_equal(back, codes[keep])


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_saturation_bound(orc, fmt):
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32) * np.float32(10 ** e)
                        for e in range(-8, 9)])
    v = np.concatenate([v, np.array([np.inf, -np.inf, 3e38, -3e38], np.float32)])
    dec = orc.decode(orc.encode(v, fmt), fmt)
    assert np.all(np.isfinite(dec))
    assert np.max(np.abs(dec)) <= MAXV[fmt]


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_matches_torch_cast_in_range(orc, fmt):
    """torch's CPU cast is RNE and non-saturating: compare where it cannot overflow."""
    lim = 464.0 if fmt == E4M3 else 61439.0
    # a strided sweep over all fp32 bit patterns
    bits = np.arange(0, 1 << 32, 251, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    with np.errstate(invalid="ignore"):
        v = v[np.isfinite(v) & (np.abs(v) <= lim)]
    got = orc.encode(v, fmt)
    ref = torch.from_numpy(v).to(TORCH_DT[fmt]).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
