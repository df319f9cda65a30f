"""Pins of the oracle's FP8 GEMM with per-tensor descale.

* a float64 matmul of the operands decoded by torch (an independent decoder),
  descaled and rounded to bf16: every output within one bf16 ulp of it and
  almost all identical, for non-square shapes in both operand formats -- a
  transposed or swapped operand fails it;
* exact-arithmetic cases that must match bit for bit: small-integer operands
  whose partial sums are exact in fp32, an identity right operand, all-ones
  operands with the closed form Y = bf16(K * da * db);
* row sampling returns the same rows as the full product.
"""
import numpy as np
import pytest
import torch

from oracle import E4M3, E5M2

TORCH_DT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}


def tdecode(c, fmt):
    return torch.from_numpy(c).view(TORCH_DT[fmt]).to(torch.float32).numpy()


def bf16_of(x64):
    """float64 -> fp32 -> bf16 (RNE), as float."""
    f = torch.from_numpy(np.asarray(x64, np.float64).astype(np.float32))
    return f.to(torch.bfloat16).to(torch.float32).numpy()


def bf16_bits_to_f32(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


def random_codes(rng, shape, fmt, sigma):
    x = (rng.standard_normal(shape) * sigma).astype(np.float32)
    return torch.from_numpy(x).to(TORCH_DT[fmt]).view(torch.uint8).numpy()


@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2)])
@pytest.mark.parametrize("M,N,K", [(16, 48, 128), (37, 80, 384), (128, 256, 256)])
def test_gemm_vs_float64_matmul(orc, fa, fb, M, N, K):
    rng = np.random.default_rng(M * N + K + fa)
    a = random_codes(rng, (M, K), fa, 30.0)
    b = random_codes(rng, (N, K), fb, 20.0)
    da, db = np.float32(1 / 448.0), np.float32(0.013)
    y = bf16_bits_to_f32(orc.gemm(a, fa, b, fb, da, db)).astype(np.float64)
    ref = tdecode(a, fa).astype(np.float64) @ tdecode(b, fb).astype(np.float64).T
    ref *= float(np.float32(da * db))
    # bf16 output rounding (<= 2^-9 relative) dominates; the fp32 accumulation
    # error (~K * 2^-24) can at most move an output to the neighbouring bf16 value
    ref_b = bf16_of(ref).astype(np.float64)
    ulp = np.abs(ref_b) * 2.0 ** -7 + 1e-30
    assert np.all(np.abs(y - ref_b) <= ulp)
    assert np.mean(y == ref_b) > 0.98
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel < 2.5e-3, rel
    # a transposed right operand is caught
    if M == N:
        bad = tdecode(a, fa).astype(np.float64) @ tdecode(b, fb).astype(np.float64)
        assert np.linalg.norm(y - bad) / np.linalg.norm(bad) > 0.5


def test_gemm_exact_small_integers(orc):
    rng = np.random.default_rng(3)
    M, N, K = 48, 64, 256
    ai = rng.integers(-4, 5, (M, K)).astype(np.float32)
    bi = rng.integers(-3, 4, (N, K)).astype(np.float32)
    a = torch.from_numpy(ai).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    b = torch.from_numpy(bi).to(torch.float8_e5m2).view(torch.uint8).numpy()
    da, db = np.float32(0.25), np.float32(2.0 ** -3)
    y = orc.gemm(a, E4M3, b, E5M2, da, db)
    exact = (ai.astype(np.int64) @ bi.astype(np.int64).T).astype(np.float64) * (0.25 * 2 ** -3)
    assert np.array_equal(bf16_bits_to_f32(y), bf16_of(exact))


def test_gemm_identity_and_ones(orc):
    K = 128
    rng = np.random.default_rng(4)
    a = random_codes(rng, (32, K), E4M3, 50.0)
    eye = np.zeros((K, K), np.uint8)
    eye[np.arange(K), np.arange(K)] = 0x38          # 1.0 in e4m3
    da, db = np.float32(0.5), np.float32(0.75)
    y = orc.gemm(a, E4M3, eye, E4M3, da, db)
    want = bf16_of(tdecode(a, E4M3).astype(np.float64) * float(np.float32(da * db)))
    assert np.array_equal(bf16_bits_to_f32(y), want)
    ones_a = np.full((16, 512), 0x38, np.uint8)
    ones_b = np.full((32, 512), 0x3C, np.uint8)     # 1.0 in e5m2
    y = orc.gemm(ones_a, E4M3, ones_b, E5M2, np.float32(3.0), np.float32(0.1))
    assert np.all(bf16_bits_to_f32(y) == bf16_of(512 * float(np.float32(np.float32(3.0) * np.float32(0.1)))))


def test_gemm_row_sampling(orc):
    rng = np.random.default_rng(11)
    a = random_codes(rng, (64, 256), E5M2, 100.0)
    b = random_codes(rng, (96, 256), E4M3, 100.0)
    full = orc.gemm(a, E5M2, b, E4M3, np.float32(0.01), np.float32(0.02))
    rows = np.array([63, 0, 17, 17], np.int64)
    part = orc.gemm(a, E5M2, b, E4M3, np.float32(0.01), np.float32(0.02), rows=rows)
    assert np.array_equal(part, full[rows])
