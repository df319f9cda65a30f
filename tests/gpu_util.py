"""Helpers of the GPU parity tests: host/device transfers and comparisons."""
import sys

import numpy as np
import torch

E4M3, E5M2 = 0, 1


def say(*a):
    """Name the case before a GPU step (flushed, so it survives a hard failure)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.to("cuda", non_blocking=False)


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy()


def f32_bits(x) -> int:
    return int(np.asarray(x, np.float32).reshape(-1)[0:1].view(np.uint32)[0])


def scalar(t: torch.Tensor) -> np.float32:
    return np.float32(t.detach().cpu().numpy().reshape(-1)[0])


def is_nan_code(c: np.ndarray, fmt: int) -> np.ndarray:
    if fmt == E4M3:
        return (c & 0x7F) == 0x7F
    return ((c & 0x7C) == 0x7C) & ((c & 0x03) != 0)


def assert_codes_equal(gpu: np.ndarray, ref: np.ndarray, fmt: int, what: str):
    """Bit-exact, except that a NaN code may carry either sign / payload."""
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    neq = gpu != ref
    if not neq.any():
        return
    nan_ok = is_nan_code(gpu, fmt) & is_nan_code(ref, fmt)
    bad = neq & ~nan_ok
    if bad.any():
        idx = np.argwhere(bad)[:5]
        ex = [(tuple(i), hex(int(gpu[tuple(i)])), hex(int(ref[tuple(i)]))) for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} codes differ, e.g. {ex}")


def assert_f32_equal(gpu, ref, what: str):
    """Bit-exact fp32 scalars, any NaN matching any NaN."""
    g, r = np.float32(gpu), np.float32(ref)
    if np.isnan(r):
        assert np.isnan(g), (what, g, r)
    else:
        assert f32_bits(g) == f32_bits(r), (what, float(g), float(r))


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gemm_compare(gpu_bits: np.ndarray, ref_bits: np.ndarray, what: str, tol: float = 5e-3):
    """Relative Frobenius error of bf16 outputs (float64), and ulp diagnostics."""
    g = bf16_to_f64(gpu_bits)
    r = bf16_to_f64(ref_bits)
    assert np.all(np.isfinite(g)), what
    denom = np.linalg.norm(r)
    rel = np.linalg.norm(g - r) / denom if denom > 0 else np.linalg.norm(g - r)
    gi = gpu_bits.astype(np.int32)
    ri = ref_bits.astype(np.int32)
    same_sign = (gi >> 15) == (ri >> 15)
    ulp = np.where(same_sign, np.abs(gi - ri), 1 << 16)
    stats = {"rel_F": float(rel), "exact": float(np.mean(gi == ri)), "max_ulp": int(ulp.max())}
    assert rel <= tol, (what, stats)
    return stats


_TDT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}


def decode_abs64(codes: np.ndarray, fmt: int) -> np.ndarray:
    """|decoded value| in float64 via torch's CPU float8 decode (test-side only)."""
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(_TDT[fmt]).to(torch.float64)
    return t.abs().numpy()


def assert_within_sum_bound(gpu_bits, ref_bits, a, fa, b, fb, da, db, rows, what):
    """Elementwise: |gpu - ref| <= bf16 rounding of both + 4 K 2^-24 sum_k |a_k b_k| * descale.

    Any summation order of K exact fp32 products errs by at most (K-1) 2^-24
    times the sum of their magnitudes (first order); two such sums differ by
    twice that, and the factor 4 leaves room for an accumulator that truncates
    instead of rounding.
    """
    K = a.shape[1]
    descale = float(np.float32(np.float32(da) * np.float32(db)))
    absprod = decode_abs64(a[rows], fa) @ decode_abs64(b, fb).T
    g = bf16_to_f64(gpu_bits)
    r = bf16_to_f64(ref_bits)
    bound = (np.abs(r) + np.abs(g)) * 2.0 ** -8 + 4.0 * K * 2.0 ** -24 * absprod * descale + 1e-37
    bad = np.abs(g - r) > bound
    if bad.any():
        i = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} outputs outside the summation bound, e.g. "
                             f"{[(tuple(x), g[tuple(x)], r[tuple(x)], bound[tuple(x)]) for x in i]}")
