"""GPU parity at the size limits: tensors beyond 2^31 elements (64-bit element
indexing in the streaming kernels) and GEMM operands just below 2^31 bytes (the
GEMMs' 32-bit operand offsets).  Inputs are built on the GPU; checks cover the
statistic exactly and sampled rows (the last ones included) against the oracle.

* absmax over 2^31 + 40 elements, planted maxima on both sides of 2^31;
* quantise of a [131088, 16384] tensor (2^31 + 2^18 elements), q and qt;
* SwiGLU requant with M F = 2^31 + 2^18 outputs, hq and hqt: every row holds the
  same set of (gate, up) pairs, shifted by the row index, so the global
  statistic is that of one row while a wrong row offset changes the bytes;
* fwd GEMMs whose A or B operand has 131056 rows of 16384 bytes (2^31 - 2^18).
"""
import numpy as np
import pytest
import torch

from gpu_util import E4M3, assert_codes_equal, assert_f32_equal, assert_within_sum_bound, gemm_compare, say, scalar

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8():
    import fp8_precision_amd
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return fp8_precision_amd


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def pattern_rows(vals: torch.Tensor, rows, cols: int, shift: int = 1) -> torch.Tensor:
    """bf16 rows r of [.., cols] with element j = vals[(shift * r + j) % len(vals)] (built on the GPU)."""
    r = torch.as_tensor(rows, device="cuda", dtype=torch.int64)
    j = torch.arange(cols, device="cuda", dtype=torch.int64)
    return vals[(shift * r[:, None] + j[None, :]) % vals.numel()]


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_absmax_beyond_2_31(fp8, orc):
    n = (1 << 31) + 40
    say("absmax large", n)
    x = torch.full((n,), 0.5, dtype=torch.bfloat16, device="cuda")
    x[7] = -3.0
    x[(1 << 31) - 1] = 5.5
    x[(1 << 31) + 33] = -7.25                 # beyond 2^31: the maximum
    got = scalar(fp8.absmax(x))
    ref = orc.absmax_bf16(bits_of(torch.tensor([0.5, -3.0, 5.5, -7.25], dtype=torch.bfloat16)))
    assert_f32_equal(got, ref, "absmax beyond 2^31")
    x[(1 << 31) + 33] = 0.5                   # now the maximum sits just below 2^31
    assert_f32_equal(scalar(fp8.absmax(x)), np.float32(5.5), "absmax below 2^31")
    del x
    free()


def test_quantize_beyond_2_31(fp8, orc):
    rows, cols = 131088, 16384
    say("quantize large", rows, cols)
    vals = ((torch.arange(251, device="cuda", dtype=torch.float32) - 125.0) * 0.0137).to(torch.bfloat16)
    x = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, rows, 4096):
        r1 = min(rows, r0 + 4096)
        x[r0:r1] = pattern_rows(vals, range(r0, r1), cols)
    am = fp8.absmax(x)
    am_ref = orc.absmax_bf16(bits_of(vals))
    assert_f32_equal(scalar(am), am_ref, "absmax")
    q, qt, s, inv = fp8.quantize(x, E4M3, am, want_q=True, want_qt=True)
    s_ref, inv_ref = orc.scale(am_ref, E4M3)
    assert_f32_equal(scalar(s), s_ref, "scale")
    sample = [0, 1, 4095, 65535, 131071, 131072, rows - 2, rows - 1]
    xs = bits_of(pattern_rows(vals, sample, cols))
    q_ref, _ = orc.quantize(xs, E4M3, s_ref)
    idx = torch.as_tensor(sample, device="cuda")
    assert_codes_equal(q[idx].cpu().numpy(), q_ref, E4M3, "q rows")
    assert_codes_equal(qt[:, idx].t().contiguous().cpu().numpy(), q_ref, E4M3, "qt columns")
    del x, q, qt
    free()


def test_swiglu_beyond_2_31(fp8, orc):
    M, F = 131088, 16384                      # M F = 2^31 + 2^18; M % 16 == 0 for hqt
    say("swiglu large", M, F)
    vals = ((torch.arange(253, device="cuda", dtype=torch.float32) - 126.0) * 0.041).to(torch.bfloat16)
    gu = torch.empty((M, 2 * F), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, M, 2048):
        r1 = min(M, r0 + 2048)
        gu[r0:r1] = pattern_rows(vals, range(r0, r1), 2 * F, shift=7)
    hq, hqt, am, inv = fp8.swiglu_requant(gu, compute_absmax=True, want_hq=True, want_hqt=False)
    # every row holds the same (gate, up) pairs: the statistic of row 0 is the global one
    row0 = bits_of(pattern_rows(vals, [0], 2 * F, shift=7))
    _, _, am_ref, inv_ref = orc.swiglu_requant(row0, want_hq=False)
    assert_f32_equal(scalar(am), am_ref, "absmax_h")
    assert_f32_equal(scalar(inv), inv_ref, "inv_scale_h")
    sample = [0, 3, 65535, 65536, 131071, M - 1]
    g_rows = bits_of(pattern_rows(vals, sample, 2 * F, shift=7))
    hq_ref, hqt_ref, _, _ = orc.swiglu_requant(g_rows, absmax_h=am_ref, want_hq=True, want_hqt=False)
    idx = torch.as_tensor(sample, device="cuda")
    assert_codes_equal(hq[idx].cpu().numpy(), hq_ref, E4M3, "hq rows")
    del hq
    free()
    # the transposed copy (recomputation form, retained statistic): sampled columns
    hq2, hqt2, _, _ = fp8.swiglu_requant(gu, absmax_h=am, compute_absmax=False, want_hq=False, want_hqt=True)
    assert_codes_equal(hqt2[:, idx].t().contiguous().cpu().numpy(), hq_ref, E4M3, "hqt columns")
    del gu, hqt2
    free()


def rand_codes(shape, seed):
    """e4m3 codes with |v| <= 15 (no NaN), random signs, generated on the GPU."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    mag = torch.randint(0, 0x58, shape, generator=g, device="cuda", dtype=torch.uint8)
    sgn = torch.randint(0, 2, shape, generator=g, device="cuda", dtype=torch.uint8) * 0x80
    return mag | sgn


@pytest.mark.parametrize("big", ["A", "B"])
def test_gemm_operand_near_2_31_bytes(fp8, orc, big):
    rows, K, small = 131056, 16384, 256      # rows x K = 2^31 - 2^18 bytes
    say("gemm large operand", big, rows, K, small)
    M, N = (rows, small) if big == "A" else (small, rows)
    xq, wq = rand_codes((M, K), 11), rand_codes((N, K), 12)
    ia = torch.tensor([2.0 ** -6], device="cuda")
    ib = torch.tensor([0.03125], device="cuda")
    y = fp8.gemm_fwd(xq, wq, ia, ib)
    torch.cuda.synchronize()
    sample = torch.as_tensor([0, 1, 65535, 65536, rows - 17, rows - 1], device="cuda")
    da, db = np.float32(2.0 ** -6), np.float32(0.03125)
    if big == "A":
        a_rows, b_all = xq[sample].cpu().numpy(), wq.cpu().numpy()
        ref = orc.gemm(a_rows, E4M3, b_all, E4M3, da, db)
        got = y[sample].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        gemm_compare(got, ref, "large A")
        assert_within_sum_bound(got, ref, a_rows, E4M3, b_all, E4M3, da, db, np.arange(len(a_rows)), "large A")
    else:
        a_all, b_rows = xq.cpu().numpy(), wq[sample].cpu().numpy()
        ref = orc.gemm(a_all, E4M3, b_rows, E4M3, da, db)
        got = y[:, sample].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        gemm_compare(got, ref, "large B")
        assert_within_sum_bound(got, ref, a_all, E4M3, b_rows, E4M3, da, db, np.arange(len(a_all)), "large B")
    del xq, wq, y
    free()
