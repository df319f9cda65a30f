"""GPU parity of fp8_gemm_fwd_swiglu_absmax: the gate/up forward GEMM with the
SwiGLU statistic taken in its epilogue.

* gu is bit-identical to fp8_gemm_fwd on the same operands;
* absmax_h is bit-exact against the oracle's SwiGLU absmax of the GPU's gu (the
  statistic fp8_swiglu_requant computes in its forward mode), at shapes with a
  ragged M (shifted-back last tile row), balanced last rounds (half tiles) and
  the 7B-class size, and it accumulates (max with the prior value);
* single-value cases: every output but one has h = 0, so absmax_h is |h| of a
  chosen gate value -- both sides of the bf16 exponents where s_g changes rule
  (g / 2 below 103, the table from 103 to 133, the large-|g| rules above),
  both signs, infinities and NaN.
"""
import numpy as np
import pytest
import torch

from gpu_util import E4M3, assert_f32_equal, dev, say, scalar, u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8():
    import fp8_precision_amd
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return fp8_precision_amd


def e4m3(values) -> np.ndarray:
    """Codes of exactly representable values (test data only), via torch's CPU cast."""
    return torch.tensor(np.asarray(values, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def scal(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def run(fp8, xq, wq, inv_x, inv_w, prior=0.0):
    am = scal(prior)
    gu = fp8.gemm_fwd_swiglu_absmax(dev(torch.from_numpy(xq)), dev(torch.from_numpy(wq)), scal(inv_x), scal(inv_w),
                                    am)
    return gu, am


@pytest.mark.parametrize("M,F,K", [(256, 128, 128), (272, 256, 384), (528, 384, 256), (1024, 1024, 512),
                                   (4352, 2048, 256), (4096, 11008, 4096)])
def test_matches_gemm_and_oracle(fp8, orc, M, F, K):
    say("gate_up fused absmax", M, F, K)
    g = torch.Generator(device="cpu").manual_seed(M + F + K)
    xq = torch.randn((M, K), generator=g).mul_(60.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    wq = torch.randn((2 * F, K), generator=g).mul_(60.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    inv_x, inv_w = np.float32(1 / 448.0), np.float32(0.0123)
    gu, am = run(fp8, xq, wq, inv_x, inv_w)
    ref_y = fp8.gemm_fwd(dev(torch.from_numpy(xq)), dev(torch.from_numpy(wq)), scal(inv_x), scal(inv_w))
    assert torch.equal(gu.view(torch.int16), ref_y.view(torch.int16)), "gu differs from fp8_gemm_fwd"
    gu_h = u16(gu)
    _, _, am_r, _ = orc.swiglu_requant(gu_h, want_hq=False)
    assert_f32_equal(scalar(am), am_r, f"absmax_h {M}x{F}x{K}")
    # accumulation: a larger prior stays, a smaller one is replaced
    big = float(np.float32(am_r) * np.float32(2.0))
    _, am2 = run(fp8, xq, wq, inv_x, inv_w, prior=big)
    assert_f32_equal(scalar(am2), np.float32(big), "larger prior kept")
    _, am3 = run(fp8, xq, wq, inv_x, inv_w, prior=float(np.float32(am_r) * np.float32(0.5)))
    assert_f32_equal(scalar(am3), am_r, "smaller prior replaced")
    torch.cuda.empty_cache()


def one_value_case(e, mant, neg):
    """Operands whose gu has g[0, 0] = (-1)^neg 2^(e-127) (1 + mant / 128) (bf16
    exponent field e, mantissa mant), u[0, 0] = 128 d, and every other gate and
    up value 0.  g = (128 + 16 m_hi + m_lo) d with d = 2^(e - 134): three exact
    e4m3 products summed exactly in fp32."""
    M, F, K = 256, 128, 128
    xq = np.zeros((M, K), np.uint8)
    xq[0, :3] = e4m3([1.0, 1.0, 1.0])
    wq = np.zeros((2 * F, K), np.uint8)
    s = -1.0 if neg else 1.0
    wq[0, :3] = e4m3([s * 128.0, s * 16.0 * (mant >> 4), s * float(mant & 15)])
    wq[F, 0] = e4m3([128.0])[0]
    # d = inv_x * inv_w = 2^(e - 134), split so that each factor is a normal fp32
    p = e - 134
    return xq, wq, np.float32(2.0 ** (p // 2)), np.float32(2.0 ** (p - p // 2))


@pytest.mark.parametrize("neg", [0, 1])
def test_single_values_across_rule_boundaries(fp8, orc, neg):
    cases = [(e, m) for e in (96, 101, 102, 103, 104, 120, 127, 132, 133, 134, 135, 140)
             for m in (0, 1, 64, 127)]
    for e, m in cases:
        xq, wq, ix, iw = one_value_case(e, m, neg)
        gu, am = run(fp8, xq, wq, ix, iw)
        gu_h = u16(gu)
        want_bits = (neg << 15) | (e << 7) | m
        assert gu_h[0, 0] == want_bits, (e, m, neg, hex(gu_h[0, 0]))
        _, _, am_r, _ = orc.swiglu_requant(gu_h, want_hq=False)
        assert_f32_equal(scalar(am), am_r, f"g bits {want_bits:#06x}")


def test_infinities_and_nan(fp8, orc):
    # +-inf gate: 256 * d overflows bf16 (d = 2^120 stays finite, so the zero
    # outputs stay 0); the up value 128 d = 2^127 is finite
    for sgn in (1.0, -1.0):
        xq, wq, _, _ = one_value_case(127, 0, 0)
        wq[0, :3] = e4m3([sgn * 128.0, sgn * 128.0, 0.0])
        gu, am = run(fp8, xq, wq, np.float32(2.0 ** 60), np.float32(2.0 ** 60))
        gu_h = u16(gu)
        assert gu_h[0, 0] == (0x7F80 if sgn > 0 else 0xFF80)
        assert np.count_nonzero(gu_h[1:]) == 0
        _, _, am_r, _ = orc.swiglu_requant(gu_h, want_hq=False)
        say("gate inf", sgn, float(scalar(am)), float(am_r))
        assert_f32_equal(scalar(am), am_r, f"gate {sgn} inf")
    # an e4m3 NaN operand code makes its output row NaN
    xq, wq, ix, iw = one_value_case(120, 5, 0)
    xq[3, 7] = 0x7F
    gu, am = run(fp8, xq, wq, ix, iw)
    assert np.isnan(scalar(am))
    _, _, am_r, _ = orc.swiglu_requant(u16(gu), want_hq=False)
    assert np.isnan(am_r)


def test_bench_path_matches_two_pass_forward(fp8, orc):
    """The forward as the step runs it -- fused GEMM, then fp8_swiglu_requant on
    the retained absmax_h -- gives the bytes of the two-pass forward (fp8_gemm_fwd,
    then fp8_swiglu_requant computing absmax_h)."""
    M, F, K = 1024, 1536, 512
    g = torch.Generator(device="cpu").manual_seed(9)
    xq = dev(torch.randn((M, K), generator=g).mul_(60.0).to(torch.float8_e4m3fn).view(torch.uint8))
    wq = dev(torch.randn((2 * F, K), generator=g).mul_(60.0).to(torch.float8_e4m3fn).view(torch.uint8))
    ix, iw = scal(1 / 448.0), scal(0.02)
    am = scal(0.0)
    gu = fp8.gemm_fwd_swiglu_absmax(xq, wq, ix, iw, am)
    hq, hqt, am_out, inv = fp8.swiglu_requant(gu, absmax_h=am, compute_absmax=False, want_hq=True, want_hqt=True)
    gu2 = fp8.gemm_fwd(xq, wq, ix, iw)
    hq2, hqt2, am2, inv2 = fp8.swiglu_requant(gu2, compute_absmax=True, want_hq=True, want_hqt=True)
    torch.cuda.synchronize()
    assert torch.equal(am.view(torch.int32), am2.view(torch.int32))
    assert torch.equal(hq, hq2) and torch.equal(hqt, hqt2)
    assert torch.equal(inv.view(torch.int32), inv2.view(torch.int32))
