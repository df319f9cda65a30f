"""GPU parity of fp8_swiglu_requant against the oracle (bit-exact).

* silu(g) for every one of the 65 536 bf16 gate values, read exactly through
  the absmax of a single-element h (u = 1), plus the sign through its code;
* forward mode on random [gate | up] tensors of ragged shapes: hq, hqt,
  absmax_h and the inverse scale;
* the recomputation invariant: with the retained statistic the bytes equal
  the forward's and the statistic is left untouched (no reduction);
* infinities and NaN in the gate.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import E4M3, assert_codes_equal, assert_f32_equal, dev, say, scalar, u16, u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8():
    import fp8_precision_amd
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return fp8_precision_amd


def bits_tensor(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16).copy()).view(torch.bfloat16)


@pytest.mark.parametrize("up_bits", [0x3F80, 0xC0A0])   # u = 1.0 and u = -5.0
# the other 15 gates of a row: 0 (outside the table's exponent range: the whole
# row takes the exact rules) or 1.0 (inside: a swept value inside the range is
# the only one that decides between the table and the rules); their up values
# are 0, so h = 0 there
@pytest.mark.parametrize("filler", [0x0000, 0x3F80])
def test_silu_every_gate_value(fp8, orc, up_bits, filler):
    say("silu sweep", hex(up_bits), hex(filler))
    n = 65536
    F = 16
    gu = np.zeros((n, 2 * F), np.uint16)
    gu[:, 1:F] = filler
    gu[:, 0] = np.arange(n, dtype=np.uint32).astype(np.uint16)
    gu[:, F] = up_bits
    gud = dev(bits_tensor(gu))
    am = torch.empty(n, dtype=torch.float32, device="cuda")
    hq = torch.empty((n, F), dtype=torch.uint8, device="cuda")
    for i in range(n):
        fp8.swiglu_requant(gud[i:i + 1], am[i:i + 1], compute_absmax=True, hq=hq[i:i + 1])
    am_g = am.cpu().numpy()
    hq_g = u8(hq)
    g = (gu[:, 0].astype(np.uint32) << 16).view(np.float32)
    bad = []
    for i in range(n):
        row = gu[i:i + 1]
        hq_r, _, am_r, _ = orc.swiglu_requant(row)
        ok_am = (np.isnan(am_r) and np.isnan(am_g[i])) or \
            np.float32(am_g[i]).view(np.uint32) == np.float32(am_r).view(np.uint32)
        if not ok_am:
            bad.append((hex(gu[i, 0]), float(g[i]), float(am_g[i]), float(am_r)))
            continue
        try:
            assert_codes_equal(hq_g[i:i + 1], hq_r, E4M3, "hq")
        except AssertionError as e:
            bad.append((hex(gu[i, 0]), str(e)))
        if len(bad) > 10:
            break
    assert not bad, bad


@pytest.mark.parametrize("M,F", [(1, 16), (5, 48), (16, 1040), (64, 2064), (130, 11008), (256, 4096)])
@pytest.mark.parametrize("sigma", [1.0, 8.0])
def test_forward_shapes(fp8, orc, M, F, sigma):
    say("swiglu fwd", M, F, sigma)
    gu = workloads.draw(11, M * 7 + F, (M, 2 * F), sigma)
    bits = u16(gu)
    gud = dev(gu)
    want_t = M % 16 == 0
    hq, hqt, am, inv = fp8.swiglu_requant(gud, compute_absmax=True, want_hq=True, want_hqt=want_t)
    hq_r, hqt_r, am_r, inv_r = orc.swiglu_requant(bits, want_hqt=want_t)
    assert_f32_equal(scalar(am), am_r, "absmax_h")
    assert_f32_equal(scalar(inv), inv_r, "inv_scale_h")
    assert_codes_equal(u8(hq), hq_r, E4M3, "hq")
    if want_t:
        assert_codes_equal(u8(hqt), hqt_r, E4M3, "hqt")
        # the flat kernel as well (forward, hq only)
        hq2, _, am2, _ = fp8.swiglu_requant(gud, compute_absmax=True, want_hq=True, want_hqt=False)
        assert_codes_equal(u8(hq2), hq_r, E4M3, "hq flat")


@pytest.mark.parametrize("M,F", [(16, 48), (64, 2064), (512, 11008)])
def test_recompute_invariant(fp8, orc, M, F):
    say("swiglu recompute", M, F)
    gu = dev(workloads.draw(12, M + F, (M, 2 * F), 2.0))
    hq, _, am, inv = fp8.swiglu_requant(gu, compute_absmax=True, want_hq=True)
    am_before = am.clone()
    hq2, hqt2, am2, inv2 = fp8.swiglu_requant(gu, absmax_h=am, compute_absmax=False, want_hq=True, want_hqt=True)
    torch.cuda.synchronize()
    assert torch.equal(am2.view(torch.int32), am_before.view(torch.int32))
    assert torch.equal(hq2, hq)
    assert torch.equal(hqt2, hq.t().contiguous())
    assert torch.equal(inv2.view(torch.int32), inv.view(torch.int32))
    # a stale retained statistic saturates instead of clipping silently
    stale = am / 8
    hq3, _, _, _ = fp8.swiglu_requant(gu, absmax_h=stale, compute_absmax=False)
    hq3_r, _, _, _ = orc.swiglu_requant(u16(gu.cpu()), absmax_h=scalar(stale))
    assert_codes_equal(u8(hq3), hq3_r, E4M3, "stale")


def test_nonfinite_gates(fp8, orc):
    say("swiglu nonfinite")
    F = 32
    gu = np.full((16, 2 * F), 0x3F80, np.uint16)
    gu[0, 0] = 0x7F80    # +inf -> silu = +inf
    gu[1, 1] = 0xFF80    # -inf -> NaN
    gu[2, 2] = 0x7FC0    # NaN
    for sl, name in [(slice(0, 1), "pos_inf"), (slice(1, 2), "neg_inf"), (slice(2, 3), "nan")]:
        rows = gu[sl]
        hq, _, am, _ = fp8.swiglu_requant(dev(bits_tensor(rows)), compute_absmax=True)
        hq_r, _, am_r, _ = orc.swiglu_requant(rows)
        assert_f32_equal(scalar(am), am_r, name)
        assert_codes_equal(u8(hq), hq_r, E4M3, name)


@pytest.mark.parametrize("M,F", [(16, 48), (512, 11008)])
def test_forward_accumulating_statistic(fp8, orc, M, F):
    """compute_absmax = 2: the statistic accumulates into a caller-cleared slot
    (no reset launch); from +0 the bytes equal the resetting forward's, a larger
    prior value stays and sets the scale (saturating like a stale statistic)."""
    say("swiglu accumulate", M, F)
    gu = dev(workloads.draw(13, M + F, (M, 2 * F), 2.0))
    hq, hqt, am, inv = fp8.swiglu_requant(gu, compute_absmax=True, want_hq=True, want_hqt=True)
    slots = torch.zeros(4, dtype=torch.float32, device="cuda")
    hq2, hqt2, am2, inv2 = fp8.swiglu_requant(gu, absmax_h=slots[1:2], compute_absmax=True, accumulate=True,
                                             want_hq=True, want_hqt=True)
    torch.cuda.synchronize()
    assert torch.equal(am2.view(torch.int32), am.view(torch.int32))
    assert torch.equal(hq2, hq) and torch.equal(hqt2, hqt)
    assert torch.equal(inv2.view(torch.int32), inv.view(torch.int32))
    assert float(slots[0]) == 0.0 and float(slots[2]) == 0.0
    big = am * 8
    prior = big.clone()
    hq3, _, am3, _ = fp8.swiglu_requant(gu, absmax_h=prior, compute_absmax=True, accumulate=True, want_hq=True)
    torch.cuda.synchronize()
    assert torch.equal(am3.view(torch.int32), big.view(torch.int32))
    hq3_r, _, _, _ = orc.swiglu_requant(u16(gu.cpu()), absmax_h=scalar(big))
    assert_codes_equal(u8(hq3), hq3_r, E4M3, "larger prior")
    with pytest.raises(ValueError):
        fp8.swiglu_requant(gu, compute_absmax=True, accumulate=True)
