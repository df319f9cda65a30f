"""The five workload configurations at full size, step by step against the oracle.

Every GPU step is compared on the GPU's own upstream bytes (so each step is
judged bit-exact where its definition allows):
  absmax, scale, quantised bytes and transposed copies: bit-exact, full tensors;
  SwiGLU requantisation: bit-exact, full tensors;
  GEMMs: relative Frobenius error <= 5e-3 and the any-order summation bound on
  sampled output rows (first, last and seeded random rows).
The 32B configuration also checks the recomputation of the MLP block: the
retained bf16 input re-quantised with its retained absmax, the gate/up GEMM
rerun, and the SwiGLU requantised with the retained absmax_h give the forward's
bytes exactly, with no reduction.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import (E4M3, E5M2, assert_codes_equal, assert_f32_equal, assert_within_sum_bound, gemm_compare,
                      say, scalar, u16, u8)

pytestmark = pytest.mark.gpu
ROWS = 256                 # a seeded sample of 256 output rows per GEMM (first, last and random rows)


@pytest.fixture(scope="module")
def fp8():
    import fp8_precision_amd
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return fp8_precision_amd


def sample_rows(P, seed):
    r = np.random.default_rng(seed).integers(0, P, ROWS - 4)
    return np.unique(np.concatenate([[0, 1, P - 2, P - 1], r])).astype(np.int64)


def quant_step(fp8, orc, x_cpu, fmt, want_qt, what):
    """GPU absmax + quantise of a bf16 tensor, compared in full with the oracle."""
    say("quantise", what, tuple(x_cpu.shape), fmt)
    xd = x_cpu.cuda()
    am = fp8.absmax(xd)
    q, qt, s, inv = fp8.quantize(xd, fmt, am, want_q=True, want_qt=want_qt)
    bits = workloads.bf16_bits(x_cpu)
    am_r = orc.absmax_bf16(bits)
    assert_f32_equal(scalar(am), am_r, f"{what} absmax")
    s_r, inv_r = orc.scale(am_r, fmt)
    assert_f32_equal(scalar(s), s_r, f"{what} scale")
    assert_f32_equal(scalar(inv), inv_r, f"{what} inv_scale")
    q_r, qt_r = orc.quantize(bits, fmt, s_r, want_q=True, want_qt=want_qt)
    q_h = u8(q)
    assert_codes_equal(q_h, q_r, fmt, f"{what} q")
    if want_qt:
        assert_codes_equal(u8(qt), qt_r, fmt, f"{what} qt")
    return xd, am, q, qt, inv, q_h


def gemm_step(orc, y, a_h, fa, b_dev, inv_a, inv_b, what, seed):
    """Sampled rows of a GPU GEMM output against the oracle on the GPU's operand bytes."""
    b_h = u8(b_dev)
    rows = sample_rows(a_h.shape[0], seed)
    ia, ib = scalar(inv_a), scalar(inv_b)
    ref = orc.gemm(a_h, fa, b_h, E4M3, ia, ib, rows=rows)
    got = u16(y)[rows]
    stats = gemm_compare(got, ref, what)
    assert_within_sum_bound(got, ref, a_h, fa, b_h, E4M3, ia, ib, rows, what)
    return stats


def linear_forward(fp8, orc, cfg, li, backward):
    L = cfg.linears[li]
    x = workloads.draw_x(cfg, li)
    w = workloads.draw_w(cfg, li)
    _, _, xq, xqt, inv_x, xq_h = quant_step(fp8, orc, x, E4M3, backward, f"{cfg.name} X_{L.name}")
    _, _, wq, wqt, inv_w, _ = quant_step(fp8, orc, w, E4M3, backward, f"{cfg.name} W_{L.name}")
    say("gemm_fwd", cfg.name, L.name)
    y = fp8.gemm_fwd(xq, wq, inv_x, inv_w)
    gemm_step(orc, y, xq_h, E4M3, wq, inv_x, inv_w, f"{cfg.name} fwd {L.name}", 100 + li)
    return x, xq, xqt, inv_x, wq, wqt, inv_w, y


def linear_backward(fp8, orc, cfg, li, xqt, inv_x, wqt, inv_w):
    L = cfg.linears[li]
    dy = workloads.draw_dy(cfg, li)
    _, _, dyq, dyqt, inv_dy, dyq_h = quant_step(fp8, orc, dy, E5M2, True, f"{cfg.name} dY_{L.name}")
    say("gemm_dgrad", cfg.name, L.name)
    dx = fp8.gemm_dgrad(dyq, E5M2, wqt, inv_dy, inv_w)
    gemm_step(orc, dx, dyq_h, E5M2, wqt, inv_dy, inv_w, f"{cfg.name} dgrad {L.name}", 200 + li)
    say("gemm_wgrad", cfg.name, L.name)
    dw = fp8.gemm_wgrad(dyqt, E5M2, xqt, inv_dy, inv_x)
    gemm_step(orc, dw, u8(dyqt), E5M2, xqt, inv_dy, inv_x, f"{cfg.name} wgrad {L.name}", 300 + li)
    say("gemm_backward", cfg.name, L.name)
    dx2, dw2 = fp8.gemm_backward(dyq, dyqt, E5M2, wqt, xqt, inv_dy, inv_w, inv_x)
    assert torch.equal(dx2.view(torch.int16), dx.view(torch.int16)), "paired dgrad differs from fp8_gemm_dgrad"
    assert torch.equal(dw2.view(torch.int16), dw.view(torch.int16)), "paired wgrad differs from fp8_gemm_wgrad"
    return dx


# every linear of each configuration, except the down linear of an MLP chain,
# which consumes the SwiGLU output (covered by test_mlp_chain)
LINEAR_CASES = [(c, i) for c in ("fc256", "layer7b", "layer14b", "layer32b") for i, L in enumerate(workloads.CONFIGS[c].linears)
                if not (workloads.CONFIGS[c].mlp_chain and L.name == "down")]


@pytest.mark.parametrize("cname,li", LINEAR_CASES)
def test_linear_fwd_bwd(fp8, orc, cname, li):
    """Each linear of a configuration, forward and (when the configuration has it) backward."""
    cfg = workloads.CONFIGS[cname]
    _, _, xqt, inv_x, _, wqt, inv_w, _ = linear_forward(fp8, orc, cfg, li, cfg.backward)
    if cfg.backward:
        linear_backward(fp8, orc, cfg, li, xqt, inv_x, wqt, inv_w)
    torch.cuda.empty_cache()


def swiglu_step(fp8, orc, gu, want_hqt, what):
    say("swiglu", what, tuple(gu.shape))
    hq, hqt, am, inv = fp8.swiglu_requant(gu, compute_absmax=True, want_hq=True, want_hqt=want_hqt)
    gu_h = u16(gu)
    hq_r, hqt_r, am_r, inv_r = orc.swiglu_requant(gu_h, want_hqt=want_hqt)
    assert_f32_equal(scalar(am), am_r, f"{what} absmax_h")
    assert_f32_equal(scalar(inv), inv_r, f"{what} inv_h")
    hq_h = u8(hq)
    assert_codes_equal(hq_h, hq_r, E4M3, f"{what} hq")
    if want_hqt:
        assert_codes_equal(u8(hqt), hqt_r, E4M3, f"{what} hqt")
    return hq, hqt, am, inv, hq_h


@pytest.mark.parametrize("cname", ["mlp7b", "layer32b"])
def test_mlp_chain(fp8, orc, cname):
    """X -> e4m3 -> gate/up GEMM -> fused SwiGLU requant -> down GEMM; for the 32B
    configuration also the down linear's backward, the MLP recomputation, and the
    MLP backward on the recomputed gate/up output: dH (the down dgrad output) ->
    fused SwiGLU backward (e5m2 [dg | du] and its transposed copy, bit-exact in
    full) -> gate/up dgrad and wgrad (sampled rows)."""
    cfg = workloads.CONFIGS[cname]
    gi = [l.name for l in cfg.linears].index("gate_up")
    di = [l.name for l in cfg.linears].index("down")
    x, xq, xqt, inv_x, wq_gu, _, inv_wgu, gu = linear_forward(fp8, orc, cfg, gi, False)
    hq, hqt, am_h, inv_h, hq_h = swiglu_step(fp8, orc, gu, cfg.recompute, f"{cname} swiglu")
    wd = workloads.draw_w(cfg, di)
    _, _, wdq, wdqt, inv_wd, _ = quant_step(fp8, orc, wd, E4M3, cfg.backward, f"{cname} W_down")
    say("gemm_fwd down", cname)
    y = fp8.gemm_fwd(hq, wdq, inv_h, inv_wd)
    gemm_step(orc, y, hq_h, E4M3, wdq, inv_h, inv_wd, f"{cname} fwd down", 400)
    if not cfg.recompute:
        return
    # down linear backward: dgrad with W_down^T, wgrad with the SwiGLU output's transposed copy
    dh = linear_backward(fp8, orc, cfg, di, hqt, inv_h, wdqt, inv_wd)
    del y
    # recomputation with retained statistics: no reduction, identical bytes
    say("recompute", cname)
    am_x = fp8.absmax(x.cuda())
    am_x_before = am_x.clone()
    xq2, _, _, inv_x2 = fp8.quantize(x.cuda(), E4M3, am_x, want_q=True)
    assert torch.equal(xq2, xq) and torch.equal(inv_x2.view(torch.int32), inv_x.view(torch.int32))
    gu2 = fp8.gemm_fwd(xq2, wq_gu, inv_x2, inv_wgu)
    assert torch.equal(gu2.view(torch.int16), gu.view(torch.int16)), "gate/up GEMM is not deterministic"
    am_h_before = am_h.clone()
    hq2, hqt2, _, inv_h2 = fp8.swiglu_requant(gu2, absmax_h=am_h, compute_absmax=False, want_hq=True, want_hqt=True)
    torch.cuda.synchronize()
    assert torch.equal(am_h.view(torch.int32), am_h_before.view(torch.int32))
    assert torch.equal(am_x.view(torch.int32), am_x_before.view(torch.int32))
    assert torch.equal(hq2, hq) and torch.equal(hqt2, hqt)
    assert torch.equal(inv_h2.view(torch.int32), inv_h.view(torch.int32))
    del hq, hqt, hq2, hqt2, hq_h
    torch.cuda.empty_cache()
    # MLP backward through the fused SwiGLU backward
    say("swiglu_backward", cname)
    dgq, dgqt, am_dg, _, inv_dg = fp8.swiglu_backward(gu2, dh, E5M2, want_q=True, want_qt=True)
    q_r, qt_r, am_r, _, inv_r = orc.swiglu_backward(u16(gu2), u16(dh), E5M2, want_q=True, want_qt=True)
    assert_f32_equal(scalar(am_dg), am_r, f"{cname} d[gate | up] absmax")
    assert_f32_equal(scalar(inv_dg), inv_r, f"{cname} d[gate | up] inv_scale")
    dgq_h = u8(dgq)
    assert_codes_equal(dgq_h, q_r, E5M2, f"{cname} d[gate | up] q")
    del q_r
    assert_codes_equal(u8(dgqt), qt_r, E5M2, f"{cname} d[gate | up] qt")
    del qt_r, gu, gu2, dh
    torch.cuda.empty_cache()
    # the gate/up backward operands: W_gu^T (the forward's statistic, recomputed) and X^T
    _, _, _, wqt_gu, inv_wgu2, _ = quant_step(fp8, orc, workloads.draw_w(cfg, gi), E4M3, True, f"{cname} W_gate_up")
    assert torch.equal(inv_wgu2.view(torch.int32), inv_wgu.view(torch.int32))
    _, xqt2, _, _ = fp8.quantize(x.cuda(), E4M3, am_x, want_q=False, want_qt=True)
    say("gemm_dgrad gate_up", cname)
    dx_gu = fp8.gemm_dgrad(dgq, E5M2, wqt_gu, inv_dg, inv_wgu)
    gemm_step(orc, dx_gu, dgq_h, E5M2, wqt_gu, inv_dg, inv_wgu, f"{cname} dgrad gate_up", 500)
    del dx_gu, dgq_h
    say("gemm_wgrad gate_up", cname)
    dw_gu = fp8.gemm_wgrad(dgqt, E5M2, xqt2, inv_dg, inv_x)
    gemm_step(orc, dw_gu, u8(dgqt), E5M2, xqt2, inv_dg, inv_x, f"{cname} wgrad gate_up", 501)
    torch.cuda.empty_cache()
