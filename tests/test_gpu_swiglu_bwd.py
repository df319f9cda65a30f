"""GPU parity of fp8_swiglu_backward (gradient of [gate | up], quantised) against the oracle.

Bit-exact: absmax, scale, inverse scale, q [M, 2F] and qt [2F, M] (a NaN code
may carry either sign), on random tensors at ragged shapes, on every finite
bf16 gate value, on special values, and on the full 7B-class tensor.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import E4M3, E5M2, assert_codes_equal, assert_f32_equal, say, scalar, u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8():
    import fp8_precision_amd
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return fp8_precision_amd


def to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def bf16(x) -> np.ndarray:
    return oracle.f32_to_bf16(np.ascontiguousarray(x, np.float32))


def check(fp8, gu, dh, fmt, want_q, want_qt, what):
    say("swiglu_backward", what, gu.shape, fmt, want_q, want_qt)
    q, qt, am, sc, inv = fp8.swiglu_backward(to_dev(gu), to_dev(dh), fmt, want_q=want_q, want_qt=want_qt)
    q_r, qt_r, am_r, sc_r, inv_r = oracle.swiglu_backward(gu, dh, fmt, want_q=want_q, want_qt=want_qt)
    assert_f32_equal(scalar(am), am_r, f"{what} absmax")
    assert_f32_equal(scalar(sc), sc_r, f"{what} scale")
    assert_f32_equal(scalar(inv), inv_r, f"{what} inv_scale")
    if want_q:
        assert_codes_equal(u8(q), q_r, fmt, f"{what} q")
    if want_qt:
        assert_codes_equal(u8(qt), qt_r, fmt, f"{what} qt")


@pytest.mark.parametrize("fmt", [E5M2, E4M3])
@pytest.mark.parametrize("M,F", [(16, 16), (64, 2064), (272, 528), (128, 1040), (512, 11008), (48, 80)])
@pytest.mark.parametrize("want", [(True, False), (True, True), (False, True)])
def test_random(fp8, fmt, M, F, want):
    rng = np.random.default_rng(M * 7 + F + fmt)
    gu = bf16(rng.standard_normal((M, 2 * F)) * 3)
    dh = bf16(rng.standard_normal((M, F)) * 1e-3)
    check(fp8, gu, dh, fmt, *want, f"random {M}x{F}")


def test_every_gate_value(fp8):
    """Every finite bf16 g with |g| <= 128 (the table range and the rules around it), u and dh random."""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    g = oracle.bf16_to_f32(b)
    keep = np.isfinite(g) & (np.abs(g) <= 128)
    gb = b[keep]
    F = 1024
    n = ((len(gb) + F - 1) // F + 15) // 16 * 16      # rows: a multiple of 16 (the transposed copy)
    gates = np.resize(gb, n * F).reshape(n, F)
    rng = np.random.default_rng(9)
    up = bf16(rng.standard_normal((n, F)))
    gu = np.ascontiguousarray(np.concatenate([gates, up], axis=1))
    dh = bf16(rng.standard_normal((n, F)) * 1e-2)
    check(fp8, gu, dh, E5M2, True, True, "every gate value")


@pytest.mark.parametrize("up,d", [(-5.0, 0.75), (1.0, -3.0)])
def test_statistic_of_every_gate_value(fp8, up, d):
    """Each of the 65536 gate patterns alone decides a call's statistic: its row
    holds the pattern (with the given u and dh) and 15 in-range neighbours with
    g = 1, u = 0, dh = 0 (dg = du = 0), so the table lookup or the exact rules
    for that one value alone give absmax; compared with the oracle's gradient
    row by row."""
    say("swiglu_backward statistic sweep", up, d)
    n, F = 65536, 16
    gu = np.zeros((n, 2 * F), np.uint16)
    gu[:, :F] = 0x3F80
    gu[:, 0] = np.arange(n, dtype=np.uint32).astype(np.uint16)
    gu[:, F] = bf16(np.float32(up))
    dh = np.zeros((n, F), np.uint16)
    dh[:, 0] = bf16(np.float32(d))
    gud, dhd = to_dev(gu), to_dev(dh)
    am = torch.empty(n, dtype=torch.float32, device="cuda")
    q = torch.empty((n, 2 * F), dtype=torch.uint8, device="cuda")
    for i in range(n):
        fp8.swiglu_backward(gud[i:i + 1], dhd[i:i + 1], E5M2, absmax=am[i:i + 1], q=q[i:i + 1])
    am_g = am.cpu().numpy()
    grad = oracle.swiglu_grad(gu, dh)
    bad = []
    for i in range(n):
        want = oracle.absmax_f32(np.ascontiguousarray(grad[i]))
        ok = (np.isnan(want) and np.isnan(am_g[i])) or \
            np.float32(am_g[i]).view(np.uint32) == np.float32(want).view(np.uint32)
        if not ok:
            bad.append((hex(gu[i, 0]), float(am_g[i]), float(want)))
            if len(bad) > 10:
                break
    assert not bad, bad


def test_special_values(fp8):
    rng = np.random.default_rng(4)
    M, F = 64, 256
    g = (rng.standard_normal((M, F)) * 4).astype(np.float32)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-30, -1e-30, 200.0, -200.0, 1e30, -1e30,
                         88.0, -88.0, -89.0, 2.0 ** -27, -(2.0 ** -27), 127.9, -127.9], np.float32)
    g.reshape(-1)[: len(specials) * 3: 3] = specials
    u = rng.standard_normal((M, F)).astype(np.float32)
    u.reshape(-1)[1: len(specials) * 3: 3] = specials
    gu = bf16(np.concatenate([g, u], axis=1))
    dh = bf16(rng.standard_normal((M, F)) * 1e-3)
    # finite part only for a meaningful scale: a separate tensor keeps the non-finite rows
    fin = np.isfinite(oracle.bf16_to_f32(gu)).all(axis=1)
    check(fp8, np.ascontiguousarray(gu[fin][:48]), np.ascontiguousarray(dh[fin][:48]), E5M2, True, True, "finite specials")
    check(fp8, gu, dh, E5M2, True, True, "with non-finite values")


@pytest.mark.parametrize("fmt", [E5M2])
def test_full_7b_shape(fp8, fmt):
    """M = 4096 tokens, F = 11008: every byte of q and qt."""
    g = torch.Generator().manual_seed(7)
    M, F = 4096, 11008
    gu = torch.randn((M, 2 * F), generator=g).mul_(2.0).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    dh = torch.randn((M, F), generator=g).mul_(1e-3).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    check(fp8, gu, dh, fmt, True, True, "7B shape")
