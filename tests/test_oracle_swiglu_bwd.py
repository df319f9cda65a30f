"""Pins of the oracle's SwiGLU backward (the gradients of gate and up, quantised).

The oracle follows the textbook derivative of h = silu(g) * u with
silu(g) = g * sigma(g), sigma(g) = 1 / (1 + e^-g):
  du = dh * silu(g),  dg = dh * u * silu'(g),  silu'(g) = sigma * (1 + g * (1 - sigma)),
one fp32 operation at a time.  Pinned here against things other than that
formula:
* silu'(g) is the derivative of the forward nonlinearity: float64 central
  differences of g / (1 + e^-g);
* every finite bf16 g: silu'(g) within a rounding-error bound of a float64
  evaluation, and silu(g) bit-identical to the forward oracle's;
* closed forms: g = 0, large positive and large negative g, infinities;
* the layout [dg | du] and the two products, against numpy float32 arithmetic;
* the whole gradient against float64 finite differences of sum(dh * h);
* the quantised output: absmax, scale and codes through the pinned codec.
"""
import numpy as np
import pytest

import oracle

E5M2 = oracle.E5M2


def all_finite_bf16():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_to_f32(b)
    return b[np.isfinite(f)]


def grad_table(g_bits):
    """(dg, du) of every g with u = d = 1: dg = silu'(g), du = silu(g)."""
    n = len(g_bits)
    gu = np.empty((n, 2), np.uint16)
    gu[:, 0] = g_bits
    gu[:, 1] = 0x3F80                       # u = 1
    dh = np.full((n, 1), 0x3F80, np.uint16)  # dh = 1
    out = oracle.swiglu_grad(gu, dh)
    return out[:, 0], out[:, 1]


def test_derivative_of_the_forward_nonlinearity():
    """silu'(g) matches float64 central differences of g / (1 + e^-g)."""
    rng = np.random.default_rng(11)
    g = oracle.bf16_to_f32(oracle.f32_to_bf16(rng.uniform(-20, 20, 4000).astype(np.float32)))
    gb = oracle.f32_to_bf16(g)
    ds, _ = grad_table(gb)
    x = g.astype(np.float64)
    silu = lambda v: v / (1.0 + np.exp(-v))
    h = 1e-6
    fd = (silu(x + h) - silu(x - h)) / (2 * h)
    assert np.all(np.abs(ds - fd) <= 2e-6 * np.maximum(1.0, np.abs(fd)) + 1e-9), np.max(np.abs(ds - fd))


def test_every_bf16_gate_against_float64():
    gb = all_finite_bf16()
    ds, s = grad_table(gb)
    g = oracle.bf16_to_f32(gb).astype(np.float64)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    ref = sig * (1.0 + g * (1.0 - sig))
    # first-order error bound of the fp32 evaluation (a few roundings per term)
    bound = 16 * 2.0 ** -24 * (np.abs(sig) + np.abs(sig * g) * (np.abs(1 - sig) + np.abs(sig)) + np.abs(ref)) + 1e-40
    # where e^-g overflows fp32 (g < -88.72) the fp32 evaluation has sigma = 0 exactly and
    # silu' = -0, while the true value is below 2e-37 in magnitude
    ovf = np.exp(np.minimum(-g, 700.0)) > np.finfo(np.float32).max
    assert np.all((ds[ovf] == 0.0) & np.signbit(ds[ovf])) and np.all(np.abs(ref[ovf]) < 2e-37)
    fin = np.isfinite(ref) & ~ovf
    assert np.all(np.isfinite(ds[fin]))
    err = np.abs(ds[fin] - ref[fin])
    assert np.all(err <= bound[fin]), (int(np.sum(err > bound[fin])), float(np.max(err / bound[fin])))
    # silu(g) is the forward's, bit for bit
    gu = np.empty((len(gb), 2), np.uint16)
    gu[:, 0], gu[:, 1] = gb, 0x3F80
    h = oracle.swiglu_h(gu)[:, 0]
    assert np.array_equal(s.view(np.uint32), h.view(np.uint32))


def test_closed_forms():
    assert oracle.swiglu_grad_one(0.0, 3.0, 2.0) == (np.float32(3.0), np.float32(0.0))   # silu'(0) = 1/2
    assert oracle.swiglu_grad_one(-0.0, 5.0, 1.0)[0] == np.float32(2.5)
    for g in (30.0, 100.0, 1e4, 1e30):                       # sigma = 1: silu' = 1, silu = g
        dg, du = oracle.swiglu_grad_one(g, 1.5, 2.0)
        assert dg == np.float32(3.0) and du == np.float32(2.0 * np.float32(g))
    for g in (-100.0, -1e4):                                  # e^-g overflows: sigma = 0
        dg, du = oracle.swiglu_grad_one(g, 1.0, 1.0)
        assert dg == 0.0 and np.signbit(dg) and du == 0.0 and np.signbit(du)
    tiny = np.float32(2.0 ** -30)                             # sigma = 1/2, 1 + g/2 rounds to 1
    assert oracle.swiglu_grad_one(tiny, 1.0, 1.0)[0] == np.float32(0.5)
    dg, du = oracle.swiglu_grad_one(np.inf, 1.0, 1.0)
    assert np.isnan(dg) and du == np.inf
    dg, du = oracle.swiglu_grad_one(-np.inf, 1.0, 1.0)
    assert np.isnan(dg) and np.isnan(du)


def test_layout_and_products():
    rng = np.random.default_rng(3)
    M, F = 24, 40
    gu = oracle.f32_to_bf16((rng.standard_normal((M, 2 * F)) * 3).astype(np.float32))
    dh = oracle.f32_to_bf16((rng.standard_normal((M, F)) * 1e-3).astype(np.float32))
    out = oracle.swiglu_grad(gu, dh)
    g, u = oracle.bf16_to_f32(np.ascontiguousarray(gu[:, :F])), oracle.bf16_to_f32(np.ascontiguousarray(gu[:, F:]))
    d = oracle.bf16_to_f32(dh)
    ds, s = grad_table(np.ascontiguousarray(gu[:, :F]).reshape(-1))
    ds, s = ds.reshape(M, F), s.reshape(M, F)
    assert np.array_equal(out[:, F:].view(np.uint32), (d * s).view(np.uint32))            # du = dh * silu
    assert np.array_equal(out[:, :F].view(np.uint32), ((d * u) * ds).view(np.uint32))     # dg = (dh * u) * silu'


def test_gradient_by_finite_differences():
    """[dg | du] is the gradient of sum(dh * silu(g) * u) (float64 central differences)."""
    rng = np.random.default_rng(5)
    M, F = 4, 8
    gu = oracle.f32_to_bf16((rng.standard_normal((M, 2 * F)) * 2).astype(np.float32))
    dh = oracle.f32_to_bf16(rng.standard_normal((M, F)).astype(np.float32))
    out = oracle.swiglu_grad(gu, dh).astype(np.float64)
    x = oracle.bf16_to_f32(gu).astype(np.float64)
    d = oracle.bf16_to_f32(dh).astype(np.float64)

    def loss(v):
        g, u = v[:, :F], v[:, F:]
        return np.sum(d * g / (1.0 + np.exp(-g)) * u)

    h = 1e-6
    num = np.empty_like(x)
    for idx in np.ndindex(*x.shape):
        a, b = x.copy(), x.copy()
        a[idx] += h
        b[idx] -= h
        num[idx] = (loss(a) - loss(b)) / (2 * h)
    assert np.allclose(out, num, rtol=2e-5, atol=2e-6), np.max(np.abs(out - num))


@pytest.mark.parametrize("fmt", [E5M2, oracle.E4M3])
def test_quantised_output(fmt):
    rng = np.random.default_rng(7 + fmt)
    M, F = 48, 80
    gu = oracle.f32_to_bf16((rng.standard_normal((M, 2 * F)) * 2).astype(np.float32))
    dh = oracle.f32_to_bf16((rng.standard_normal((M, F)) * 1e-3).astype(np.float32))
    q, qt, am, sc, inv = oracle.swiglu_backward(gu, dh, fmt, want_q=True, want_qt=True)
    v = oracle.swiglu_grad(gu, dh)
    assert am == np.max(np.abs(v))
    s_r, inv_r = oracle.scale(am, fmt)
    assert sc == s_r and inv == inv_r
    assert np.array_equal(q, oracle.encode((v * s_r).astype(np.float32), fmt))
    assert np.array_equal(qt, q.T)
    # the absmax element lands on +-max (no clipping with a fresh statistic)
    top = oracle.decode(q.reshape(-1)[np.argmax(np.abs(v))], fmt)
    assert abs(top) == oracle.FP8_MAX[fmt]
