"""GPU parity of the block (MX) calls against the oracle.

fp8_mx_quantize (bit-exact codes and E8M0 scales):
* every bf16 pattern, in blocks whose maximum is planted at 1, 2 and 32 times
  the largest magnitude of the others (so each pattern is seen under several
  block scales), both formats; NaN and infinity patterns make their block's
  scale NaN;
* all-zero, tiny (clamped scale), saturating and mixed blocks;
* random tensors over several grid-stride rounds and the 7B-layer input and
  weight at full size; scales compared in the library's step-major layout.

fp8_mx_gemm_fwd (the oracle's MX GEMM on the GPU's own codes and scales;
relative Frobenius error <= 5e-3 and the any-order fp32 summation bound):
* with every scale 1.0 it equals the per-tensor GEMM with unit factors, bit
  for bit (same tiles, same reduction order, the block-scaled instruction);
* every output of a launch over two rounds with ragged rows and columns
  (tiles shifted back at both edges), for E4M3 and E5M2 inputs, on data whose
  blocks span 2^30 of scale;
* the 7B-layer QKV forward and the 14B-layer (outlier channels) QKV forward at
  full size on sampled rows;
* every output of a launch whose last tiles run as half tiles, at reductions of
  1, 2, 3 and 5 steps (every branch of the half tile's step loop);
* a NaN scale makes exactly its row's (column's) outputs NaN.

fp8_mx_gemm_backward (dgrad and wgrad of a linear in one launch): every output
against the oracle and bit for bit the separate fp8_mx_gemm_fwd calls, at a
shape run entirely as half tiles and one with a full round and a half-tile
round; the 7B down projection's backward at full size (bit for bit the separate
calls, sampled rows against the oracle).
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import E4M3, E5M2, assert_codes_equal, bf16_to_f64, decode_abs64, gemm_compare, say, u16, u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8():
    import fp8_precision_amd
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return fp8_precision_amd


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def step_major(sc):
    """Row-major scales [rows, cols / 32] -> the library's step-major [cols / 128, rows, 4]."""
    rows, nb = sc.shape
    return np.ascontiguousarray(sc.reshape(rows, nb // 4, 4).transpose(1, 0, 2))


def row_major(sc):
    """The library's step-major scales [cols / 128, rows, 4] -> [rows, cols / 32]."""
    ns, rows, _ = sc.shape
    return np.ascontiguousarray(sc.transpose(1, 0, 2).reshape(rows, 4 * ns))


def check_mx(fp8, orc, bits, fmt, what):
    say("mx_quantize", what, bits.shape, fmt)
    q, sc = fp8.mx_quantize(to_dev(bits), fmt)
    torch.cuda.synchronize()
    q_r, sc_r = orc.mx_quantize(np.ascontiguousarray(bits), fmt)
    sc_r = step_major(sc_r)
    gq, gs = u8(q), u8(sc)
    bad = np.argwhere(gs != sc_r)
    assert bad.size == 0, (what, "scales", bad[:4].tolist(), gs[tuple(bad[0])], sc_r[tuple(bad[0])])
    bad = np.argwhere(gq != q_r)
    assert bad.size == 0, (what, "codes", bad[:4].tolist(), hex(gq[tuple(bad[0])]), hex(q_r[tuple(bad[0])]))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("lift", [0, 1, 5])
def test_every_bf16_pattern(fp8, orc, fmt, lift):
    """31 patterns per block and a planted maximum 2^lift times their largest magnitude."""
    pats = np.arange(65536, dtype=np.uint32)
    pats = np.concatenate([pats, pats[:(-len(pats)) % 31]])     # whole blocks of 31
    blocks = pats.reshape(-1, 31)
    mag = blocks & 0x7FFF
    finite = np.where(mag < 0x7F80, mag, 0)
    top = finite.max(axis=1)
    # the planted maximum: the largest finite magnitude times 2^lift (bf16 bits: add to the
    # exponent field; kept finite and made at least the smallest normal)
    planted = np.minimum(np.maximum(top, 0x80) + (lift << 7), 0x7F7F)
    x = np.concatenate([planted[:, None], blocks], axis=1).astype(np.uint16)
    x = np.concatenate([x, np.zeros(((-len(x)) % 4, 32), np.uint16)])       # whole rows of 4 blocks
    check_mx(fp8, orc, x.reshape(-1, 128), fmt, f"every pattern, lift {lift}")


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_special_blocks(fp8, orc, fmt):
    rows = []
    rows.append(np.zeros(32, np.uint16))                                    # all zero
    z = np.zeros(32, np.uint16); z[3] = 0x8000; rows.append(z)              # -0
    rows.append(np.full(32, 0x0001, np.uint16))                             # smallest subnormal: clamped scale
    t = np.full(32, 0x0C00, np.uint16); t[7] = 0x8C40; rows.append(t)       # tiny normals
    s = np.full(32, 0x3F00, np.uint16); s[0] = 0x41F8; s[1] = 0xC1F8; rows.append(s)   # 31, -31: saturate
    for bad in (0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x7F81):
        r = np.full(32, 0x3FC0, np.uint16); r[17] = bad; rows.append(r)
    big = np.full(32, 0x7F7F, np.uint16); big[4] = 0xFF7F; rows.append(big)  # largest finite
    while len(rows) % 4:
        rows.append(np.full(32, 0x3F80, np.uint16))
    check_mx(fp8, orc, np.stack(rows).reshape(len(rows) // 4, 128), fmt, "special blocks")


@pytest.mark.parametrize("rows,cols", [(1, 128), (3, 384), (17, 4224), (1024, 1024), (777, 2176)])
def test_random_shapes(fp8, orc, rows, cols):
    x = workloads.draw(31, rows + cols, (rows, cols), 2.0)
    bits = workloads.bf16_bits(x)
    for fmt in (E4M3, E5M2):
        check_mx(fp8, orc, bits, fmt, f"random {rows}x{cols}")


def test_layer7b_full_size(fp8, orc):
    cfg = workloads.CONFIGS["layer7b"]
    for li, draw in ((0, workloads.draw_x), (0, workloads.draw_w), (2, workloads.draw_w)):
        x = draw(cfg, li)
        check_mx(fp8, orc, workloads.bf16_bits(x), E4M3, f"7B {draw.__name__} linear {li}")


def mx_bound_check(y_bits, ref_bits, a, sa, fa, b, sb, rows, what):
    """|gpu - oracle| within the bf16 rounding of both plus 4 K 2^-24 sum_k |a_k b_k| (scaled)."""
    K = a.shape[1]
    ea = np.exp2(np.repeat(sa[rows].astype(np.float64) - 127, 32, axis=1))
    eb = np.exp2(np.repeat(sb.astype(np.float64) - 127, 32, axis=1))
    absprod = (decode_abs64(a[rows], fa) * ea) @ (decode_abs64(b, E4M3) * eb).T
    g, r = bf16_to_f64(y_bits), bf16_to_f64(ref_bits)
    bound = (np.abs(r) + np.abs(g)) * 2.0 ** -8 + 4.0 * K * 2.0 ** -24 * absprod + 1e-37
    bad = np.abs(g - r) > bound
    assert not bad.any(), (what, int(bad.sum()), np.argwhere(bad)[:4].tolist())


def mx_operands(fp8, x, w, fx=E4M3):
    xq, sx = fp8.mx_quantize(x.cuda(), fx)
    wq, sw = fp8.mx_quantize(w.cuda(), E4M3)
    return xq, sx, wq, sw


def test_unit_scales_equal_per_tensor_gemm(fp8):
    say("mx_gemm unit scales", 4096, 4352, 1024)
    g = torch.Generator(device="cuda").manual_seed(5)
    a = torch.randn((4096, 1024), generator=g, device="cuda").mul_(60).to(torch.float8_e4m3fn).view(torch.uint8)
    b = torch.randn((4352, 1024), generator=g, device="cuda").mul_(60).to(torch.float8_e4m3fn).view(torch.uint8)
    sa = torch.full((8, 4096, 4), 127, dtype=torch.uint8, device="cuda")
    sb = torch.full((8, 4352, 4), 127, dtype=torch.uint8, device="cuda")
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    y = u16(fp8.mx_gemm_fwd(a, sa, b, sb))
    ref = u16(fp8.gemm_fwd(a, b, one, one))
    bad = np.argwhere(y != ref)
    assert bad.size == 0, ("unit-scale MX product differs from the per-tensor one", bad[:4].tolist())


@pytest.mark.parametrize("fx", [E4M3, E5M2])
def test_every_output_two_rounds(fp8, orc, fx):
    """4000 x 4368 x 512: 16 x 18 = 288 tiles (a round and 32 more), last row and
    column tiles shifted back; blocks scaled over 2^30."""
    M, N, K = 4000, 4368, 512
    say("mx_gemm every output", M, N, K, fx)
    rng = np.random.default_rng(17 + fx)
    xs = rng.standard_normal((M, K)) * np.exp2(rng.integers(-15, 15, (M, K // 32))).repeat(32, axis=1)
    ws = rng.standard_normal((N, K)) * np.exp2(rng.integers(-6, 6, (1, K // 32))).repeat(32, axis=1)
    x = torch.from_numpy(xs.astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(ws.astype(np.float32)).to(torch.bfloat16)
    xq, sx, wq, sw = mx_operands(fp8, x, w, fx)
    y = u16(fp8.mx_gemm_fwd(xq, sx, wq, sw, fx))
    a, sa, b, sb = u8(xq), row_major(u8(sx)), u8(wq), row_major(u8(sw))
    ref = orc.mx_gemm(a, sa, fx, b, sb, E4M3)
    gemm_compare(y, ref, "mx every output")
    rows = np.arange(M, dtype=np.int64)
    for r0 in range(0, M, 1000):
        rr = rows[r0:r0 + 1000]
        mx_bound_check(y[rr], ref[rr], a, sa, fx, b, sb, rr, "mx every output")


@pytest.mark.parametrize("K", [128, 256, 384, 640])
def test_half_tile_round_short_reductions(fp8, orc, K):
    """4352 x 4096: one round, then 16 tiles as 32 half tiles, at reductions of 1, 2,
    3 and 5 steps of 128 (every branch of the half tile's step loop), every output."""
    M, N = 4352, 4096
    say("mx_gemm half-tile round", M, N, K)
    x = workloads.draw(83, K, (M, K), 4.0)
    w = workloads.draw(83, K + 1, (N, K), 0.02)
    xq, sx, wq, sw = mx_operands(fp8, x, w)
    y = u16(fp8.mx_gemm_fwd(xq, sx, wq, sw))
    a, sa, b, sb = u8(xq), row_major(u8(sx)), u8(wq), row_major(u8(sw))
    ref = orc.mx_gemm(a, sa, E4M3, b, sb, E4M3)
    gemm_compare(y, ref, f"mx half-tile round K={K}")
    for r0 in range(0, M, 1088):
        rr = np.arange(r0, min(r0 + 1088, M), dtype=np.int64)
        mx_bound_check(y[rr], ref[rr], a, sa, E4M3, b, sb, rr, f"mx half-tile round K={K}")


@pytest.mark.parametrize("cfg_name", ["layer7b", "layer14b"])
def test_qkv_forward_full_size(fp8, orc, cfg_name):
    cfg = workloads.CONFIGS[cfg_name]
    x, w = workloads.draw_x(cfg, 0), workloads.draw_w(cfg, 0)
    say("mx_gemm qkv full size", cfg_name, tuple(x.shape), tuple(w.shape))
    xq, sx, wq, sw = mx_operands(fp8, x, w)
    y = u16(fp8.mx_gemm_fwd(xq, sx, wq, sw))
    a, sa, b, sb = u8(xq), row_major(u8(sx)), u8(wq), row_major(u8(sw))
    rng = np.random.default_rng(3)
    M = a.shape[0]
    rows = np.unique(np.concatenate([[0, 1, M - 2, M - 1], rng.integers(0, M, 252)])).astype(np.int64)
    ref = orc.mx_gemm(a, sa, E4M3, b, sb, E4M3, rows=rows)
    gemm_compare(y[rows], ref, f"{cfg_name} mx qkv")
    mx_bound_check(y[rows], ref, a, sa, E4M3, b, sb, rows, f"{cfg_name} mx qkv")


def test_nan_scale(fp8):
    M, N, K = 512, 768, 256
    say("mx_gemm nan scale", M, N, K)
    g = torch.Generator(device="cuda").manual_seed(8)
    a = torch.randn((M, K), generator=g, device="cuda").mul_(30).to(torch.float8_e4m3fn).view(torch.uint8)
    b = torch.randn((N, K), generator=g, device="cuda").mul_(30).to(torch.float8_e4m3fn).view(torch.uint8)
    sa = torch.full((K // 128, M, 4), 120, dtype=torch.uint8, device="cuda")
    sb = torch.full((K // 128, N, 4), 125, dtype=torch.uint8, device="cuda")
    sa[5 // 4, 300, 5 % 4] = 255           # block 5 of row 300
    sb[0, 700, 0] = 255                     # block 0 of row 700
    y = bf16_to_f64(u16(fp8.mx_gemm_fwd(a, sa, b, sb)))
    want = np.zeros((M, N), bool)
    want[300, :] = True
    want[:, 700] = True
    assert np.array_equal(np.isnan(y), want)


def check_mx_swiglu(fp8, orc, gu_bits, what):
    say("mx_swiglu_requant", what, gu_bits.shape)
    hq, sc = fp8.mx_swiglu_requant(to_dev(gu_bits))
    torch.cuda.synchronize()
    hq_r, sc_r = orc.mx_swiglu(np.ascontiguousarray(gu_bits))
    gs = u8(sc)
    bad = np.argwhere(gs != step_major(sc_r))
    assert bad.size == 0, (what, "scales", bad[:4].tolist())
    # a NaN h's code is a NaN code whose sign is not fixed (IEEE leaves the sign of a NaN open)
    assert_codes_equal(u8(hq), hq_r, E4M3, what)


def test_mx_swiglu_every_gate_value(fp8, orc):
    """All 65536 bf16 gate values (infinities and NaN included) against two up values,
    128 features per row: blocks mixing tiny, large, NaN and infinite h."""
    g = np.arange(65536, dtype=np.uint16).reshape(-1, 128)
    for ubits in (0x3F80, 0xC2C8):                     # u = 1, u = -100
        u = np.full(g.shape, ubits, np.uint16)
        check_mx_swiglu(fp8, orc, np.concatenate([g, u], axis=1), f"every gate value, u {ubits:#x}")


@pytest.mark.parametrize("M,F", [(1, 128), (7, 384), (33, 11008), (4096, 11008)])
def test_mx_swiglu_shapes(fp8, orc, M, F):
    x = workloads.draw(57, M + F, (M, 2 * F), 2.0)
    check_mx_swiglu(fp8, orc, workloads.bf16_bits(x), f"{M}x{F}")


def check_mx_t(fp8, orc, bits, fmt, what):
    """The transposed MX quantisation against the oracle's MX quantisation of x^T."""
    say("mx_quantize_t", what, bits.shape, fmt)
    qt, sc = fp8.mx_quantize_t(to_dev(bits), fmt)
    torch.cuda.synchronize()
    q_r, sc_r = orc.mx_quantize(np.ascontiguousarray(bits.T), fmt)
    bad = np.argwhere(u8(sc) != step_major(sc_r))
    assert bad.size == 0, (what, "scales", bad[:4].tolist())
    assert_codes_equal(u8(qt), q_r, fmt, what)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_mx_quantize_t_every_pattern(fp8, orc, fmt):
    """Every bf16 pattern down the columns of a 512 x 128 tensor (blocks of 32 rows
    mix all magnitudes, infinities and NaN), and planted column maxima."""
    x = np.arange(65536, dtype=np.uint16).reshape(128, 512).T.copy()
    check_mx_t(fp8, orc, x, fmt, "every pattern")
    rng = np.random.default_rng(fmt)
    y = workloads.bf16_bits(workloads.draw(61, fmt, (512, 256), 1.0)).copy()
    y[rng.integers(0, 512, 64), rng.integers(0, 256, 64)] = 0x4F80     # 2^32: saturating maxima elsewhere
    check_mx_t(fp8, orc, y, fmt, "planted maxima")


@pytest.mark.parametrize("rows,cols", [(128, 128), (384, 1280), (4096, 4096)])
def test_mx_quantize_t_shapes(fp8, orc, rows, cols):
    x = workloads.bf16_bits(workloads.draw(67, rows, (rows, cols), 3.0))
    check_mx_t(fp8, orc, x, E5M2, f"{rows}x{cols}")


def test_mx_backward_products(fp8, orc):
    """dgrad = dY . W and wgrad = dY^T . X on block-scaled operands (dY e5m2 blocked
    along N for dgrad and along M for wgrad, W^T and X^T from fp8_mx_quantize_t),
    against the oracle's MX GEMM on the same codes, every output."""
    M, N, K = 512, 768, 640
    dy = workloads.draw(71, 1, (M, N), 1e-3)
    w = workloads.draw(71, 2, (N, K), 0.02)
    x = workloads.draw(71, 3, (M, K), 1.0)
    E5 = E5M2
    dyq, sdy = fp8.mx_quantize(dy.cuda(), E5)
    wt, swt = fp8.mx_quantize_t(w.cuda(), E4M3)
    dx = u16(fp8.mx_gemm_fwd(dyq, sdy, wt, swt, E5))
    a, sa, b, sb = u8(dyq), row_major(u8(sdy)), u8(wt), row_major(u8(swt))
    ref = orc.mx_gemm(a, sa, E5, b, sb, E4M3)
    gemm_compare(dx, ref, "mx dgrad")
    mx_bound_check(dx, ref, a, sa, E5, b, sb, np.arange(M, dtype=np.int64), "mx dgrad")
    dyt, sdyt = fp8.mx_quantize_t(dy.cuda(), E5)
    xt, sxt = fp8.mx_quantize_t(x.cuda(), E4M3)
    dw = u16(fp8.mx_gemm_fwd(dyt, sdyt, xt, sxt, E5))
    a, sa, b, sb = u8(dyt), row_major(u8(sdyt)), u8(xt), row_major(u8(sxt))
    ref = orc.mx_gemm(a, sa, E5, b, sb, E4M3)
    gemm_compare(dw, ref, "mx wgrad")
    mx_bound_check(dw, ref, a, sa, E5, b, sb, np.arange(N, dtype=np.int64), "mx wgrad")


def mx_backward_operands(fp8, M, N, K, seed, dy_fmt=E5M2):
    """dY (e5m2 unless given), W and X of a linear, block-quantised for both backward products."""
    dy = workloads.draw(seed, 1, (M, N), 1e-3).cuda()
    w = workloads.draw(seed, 2, (N, K), 0.02).cuda()
    x = workloads.draw(seed, 3, (M, K), 1.0).cuda()
    dyq, sdy = fp8.mx_quantize(dy, dy_fmt)
    dyqt, sdyt = fp8.mx_quantize_t(dy, dy_fmt)
    wqt, swt = fp8.mx_quantize_t(w, E4M3)
    xqt, sxt = fp8.mx_quantize_t(x, E4M3)
    return dyq, sdy, dyqt, sdyt, wqt, swt, xqt, sxt


@pytest.mark.parametrize("M,N,K,fa", [(512, 768, 640, E5M2), (4096, 256, 4096, E5M2), (512, 768, 640, E4M3),
                                      (4096, 256, 4096, E4M3)])
def test_mx_gemm_backward_every_output(fp8, orc, M, N, K, fa):
    """fp8_mx_gemm_backward: dgrad and wgrad in one launch, every output against the
    oracle and bit for bit the two products run as separate fp8_mx_gemm_fwd calls.
    512 x 768 x 640: 6 + 9 tiles, all run as half tiles (ragged last column tiles);
    4096 x 256 x 4096: 16 + 256 tiles, a full round and 16 tiles of the second
    problem as 32 half tiles."""
    say("mx_gemm_backward every output", M, N, K, fa)
    ops = mx_backward_operands(fp8, M, N, K, 73, fa)
    dyq, sdy, dyqt, sdyt, wqt, swt, xqt, sxt = ops
    dx, dw = fp8.mx_gemm_backward(*ops, dy_fmt=fa)
    dx, dw = u16(dx), u16(dw)
    dx1 = u16(fp8.mx_gemm_fwd(dyq, sdy, wqt, swt, fa))
    dw1 = u16(fp8.mx_gemm_fwd(dyqt, sdyt, xqt, sxt, fa))
    assert np.array_equal(dx, dx1), np.argwhere(dx != dx1)[:4].tolist()
    assert np.array_equal(dw, dw1), np.argwhere(dw != dw1)[:4].tolist()
    a, sa, b, sb = u8(dyq), row_major(u8(sdy)), u8(wqt), row_major(u8(swt))
    ref = orc.mx_gemm(a, sa, fa, b, sb, E4M3)
    gemm_compare(dx, ref, "mx backward dgrad")
    mx_bound_check(dx, ref, a, sa, fa, b, sb, np.arange(M, dtype=np.int64), "mx backward dgrad")
    a, sa, b, sb = u8(dyqt), row_major(u8(sdyt)), u8(xqt), row_major(u8(sxt))
    ref = orc.mx_gemm(a, sa, fa, b, sb, E4M3)
    gemm_compare(dw, ref, "mx backward wgrad")
    mx_bound_check(dw, ref, a, sa, fa, b, sb, np.arange(N, dtype=np.int64), "mx backward wgrad")


def test_mx_gemm_backward_mixed_lengths(fp8, orc):
    """512 x 4608 x 3328: products of different reduction lengths whose long tiles do
    not fill the grid evenly (one round mixes long and short tiles): every output
    against the oracle and bit for bit the separate calls."""
    M, N, K = 512, 4608, 3328
    say("mx_gemm_backward mixed reduction lengths", M, N, K)
    ops = mx_backward_operands(fp8, M, N, K, 89)
    dyq, sdy, dyqt, sdyt, wqt, swt, xqt, sxt = ops
    dx, dw = fp8.mx_gemm_backward(*ops, dy_fmt=E5M2)
    dx, dw = u16(dx), u16(dw)
    assert np.array_equal(dx, u16(fp8.mx_gemm_fwd(dyq, sdy, wqt, swt, E5M2)))
    assert np.array_equal(dw, u16(fp8.mx_gemm_fwd(dyqt, sdyt, xqt, sxt, E5M2)))
    for y, (a, sa, b, sb), what in ((dx, (dyq, sdy, wqt, swt), "dgrad"), (dw, (dyqt, sdyt, xqt, sxt), "wgrad")):
        a, sa, b, sb = u8(a), row_major(u8(sa)), u8(b), row_major(u8(sb))
        ref = orc.mx_gemm(a, sa, E5M2, b, sb, E4M3)
        gemm_compare(y, ref, f"mx mixed-length {what}")
        mx_bound_check(y, ref, a, sa, E5M2, b, sb, np.arange(a.shape[0], dtype=np.int64), f"mx mixed-length {what}")


def test_mx_gemm_backward_down_7b(fp8, orc):
    """The 7B down projection's backward (M = 4096, N = 4096, K = 11008: 688 + 688
    tiles, five rounds and 96 tiles as half tiles): bit for bit the separate calls
    over every output, and sampled rows of both products against the oracle."""
    M, N, K = 4096, 4096, 11008
    say("mx_gemm_backward 7B down", M, N, K)
    ops = mx_backward_operands(fp8, M, N, K, 79)
    dyq, sdy, dyqt, sdyt, wqt, swt, xqt, sxt = ops
    dx, dw = fp8.mx_gemm_backward(*ops, dy_fmt=E5M2)
    dx, dw = u16(dx), u16(dw)
    dx1 = u16(fp8.mx_gemm_fwd(dyq, sdy, wqt, swt, E5M2))
    dw1 = u16(fp8.mx_gemm_fwd(dyqt, sdyt, xqt, sxt, E5M2))
    assert np.array_equal(dx, dx1), np.argwhere(dx != dx1)[:4].tolist()
    assert np.array_equal(dw, dw1), np.argwhere(dw != dw1)[:4].tolist()
    rng = np.random.default_rng(11)
    for y, (a, sa, b, sb), P, what in ((dx, (dyq, sdy, wqt, swt), M, "dgrad"), (dw, (dyqt, sdyt, xqt, sxt), N, "wgrad")):
        a, sa, b, sb = u8(a), row_major(u8(sa)), u8(b), row_major(u8(sb))
        rows = np.unique(np.concatenate([[0, P - 1], rng.integers(0, P, 62)])).astype(np.int64)
        ref = orc.mx_gemm(a, sa, E5M2, b, sb, E4M3, rows=rows)
        gemm_compare(y[rows], ref, f"7B down mx {what}")
        mx_bound_check(y[rows], ref, a, sa, E5M2, b, sb, rows, f"7B down mx {what}")


def planted_finite_blocks(seed):
    """A finite 256 x 256 bf16 tensor whose row and column blocks hit the edges of
    the block rule: all-zero and all-subnormal 32 x 32 squares, block maxima at
    the smallest normal, at and just past the magnitudes where an E4M3 (464 2^e)
    or E5M2 (61440 2^e) code would round past the largest finite one, at and just
    below powers of two, the largest finite bf16, with either sign."""
    rng = np.random.default_rng(seed)
    bits = workloads.bf16_bits(workloads.draw(seed, 1, (256, 256), 2.0))
    bits[32:64, 64:96] = 0
    sub = rng.integers(1, 0x80, size=(32, 32), dtype=np.uint16)
    bits[64:96, 128:160] = sub | (rng.integers(0, 2, size=(32, 32), dtype=np.uint16) << 15)
    maxima = [0x0080, 0x43E8, 0x43E9, 0x43E7, 0xC3E9, 0x4770, 0x476F, 0x4771, 0xC770, 0x4380, 0x437F,
              0x7F7F, 0xFF7F, 0x3F80, 0x3F7F, 0x0100]
    small = lambda shape, m: (rng.integers(0, max(m & 0x7FFF, 1), size=shape, dtype=np.uint16)
                              | (rng.integers(0, 2, size=shape, dtype=np.uint16) << 15))
    for i, m in enumerate(maxima):
        # a row block (row 128 + i, columns 32 .. 63) and a column block (column 160 + i,
        # rows 192 .. 223) with small values and one planted maximum at a varying place
        r = 128 + i
        bits[r, 32:64] = small(32, m)
        bits[r, 32 + (5 * i) % 32] = m
        c = 160 + i
        bits[192:224, c] = small(32, m)
        bits[192 + (7 * i) % 32, c] = m
    return bits


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_mx_quantize_both_planted_blocks(fp8, orc, fmt):
    """Finite tiles (the scaled-conversion path) at the block rule's edges: bit for bit the oracle's."""
    bits = planted_finite_blocks(91 + fmt)
    say("mx_quantize_both planted", fmt)
    q, sq, qt, sqt = fp8.mx_quantize_both(to_dev(bits), fmt)
    torch.cuda.synchronize()
    q_r, sq_r = orc.mx_quantize(np.ascontiguousarray(bits), fmt)
    qt_r, sqt_r = orc.mx_quantize(np.ascontiguousarray(bits.T), fmt)
    assert np.array_equal(u8(sq), step_major(sq_r)), "row-block scales"
    assert np.array_equal(u8(sqt), step_major(sqt_r)), "column-block scales"
    assert_codes_equal(u8(q), q_r, fmt, "q")
    assert_codes_equal(u8(qt), qt_r, fmt, "qt")
    # the same tensor with one NaN: its wave takes the per-element rule, the others not
    bits[100, 77] = 0x7FC1
    q, sq, qt, sqt = fp8.mx_quantize_both(to_dev(bits), fmt)
    torch.cuda.synchronize()
    q_r, sq_r = orc.mx_quantize(np.ascontiguousarray(bits), fmt)
    qt_r, sqt_r = orc.mx_quantize(np.ascontiguousarray(bits.T), fmt)
    assert np.array_equal(u8(sq), step_major(sq_r)) and np.array_equal(u8(sqt), step_major(sqt_r)), "scales"
    assert_codes_equal(u8(q), q_r, fmt, "q with a NaN")
    assert_codes_equal(u8(qt), qt_r, fmt, "qt with a NaN")


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("rows,cols", [(512, 128), (384, 1280), (4096, 4096)])
def test_mx_quantize_both_matches_the_two_calls(fp8, orc, fmt, rows, cols):
    """One read, both blockings: bit for bit the oracle's (and so the two separate calls')."""
    if rows == 512:
        bits = np.arange(65536, dtype=np.uint16).reshape(128, 512).T.copy()    # every pattern
    else:
        bits = workloads.bf16_bits(workloads.draw(73, rows + fmt, (rows, cols), 2.0))
    say("mx_quantize_both", rows, cols, fmt)
    q, sq, qt, sqt = fp8.mx_quantize_both(to_dev(bits), fmt)
    torch.cuda.synchronize()
    q_r, sq_r = orc.mx_quantize(np.ascontiguousarray(bits), fmt)
    qt_r, sqt_r = orc.mx_quantize(np.ascontiguousarray(bits.T), fmt)
    assert np.array_equal(u8(sq), step_major(sq_r)), "row-block scales"
    assert np.array_equal(u8(sqt), step_major(sqt_r)), "column-block scales"
    assert_codes_equal(u8(q), q_r, fmt, "q")
    assert_codes_equal(u8(qt), qt_r, fmt, "qt")
