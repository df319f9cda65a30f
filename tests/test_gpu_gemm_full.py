"""Every output of GEMM launches that span several rounds of the persistent grid.

The persistent kernels walk their tiles round by round (a grouped raster order,
renumbered XCD-major); a launch whose last round is short runs its last tiles
as half tiles in a second launch.  Sampled rows cannot show a tile that was
skipped, computed twice with the wrong origin or stored to a neighbour's place
in a later round, so here every output element of such launches is compared
with the oracle (relative Frobenius error <= 5e-3 and the any-order fp32
summation bound), for each compiled form:

* forward (e4m3 x e4m3, K-major), three full rounds (the 7B qkv shape) and a
  launch with a balanced half-tile round (at reductions of 1, 2, 3, 4 and 5
  steps: every branch of the half tile's three-stage step loop), and the edge
  form (a matrix with fewer than 256 rows) over two rounds;
* a forward whose B operand is larger than the Infinity Cache (groups of 24
  tile rows instead of 8): every output bit for bit against the same product
  in column slices (each with the default groups), sampled rows against the
  oracle;
* the backward pair (e5m2 x e4m3, one launch for dgrad and wgrad): the 7B qkv
  pair (four rounds, long dgrad tiles first), and a pair whose tiles end in a
  balanced half-tile round;
* the same pair on the untransposed operands (MN-major, two rounds);
* pairs whose products differ in reduction length, with long and short tiles
  in one round: every output, and bit for bit the separate dgrad / wgrad calls
  and the MN-major pair;
* the gate/up forward with the SwiGLU statistic in its epilogue, with a
  half-tile round.

NaN and infinite operand codes are checked too: the outputs they reach are
NaN or infinite exactly where the oracle's are.
"""
import numpy as np
import pytest
import torch

from gpu_util import (E4M3, E5M2, assert_f32_equal, assert_within_sum_bound, bf16_to_f64, dev, gemm_compare, say, u16,
                      u8)

pytestmark = pytest.mark.gpu

TDT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}
SIGMA = {E4M3: 60.0, E5M2: 3000.0}


@pytest.fixture(scope="module")
def fp8():
    import fp8_precision_amd
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return fp8_precision_amd


def scal(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def rand_codes(g, shape, fmt):
    """Codes of N(0, sigma) values (torch's CPU cast; test data only)."""
    return torch.randn(shape, generator=g).mul_(SIGMA[fmt]).to(TDT[fmt]).view(torch.uint8).numpy()


def check_full(orc, y_gpu, a, fa, b, inv_a, inv_b, what):
    """Every output of y_gpu = A . B^T against the oracle."""
    ref = orc.gemm(a, fa, b, E4M3, inv_a, inv_b)
    y = u16(y_gpu)
    assert y.shape == ref.shape, (what, y.shape, ref.shape)
    stats = gemm_compare(y, ref, what)
    # the elementwise bound, in row blocks to bound the host memory it needs
    for r0 in range(0, a.shape[0], 2048):
        rows = np.arange(r0, min(r0 + 2048, a.shape[0]), dtype=np.int64)
        assert_within_sum_bound(y[rows], ref[rows], a, fa, b, E4M3, inv_a, inv_b, rows, what)
    return stats


INV_A = {E4M3: np.float32(1 / 448.0), E5M2: np.float32(1 / 57344.0)}
INV_B = np.float32(0.0123)


# (name, P, Q, R): 4096 x 12288 = 768 tiles = three rounds of 256; 4352 x 4096 =
# 272 tiles = one round and 16 tiles run as 32 half tiles; 128 x 76800 (edge form,
# fewer than 256 rows) = 300 tiles = two rounds.
FWD = [("7B qkv fwd, 3 rounds", 4096, 12288, 4096),
       ("balanced half-tile round", 4352, 4096, 512),
       ("edge form, 2 rounds", 128, 76800, 256)]


# The half-tile round runs a three-stage pipeline whose step loop has separate
# branches for 1, 2, 3 and more reduction steps: 4352 x 4096 (one round, then 16
# tiles as 32 half tiles) at reductions of 1, 2, 3 and 5 steps of 128.
FWD += [(f"half-tile round, {R // 128} reduction steps", 4352, 4096, R) for R in (128, 256, 384, 640)]


@pytest.mark.parametrize("name,P,Q,R", FWD)
def test_forward_every_output(fp8, orc, name, P, Q, R):
    say("gemm full output fwd", name, P, Q, R)
    g = torch.Generator(device="cpu").manual_seed(P + 7 * Q + R)
    a, b = rand_codes(g, (P, R), E4M3), rand_codes(g, (Q, R), E4M3)
    y = fp8.gemm_fwd(dev(torch.from_numpy(a)), dev(torch.from_numpy(b)), scal(INV_A[E4M3]), scal(INV_B))
    check_full(orc, y, a, E4M3, b, INV_A[E4M3], INV_B, name)


def test_forward_large_b_groups(fp8, orc):
    """6800 x 16592 x 16384: B is 272 MB, so the launch walks groups of 24 tile
    rows (27 row tiles: a full group and a group of 3; the last row and column
    tiles ragged).  Each output is reduced in the same order whatever tile or
    raster position computes it, so the launch must equal, bit for bit, the
    same product computed in column slices of 4096 (64 MiB of B each: the
    default groups of 8; the 208-column remainder in the edge form)."""
    P, Q, R = 6800, 16592, 16384
    say("gemm full output, large B", P, Q, R)
    g = torch.Generator(device="cuda").manual_seed(24)
    a = torch.randn((P, R), generator=g, device="cuda").mul_(SIGMA[E4M3]).to(TDT[E4M3]).view(torch.uint8)
    b = torch.randn((Q, R), generator=g, device="cuda").mul_(SIGMA[E4M3]).to(TDT[E4M3]).view(torch.uint8)
    ia, ib = scal(INV_A[E4M3]), scal(INV_B)
    y = torch.full((P, Q), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)   # 0xFFFF: NaN
    fp8.gemm_fwd(a, b, ia, ib, out=y)
    yh = u16(y)
    for c0 in range(0, Q, 4096):
        c1 = min(c0 + 4096, Q)
        ys = u16(fp8.gemm_fwd(a, b[c0:c1], ia, ib))
        bad = np.argwhere(ys != yh[:, c0:c1])
        assert bad.size == 0, ("large-B launch differs from its column slice", c0, c1, bad[:4].tolist())
    rows = np.unique(np.concatenate([[0, 255, 256, 6143, 6144, P - 1],
                                     np.random.default_rng(24).integers(0, P, 26)])).astype(np.int64)
    a_h, b_h = u8(a), u8(b)
    ref = orc.gemm(a_h, E4M3, b_h, E4M3, INV_A[E4M3], INV_B, rows=rows)
    gemm_compare(yh[rows], ref, "large-B forward, sampled rows")
    assert_within_sum_bound(yh[rows], ref, a_h, E4M3, b_h, E4M3, INV_A[E4M3], INV_B, rows, "large-B forward")


# (name, M, N, K): the qkv pair has 256 dgrad tiles (reduction 12288) and 768
# wgrad tiles (reduction 4096): four rounds; the second pair has 128 + 160 = 288
# tiles: one round, then 32 tiles as 64 half tiles.
PAIRS = [("7B qkv backward pair, 4 rounds", 4096, 12288, 4096),
         ("pair with a half-tile round", 2048, 2560, 4096)]


def pair_operands(g, M, N, K, fa):
    dyq = rand_codes(g, (M, N), fa)
    wq = rand_codes(g, (N, K), E4M3)
    xq = rand_codes(g, (M, K), E4M3)
    return dyq, wq, xq


@pytest.mark.parametrize("name,M,N,K", PAIRS)
def test_backward_pair_every_output(fp8, orc, name, M, N, K):
    say("gemm full output backward pair", name, M, N, K)
    g = torch.Generator(device="cpu").manual_seed(M + 3 * N + 5 * K)
    dyq, wq, xq = pair_operands(g, M, N, K, E5M2)
    dyqt, wqt, xqt = (np.ascontiguousarray(t.T) for t in (dyq, wq, xq))
    ia, iw, ix = INV_A[E5M2], np.float32(1 / 448.0), INV_B
    dx, dw = fp8.gemm_backward(*(dev(torch.from_numpy(t)) for t in (dyq, dyqt)), E5M2,
                               dev(torch.from_numpy(wqt)), dev(torch.from_numpy(xqt)), scal(ia), scal(iw), scal(ix))
    check_full(orc, dx, dyq, E5M2, wqt, ia, iw, name + " dgrad")
    check_full(orc, dw, dyqt, E5M2, xqt, ia, ix, name + " wgrad")


# Pairs whose two products differ in reduction length, with a long-tile count that
# does not fill the 256-CU grid evenly, so that one round mixes long and short tiles:
# 512 x 4608 x 3328 (26 dgrad tiles of 36 steps, 234 wgrad tiles of 4 steps; the
# last 4 as half tiles) and
# 512 x 4352 x 3584 (28 of 34 steps, 238 of 4; the last 10 as half tiles).
MIXED_PAIRS = [(512, 4608, 3328), (512, 4352, 3584)]


@pytest.mark.parametrize("M,N,K", MIXED_PAIRS)
def test_backward_pair_mixed_lengths(fp8, orc, M, N, K):
    """Every output against the oracle; bit for bit the separate dgrad and wgrad
    calls (each output is reduced in the same order whichever slot computes it),
    and the untransposed-operand pair bit for bit the same."""
    say("gemm backward pair, mixed reduction lengths", M, N, K)
    g = torch.Generator(device="cpu").manual_seed(M + N + K)
    dyq, wq, xq = pair_operands(g, M, N, K, E5M2)
    dyqt, wqt, xqt = (np.ascontiguousarray(t.T) for t in (dyq, wq, xq))
    ia, iw, ix = INV_A[E5M2], np.float32(1 / 448.0), INV_B
    d = {n: dev(torch.from_numpy(t)) for n, t in (("dyq", dyq), ("dyqt", dyqt), ("wq", wq), ("wqt", wqt),
                                                    ("xq", xq), ("xqt", xqt))}
    sa, sw, sx = scal(ia), scal(iw), scal(ix)
    dx, dw = fp8.gemm_backward(d["dyq"], d["dyqt"], E5M2, d["wqt"], d["xqt"], sa, sw, sx)
    dx1 = fp8.gemm_dgrad(d["dyq"], E5M2, d["wqt"], sa, sw)
    dw1 = fp8.gemm_wgrad(d["dyqt"], E5M2, d["xqt"], sa, sx)
    dxm, dwm = fp8.gemm_backward_mn(d["dyq"], E5M2, d["wq"], d["xq"], sa, sw, sx)
    for what, x, y in (("dgrad vs separate", dx, dx1), ("wgrad vs separate", dw, dw1),
                       ("dgrad vs MN-major pair", dx, dxm), ("wgrad vs MN-major pair", dw, dwm)):
        bad = np.argwhere(u16(x) != u16(y))
        assert bad.size == 0, (what, bad[:4].tolist())
    check_full(orc, dx, dyq, E5M2, wqt, ia, iw, "mixed-length pair dgrad")
    check_full(orc, dw, dyqt, E5M2, xqt, ia, ix, "mixed-length pair wgrad")


def test_backward_pair_mn_every_output(fp8, orc):
    M, N, K = 2048, 2560, 4096
    say("gemm full output backward pair MN-major", M, N, K)
    g = torch.Generator(device="cpu").manual_seed(11)
    dyq, wq, xq = pair_operands(g, M, N, K, E5M2)
    ia, iw, ix = INV_A[E5M2], np.float32(1 / 448.0), INV_B
    dx, dw = fp8.gemm_backward_mn(dev(torch.from_numpy(dyq)), E5M2, dev(torch.from_numpy(wq)),
                                  dev(torch.from_numpy(xq)), scal(ia), scal(iw), scal(ix))
    check_full(orc, dx, dyq, E5M2, np.ascontiguousarray(wq.T), ia, iw, "MN pair dgrad")
    check_full(orc, dw, np.ascontiguousarray(dyq.T), E5M2, np.ascontiguousarray(xq.T), ia, ix, "MN pair wgrad")


def test_gate_up_every_output(fp8, orc):
    """16 x 18 = 288 gate/up tiles (128 gate + 128 up columns each): a round and a
    half-tile round; gu compared in full and absmax_h bit-exact with the oracle's
    SwiGLU statistic of the GPU's own gu."""
    M, F, K = 4096, 2304, 1024
    say("gemm full output gate/up", M, F, K)
    g = torch.Generator(device="cpu").manual_seed(13)
    x, w = rand_codes(g, (M, K), E4M3), rand_codes(g, (2 * F, K), E4M3)
    ix, iw = np.float32(1 / 448.0), np.float32(1 / 448.0)
    am = torch.zeros(1, dtype=torch.float32, device="cuda")
    gu = fp8.gemm_fwd_swiglu_absmax(dev(torch.from_numpy(x)), dev(torch.from_numpy(w)), scal(ix), scal(iw), am)
    check_full(orc, gu, x, E4M3, w, ix, iw, "gate/up")
    _, _, am_r, _ = orc.swiglu_requant(u16(gu), want_hq=False)
    assert_f32_equal(am.item(), am_r, "gate/up absmax_h")


def nonfinite_compare(y_bits, ref_bits, what):
    """NaN exactly where the oracle has NaN, the same infinities, rel_F on the rest."""
    g, r = bf16_to_f64(y_bits), bf16_to_f64(ref_bits)
    assert np.array_equal(np.isnan(g), np.isnan(r)), (what, int(np.isnan(g).sum()), int(np.isnan(r).sum()))
    inf = np.isinf(r)
    assert np.array_equal(np.isinf(g), inf) and np.array_equal(g[inf], r[inf]), what
    fin = np.isfinite(r)
    rel = np.linalg.norm(g[fin] - r[fin]) / np.linalg.norm(r[fin])
    assert rel <= 5e-3, (what, rel)
    return int(np.isnan(r).sum()), int(inf.sum())


@pytest.mark.parametrize("entry", ["fwd", "backward"])
def test_nan_and_infinite_operand_codes(fp8, orc, entry):
    """NaN codes in A and B (e4m3 0x7F / 0xFF, e5m2 0x7E) and an e5m2 infinity
    (0x7C) with a zero partner in one column: the outputs of that row / column
    are NaN or infinite exactly as the oracle's, every other output finite and
    within tolerance.  Shapes span several tiles with a ragged edge."""
    P, Q, R = 1040, 784, 640
    say("gemm non-finite codes", entry, P, Q, R)
    g = torch.Generator(device="cpu").manual_seed(17)
    fa = E4M3 if entry == "fwd" else E5M2
    a, b = rand_codes(g, (P, R), fa), rand_codes(g, (Q, R), E4M3)
    a[5, 17] = 0x7F if fa == E4M3 else 0x7E          # NaN in row 5 of A
    b[300, 40] = 0xFF                                # NaN in row 300 of B (an output column)
    if fa == E5M2:
        a[777, 99] = 0x7C                            # +inf in row 777 ...
        b[:, 99] = np.where(np.arange(Q) % 3 == 0, 0x00, b[:, 99])   # ... times zeros in a third of the columns
    ia, ib = INV_A[fa], INV_B
    A, B = dev(torch.from_numpy(a)), dev(torch.from_numpy(b))
    if entry == "fwd":
        y = fp8.gemm_fwd(A, B, scal(ia), scal(ib))
    else:
        y = fp8.gemm_dgrad(A, fa, B, scal(ia), scal(ib))
    ref = orc.gemm(a, fa, b, E4M3, ia, ib)
    nans, infs = nonfinite_compare(u16(y), ref, entry)
    assert nans >= P + Q - 1
    if fa == E5M2:
        assert infs > 0
