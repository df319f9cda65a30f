"""GPU parity of the FP8 GEMMs (fwd / dgrad / wgrad) against the oracle.

* exact-arithmetic operands (small integers: every partial sum exact in fp32,
  so any summation order gives the same value) -> bit-exact;
* an identity right operand and all-ones operands (closed form K * da * db);
* random operands at shapes spanning several 256 x 256 tiles with ragged
  edges, both operand formats: relative Frobenius error <= 5e-3, and every
  output within the error bound of an fp32 sum in arbitrary order;
* the pages' shapes at full size on sampled rows;
* determinism: the same call twice gives identical bytes.
"""
import numpy as np
import pytest
import torch

from gpu_util import E4M3, E5M2, assert_within_sum_bound, dev, gemm_compare, say, u16

pytestmark = pytest.mark.gpu

TDT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}


@pytest.fixture(scope="module")
def fp8():
    import fp8_precision_amd
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return fp8_precision_amd


def codes_of(values: np.ndarray, fmt: int) -> np.ndarray:
    """Encode exactly representable values (test data only) via torch's CPU cast."""
    return torch.from_numpy(values.astype(np.float32)).to(TDT[fmt]).view(torch.uint8).numpy()


def random_codes(rng, shape, fmt, sigma):
    return codes_of(rng.standard_normal(shape) * sigma, fmt)


def scal(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def run(fp8, entry, a, fa, b, inv_a, inv_b):
    """Call one entry point with TN operands a [P, R], b [Q, R]; returns bf16 [P, Q]."""
    A, B = dev(torch.from_numpy(a)), dev(torch.from_numpy(b))
    ia, ib = scal(inv_a), scal(inv_b)
    if entry == "fwd":
        return fp8.gemm_fwd(A, B, ia, ib)
    if entry == "dgrad":
        return fp8.gemm_dgrad(A, fa, B, ia, ib)
    return fp8.gemm_wgrad(A, fa, B, ia, ib)


ENTRIES = [("fwd", E4M3), ("dgrad", E5M2), ("wgrad", E5M2), ("dgrad", E4M3), ("wgrad", E4M3)]


@pytest.mark.parametrize("entry,fa", ENTRIES)
@pytest.mark.parametrize("P,Q,R", [(256, 256, 256), (384, 512, 1024), (128, 256, 256), (272, 528, 384)])
def test_exact_small_integers(fp8, orc, entry, fa, P, Q, R):
    say("gemm exact", entry, fa, P, Q, R)
    rng = np.random.default_rng(P + Q + R)
    a = codes_of(rng.integers(-4, 5, (P, R)), fa)
    b = codes_of(rng.integers(-3, 4, (Q, R)), E4M3)
    inv_a, inv_b = np.float32(0.25), np.float32(2.0 ** -5)
    y = u16(run(fp8, entry, a, fa, b, inv_a, inv_b))
    ref = orc.gemm(a, fa, b, E4M3, inv_a, inv_b)
    assert np.array_equal(y, ref)


def test_identity_and_ones(fp8, orc):
    say("gemm identity/ones")
    rng = np.random.default_rng(5)
    K = 256
    a = random_codes(rng, (256, K), E4M3, 60.0)
    eye = np.zeros((K, K), np.uint8)
    eye[np.arange(K), np.arange(K)] = 0x38
    y = u16(run(fp8, "fwd", a, E4M3, eye, np.float32(0.5), np.float32(0.75)))
    assert np.array_equal(y, orc.gemm(a, E4M3, eye, E4M3, np.float32(0.5), np.float32(0.75)))
    ones_a = np.full((128, 2048), 0x3C, np.uint8)   # 1.0 in e5m2
    ones_b = np.full((272, 2048), 0x38, np.uint8)   # 1.0 in e4m3
    y = u16(run(fp8, "wgrad", ones_a, E5M2, ones_b, np.float32(3.0), np.float32(0.1)))
    assert np.array_equal(y, orc.gemm(ones_a, E5M2, ones_b, E4M3, np.float32(3.0), np.float32(0.1)))
    assert len(np.unique(y)) == 1


@pytest.mark.parametrize("entry,fa", ENTRIES)
@pytest.mark.parametrize("P,Q,R", [(16, 16, 128), (128, 256, 256), (272, 528, 384), (512, 768, 1024),
                                   (1040, 272, 640), (768, 1280, 2048), (256, 512, 128), (528, 1008, 384)])
def test_random_shapes(fp8, orc, entry, fa, P, Q, R):
    say("gemm random", entry, fa, P, Q, R)
    rng = np.random.default_rng(P * 3 + Q * 5 + R)
    a = random_codes(rng, (P, R), fa, 40.0 if fa == E4M3 else 2000.0)
    b = random_codes(rng, (Q, R), E4M3, 40.0)
    inv_a, inv_b = np.float32(1 / 448.0), np.float32(0.0123)
    yt = run(fp8, entry, a, fa, b, inv_a, inv_b)
    y = u16(yt)
    ref = orc.gemm(a, fa, b, E4M3, inv_a, inv_b)
    gemm_compare(y, ref, f"{entry} {P}x{Q}x{R}")
    assert_within_sum_bound(y, ref, a, fa, b, E4M3, inv_a, inv_b, np.arange(P), f"{entry} {P}x{Q}x{R}")
    # determinism
    y2 = u16(run(fp8, entry, a, fa, b, inv_a, inv_b))
    assert np.array_equal(y, y2)


# Launches whose last round is balanced with 128-row half tiles: 17 x 16 tiles
# (a full round of 256, then the 16 tiles of the last tile row as 32 halves),
# with an exact and a ragged last tile row, even and odd reductions.
@pytest.mark.parametrize("entry,fa", [("fwd", E4M3), ("wgrad", E5M2)])
@pytest.mark.parametrize("P,Q,R", [(4352, 4096, 256), (4304, 4096, 384), (4208, 4000, 128)])
def test_balanced_last_round(fp8, orc, entry, fa, P, Q, R):
    say("gemm balanced tail", entry, fa, P, Q, R)
    rng = np.random.default_rng(P + Q + R + fa)
    a = random_codes(rng, (P, R), fa, 40.0 if fa == E4M3 else 2000.0)
    b = random_codes(rng, (Q, R), E4M3, 40.0)
    inv_a, inv_b = np.float32(1 / 448.0), np.float32(0.0123)
    y = u16(run(fp8, entry, a, fa, b, inv_a, inv_b))
    # every row of the last tile row (the half tiles) and of its neighbour, plus a sample
    rows = np.unique(np.concatenate([np.arange(4096 - 64, P), np.random.default_rng(2).integers(0, 4096, 64)]))
    ref = orc.gemm(a, fa, b, E4M3, inv_a, inv_b, rows=rows.astype(np.int64))
    gemm_compare(y[rows], ref, f"{entry} {P}x{Q}x{R}")
    assert_within_sum_bound(y[rows], ref, a, fa, b, E4M3, inv_a, inv_b, rows.astype(np.int64), f"{entry} {P}x{Q}x{R}")
    # rows computed by half tiles are bit-identical to the same rows computed by
    # full tiles: put the last 256 rows first in a 4096-row launch (exactly one
    # full round of 16 x 16 tiles, nothing split)
    a2 = np.ascontiguousarray(np.concatenate([a[P - 256:], a[:4096 - 256]]))
    y2 = u16(run(fp8, entry, a2, fa, b, inv_a, inv_b))
    assert np.array_equal(y[P - 256:], y2[:256])


FULL = [
    ("7B gate/up fwd", "fwd", E4M3, 4096, 22016, 4096),
    ("7B down fwd", "fwd", E4M3, 4096, 4096, 11008),
    ("7B qkv dgrad", "dgrad", E5M2, 4096, 4096, 12288),
    ("7B gate/up wgrad", "wgrad", E5M2, 22016, 4096, 4096),
    ("14B down dgrad", "dgrad", E5M2, 8192, 13824, 5120),
    ("32B qkv wgrad", "wgrad", E5M2, 7168, 5120, 16384),
]


@pytest.mark.parametrize("name,entry,fa,P,Q,R", FULL)
def test_full_size_sampled_rows(fp8, orc, name, entry, fa, P, Q, R):
    say("gemm full", name, P, Q, R)
    g = torch.Generator(device="cpu").manual_seed(P + Q + R)
    # operands: decoded values ~N(0, sigma) encoded by torch's cast (test data only)
    a = torch.randn((P, R), generator=g).mul_(60.0 if fa == E4M3 else 3000.0).to(TDT[fa]).view(torch.uint8)
    b = torch.randn((Q, R), generator=g).mul_(60.0).to(TDT[E4M3]).view(torch.uint8)
    inv_a, inv_b = np.float32(1 / 448.0), np.float32(1 / 448.0)
    yt = run(fp8, entry, a.numpy(), fa, b.numpy(), inv_a, inv_b)
    rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(P - 8, P),
                                     np.random.default_rng(1).integers(0, P, 48)])).astype(np.int64)
    y = u16(yt)[rows]
    ref = orc.gemm(a.numpy(), fa, b.numpy(), E4M3, inv_a, inv_b, rows=rows)
    gemm_compare(y, ref, name)
    assert_within_sum_bound(y, ref, a.numpy(), fa, b.numpy(), E4M3, inv_a, inv_b, rows, name)


@pytest.mark.parametrize("M,N,K", [(4096, 12288, 4096), (256, 512, 384), (4096, 4096, 11008), (128, 256, 256)])
def test_backward_pair_matches_separate_calls(fp8, orc, M, N, K):
    """fp8_gemm_backward gives exactly the bytes of fp8_gemm_dgrad and fp8_gemm_wgrad."""
    say("gemm backward pair", M, N, K)
    g = torch.Generator(device="cpu").manual_seed(M + N + K)
    dyq = torch.randn((M, N), generator=g).mul_(3000.0).to(TDT[E5M2]).view(torch.uint8)
    wqt = torch.randn((K, N), generator=g).mul_(60.0).to(TDT[E4M3]).view(torch.uint8)
    xqt = torch.randn((K, M), generator=g).mul_(60.0).to(TDT[E4M3]).view(torch.uint8)
    dyqt = dyq.t().contiguous()
    d = lambda t: dev(t)
    ia, ib, ic = scal(1 / 57344.0), scal(1 / 448.0), scal(0.0123)
    dx, dw = fp8.gemm_backward(d(dyq), d(dyqt), E5M2, d(wqt), d(xqt), ia, ib, ic)
    dx2 = fp8.gemm_dgrad(d(dyq), E5M2, d(wqt), ia, ib)
    dw2 = fp8.gemm_wgrad(d(dyqt), E5M2, d(xqt), ia, ic)
    assert torch.equal(dx.view(torch.int16), dx2.view(torch.int16))
    assert torch.equal(dw.view(torch.int16), dw2.view(torch.int16))
    rows = np.array([0, M // 2, M - 1], np.int64)
    ref = orc.gemm(dyq.numpy(), E5M2, wqt.numpy(), E4M3, np.float32(1 / 57344.0), np.float32(1 / 448.0), rows=rows)
    gemm_compare(u16(dx)[rows], ref, "backward dgrad rows")


def test_binding_refuses_host_or_empty_scalars(fp8):
    """The inverse scales and statistics are device fp32 scalars: a host tensor
    (whose address a kernel could not read) or an empty one is refused by the
    binding before anything is launched."""
    say("binding scalar checks")
    xq = torch.zeros((256, 256), dtype=torch.uint8, device="cuda")
    wq = torch.zeros_like(xq)
    one = scal(1.0)
    host = torch.ones(1, dtype=torch.float32)
    empty = torch.empty(0, dtype=torch.float32, device="cuda")
    with pytest.raises(TypeError):
        fp8.gemm_fwd(xq, wq, host, one)
    with pytest.raises(ValueError):
        fp8.gemm_fwd(xq, wq, one, empty)
    with pytest.raises(TypeError):
        fp8.gemm_dgrad(xq, E5M2, wq, one, host)
    with pytest.raises(TypeError):
        fp8.gemm_wgrad(xq, E5M2, wq, host, one)
    with pytest.raises(TypeError):
        fp8.gemm_backward(xq, xq, E5M2, wq, wq, one, one, host)
    with pytest.raises(TypeError):
        fp8.gemm_backward_mn(xq, E5M2, wq, wq, one, host, one)
    x = torch.zeros((16, 16), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        fp8.quantize(x, E4M3, empty)
    with pytest.raises(TypeError):
        fp8.quantize(x, E4M3, torch.zeros(1, dtype=torch.float64, device="cuda"))
    torch.cuda.synchronize()
