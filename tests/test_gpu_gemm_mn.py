"""GPU parity of the backward GEMMs on untransposed (MN-major) FP8 operands.

fp8_gemm_dgrad_mn reads W [N, K] and fp8_gemm_wgrad_mn reads dY [M, N] and
X [M, K] as stored, through LDS transpose reads.  Checked against:
* the oracle (the same product written out, on the transposed operands):
  bit-exact on exact-arithmetic operands, relative Frobenius error <= 5e-3 and
  the fp32 summation bound on random operands, at ragged shapes that span
  several tiles and at the pages' full sizes on sampled rows;
* the transposed-copy entry points: both layouts feed the matrix instructions
  the same bytes in the same order, so the outputs must be identical;
* determinism, and fp8_gemm_backward_mn against the two separate calls.
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


def scal(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def codes(values: np.ndarray, fmt: int) -> np.ndarray:
    """Encode exactly representable values (test data only) via torch's CPU cast."""
    return torch.from_numpy(values.astype(np.float32)).to(TDT[fmt]).view(torch.uint8).numpy()


def rand_codes(g, shape, fmt, sigma):
    return torch.randn(shape, generator=g).mul_(sigma).to(TDT[fmt]).view(torch.uint8).numpy()


def run_mn(fp8, entry, dyq, fa, other, ia, ib):
    """dgrad: (dyq [M, N], wq [N, K]) -> [M, K]; wgrad: (dyq [M, N], xq [M, K]) -> [N, K]."""
    D, O = dev(torch.from_numpy(np.ascontiguousarray(dyq))), dev(torch.from_numpy(np.ascontiguousarray(other)))
    if entry == "dgrad":
        return fp8.gemm_dgrad_mn(D, fa, O, scal(ia), scal(ib))
    return fp8.gemm_wgrad_mn(D, fa, O, scal(ia), scal(ib))


def tn_operands(entry, dyq, other):
    """The same product in the oracle's TN form out = A . B^T."""
    if entry == "dgrad":
        return dyq, np.ascontiguousarray(other.T)          # A = dY [M, N], B = W^T [K, N]
    return np.ascontiguousarray(dyq.T), np.ascontiguousarray(other.T)   # A = dY^T [N, M], B = X^T [K, M]


SHAPES = [(256, 256, 256), (128, 256, 384), (272, 528, 384), (512, 768, 1024), (1040, 272, 640),
          (768, 1280, 2048), (16, 16, 128), (384, 144, 256)]


def reducible(entry, shapes):
    """(entry, M, N, K) cases whose reduction length (N for dgrad, M for wgrad) is
    a multiple of 128, as the MN-major entry points require."""
    return [(entry, M, N, K) for M, N, K in shapes if (N if entry == "dgrad" else M) % 128 == 0]


EXACT_SHAPES = [(256, 256, 256), (128, 384, 256), (272, 384, 528), (384, 128, 144)]


@pytest.mark.parametrize("entry,M,N,K", reducible("dgrad", EXACT_SHAPES) + reducible("wgrad", EXACT_SHAPES))
@pytest.mark.parametrize("fa", [E5M2, E4M3])
def test_exact_small_integers(fp8, orc, entry, fa, M, N, K):
    say("gemm_mn exact", entry, fa, M, N, K)
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    dyq = codes(rng.integers(-4, 5, (M, N)), fa)
    other = codes(rng.integers(-3, 4, (N, K) if entry == "dgrad" else (M, K)), E4M3)
    ia, ib = np.float32(0.25), np.float32(2.0 ** -5)
    y = u16(run_mn(fp8, entry, dyq, fa, other, ia, ib))
    A, B = tn_operands(entry, dyq, other)
    assert np.array_equal(y, orc.gemm(A, fa, B, E4M3, ia, ib))


@pytest.mark.parametrize("entry,M,N,K", reducible("dgrad", SHAPES) + reducible("wgrad", SHAPES))
@pytest.mark.parametrize("fa", [E5M2, E4M3])
def test_random_and_identical_to_transposed_path(fp8, orc, entry, fa, M, N, K):
    say("gemm_mn random", entry, fa, M, N, K)
    g = torch.Generator(device="cpu").manual_seed(M * 3 + N * 5 + K * 7 + fa)
    dyq = rand_codes(g, (M, N), fa, 40.0 if fa == E4M3 else 2000.0)
    other = rand_codes(g, (N, K) if entry == "dgrad" else (M, K), E4M3, 40.0)
    ia, ib = np.float32(1 / 448.0), np.float32(0.0123)
    yt = run_mn(fp8, entry, dyq, fa, other, ia, ib)
    y = u16(yt)
    A, B = tn_operands(entry, dyq, other)
    # the transposed-copy entry point on the same product: identical bytes
    At, Bt = dev(torch.from_numpy(A)), dev(torch.from_numpy(B))
    if entry == "dgrad":
        y_t = fp8.gemm_dgrad(At, fa, Bt, scal(ia), scal(ib))
    else:
        y_t = fp8.gemm_wgrad(At, fa, Bt, scal(ia), scal(ib))
    assert np.array_equal(y, u16(y_t)), "MN-major and transposed-copy paths differ"
    ref = orc.gemm(A, fa, B, E4M3, ia, ib)
    P = A.shape[0]
    gemm_compare(y, ref, f"{entry}_mn {M}x{N}x{K}")
    assert_within_sum_bound(y, ref, A, fa, B, E4M3, ia, ib, np.arange(P), f"{entry}_mn {M}x{N}x{K}")
    assert np.array_equal(y, u16(run_mn(fp8, entry, dyq, fa, other, ia, ib)))      # determinism


FULL = [
    ("7B qkv dgrad", "dgrad", 4096, 12288, 4096),
    ("7B gate/up dgrad", "dgrad", 4096, 22016, 4096),
    ("7B gate/up wgrad", "wgrad", 4096, 22016, 4096),
    ("7B down wgrad", "wgrad", 4096, 4096, 11008),
    ("14B down dgrad", "dgrad", 8192, 5120, 13824),
    ("32B qkv wgrad", "wgrad", 16384, 7168, 5120),
]


@pytest.mark.parametrize("name,entry,M,N,K", FULL)
def test_full_size_sampled_rows(fp8, orc, name, entry, M, N, K):
    say("gemm_mn full", name, M, N, K)
    g = torch.Generator(device="cpu").manual_seed(M + N + K)
    dyq = rand_codes(g, (M, N), E5M2, 3000.0)
    other = rand_codes(g, (N, K) if entry == "dgrad" else (M, K), E4M3, 60.0)
    ia, ib = np.float32(1 / 57344.0), np.float32(1 / 448.0)
    y = u16(run_mn(fp8, entry, dyq, E5M2, other, ia, ib))
    A, B = tn_operands(entry, dyq, other)
    P = A.shape[0]
    rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(P - 8, P),
                                     np.random.default_rng(2).integers(0, P, 40)])).astype(np.int64)
    ref = orc.gemm(A, E5M2, B, E4M3, ia, ib, rows=rows)
    gemm_compare(y[rows], ref, name)
    assert_within_sum_bound(y[rows], ref, A, E5M2, B, E4M3, ia, ib, rows, name)


@pytest.mark.parametrize("M,N,K", [(4096, 12288, 4096), (256, 512, 384), (4096, 4096, 11008), (128, 256, 144)])
def test_backward_mn_matches_separate_calls(fp8, orc, M, N, K):
    """fp8_gemm_backward_mn gives exactly the bytes of the two _mn calls and of fp8_gemm_backward."""
    say("gemm_mn backward pair", M, N, K)
    g = torch.Generator(device="cpu").manual_seed(M + 2 * N + 3 * K)
    dyq = torch.randn((M, N), generator=g).mul_(3000.0).to(TDT[E5M2]).view(torch.uint8)
    wq = torch.randn((N, K), generator=g).mul_(60.0).to(TDT[E4M3]).view(torch.uint8)
    xq = torch.randn((M, K), generator=g).mul_(60.0).to(TDT[E4M3]).view(torch.uint8)
    ia, ib, ic = scal(1 / 57344.0), scal(1 / 448.0), scal(0.0123)
    d = lambda t: dev(t.contiguous())
    dx, dw = fp8.gemm_backward_mn(d(dyq), E5M2, d(wq), d(xq), ia, ib, ic)
    dx2 = fp8.gemm_dgrad_mn(d(dyq), E5M2, d(wq), ia, ib)
    dw2 = fp8.gemm_wgrad_mn(d(dyq), E5M2, d(xq), ia, ic)
    assert torch.equal(dx.view(torch.int16), dx2.view(torch.int16))
    assert torch.equal(dw.view(torch.int16), dw2.view(torch.int16))
    dx3, dw3 = fp8.gemm_backward(d(dyq), d(dyq.t()), E5M2, d(wq.t()), d(xq.t()), ia, ib, ic)
    assert torch.equal(dx.view(torch.int16), dx3.view(torch.int16))
    assert torch.equal(dw.view(torch.int16), dw3.view(torch.int16))
    rows = np.array([0, M // 2, M - 1], np.int64)
    ref = orc.gemm(dyq.numpy(), E5M2, np.ascontiguousarray(wq.numpy().T), E4M3, np.float32(1 / 57344.0),
                   np.float32(1 / 448.0), rows=rows)
    gemm_compare(u16(dx)[rows], ref, "backward_mn dgrad rows")
