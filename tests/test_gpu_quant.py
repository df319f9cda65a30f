"""GPU parity of fp8_absmax and fp8_quantize against the oracle (bit-exact).

* absmax: ragged lengths (including n < 8 and n % 8 != 0), planted maxima,
  -0, infinities, NaN, subnormals; the running (accumulating) form over pieces
  and prior values;
* the scale and inverse scale for every positive finite bf16 absmax;
* every bf16 input pattern quantised under a set of retained absmax values
  (fresh, stale, zero, tiny -> clamped scale, huge, inf, NaN), both formats,
  with and without the transposed copy;
* random tensors whose shapes span several tiles with ragged tails.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import E4M3, E5M2, assert_codes_equal, assert_f32_equal, dev, say, scalar, u16, u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8():
    import fp8_precision_amd
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return fp8_precision_amd


@pytest.mark.parametrize("n", [1, 2, 7, 8, 9, 15, 17, 255, 1024, 4097, 65536 * 3 + 5, (1 << 22) + 3, 33554432])
def test_absmax_lengths(fp8, orc, n):
    say("absmax", n)
    x = workloads.draw(100, n % 997, (n,), 1.0)
    bits = u16(x)
    if n > 3:
        bits[n // 3] = 0xC4E0       # -1792, planted (negative) maximum
        bits[-1] = 0x44DF           # a large positive value in the ragged tail
    xt = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    got = scalar(fp8.absmax(dev(xt)))
    torch.cuda.synchronize()
    assert_f32_equal(got, orc.absmax_bf16(bits), f"absmax n={n}")


def test_absmax_special_values(fp8, orc):
    base = np.zeros(4099, np.uint16)
    cases = {
        "zeros": [],
        "neg_zero": [(5, 0x8000)],
        "subnormal": [(7, 0x0001), (4000, 0x8003)],
        "neg_inf": [(11, 0xFF80)],
        "pos_inf_tail": [(4098, 0x7F80)],
        "nan": [(13, 0x7FC1), (14, 0x3F80)],
        "neg_nan": [(4097, 0xFFC0)],
    }
    for name, sets in cases.items():
        say("absmax special", name)
        b = base.copy()
        for i, v in sets:
            b[i] = v
        xt = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16)
        got = scalar(fp8.absmax(dev(xt)))
        assert_f32_equal(got, orc.absmax_bf16(b), name)


def test_absmax_accumulate(fp8, orc):
    """fp8_absmax_accumulate: a tensor in pieces gives the whole tensor's absmax;
    a prior value is kept when larger (NaN and +inf stay); neighbours untouched."""
    n = 3 * 65536 + 40
    x = workloads.draw(101, 7, (n,), 1.0)
    bits = u16(x)
    bits[70000] = 0xC2F6                                     # -123, the planted maximum
    whole = orc.absmax_bf16(bits)
    xd = dev(torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16))
    stats = torch.full((5,), -7.0, dtype=torch.float32, device="cuda")
    stats[2] = 0.0
    cuts = [0, 65536, 65536 + 1000, n]                        # 16-byte aligned piece starts
    for a, b in zip(cuts[:-1], cuts[1:]):
        fp8.absmax(xd[a:b], out=stats[2:3], accumulate=True)
    torch.cuda.synchronize()
    got = stats.cpu().numpy()
    assert_f32_equal(got[2], whole, "pieces")
    assert np.all(got[[0, 1, 3, 4]] == -7.0), "neighbouring statistics changed"
    say("absmax accumulate priors")
    for prior, want in [(1e6, np.float32(1e6)), (1.0, whole), (0.0, whole),
                        (float("inf"), np.float32("inf")), (float("nan"), None)]:
        o = torch.tensor([prior], dtype=torch.float32, device="cuda")
        fp8.absmax(xd, out=o, accumulate=True)
        r = scalar(o)
        if want is None:
            assert np.isnan(r)
        else:
            assert_f32_equal(r, want, f"prior {prior}")
    # a NaN in the data wins over any prior, as in fp8_absmax
    b2 = bits.copy()
    b2[5] = 0x7FC1
    o = torch.tensor([1e30], dtype=torch.float32, device="cuda")
    fp8.absmax(dev(torch.from_numpy(b2.view(np.int16).copy()).view(torch.bfloat16)), out=o, accumulate=True)
    assert np.isnan(scalar(o))
    with pytest.raises(ValueError):
        fp8.absmax(xd, accumulate=True)


def test_absmax_accumulate_many(fp8, orc):
    """Up to 8 tensors in one launch: each slot gets its tensor's absmax (sizes
    from a ragged 37 elements to 48 M, below and above the non-temporal
    threshold), a shared slot gets the maximum of its tensors, priors stay."""
    say("absmax many")
    sizes = [37, 1 << 20, 3 * (1 << 24) + 5, 4096 * 4096]
    xs, bits = [], []
    for k, n in enumerate(sizes):
        b = u16(workloads.draw(102, k, (n,), 1.0 + k))
        b[(n * 2) // 3] = 0xC300 + 16 * k                     # a planted negative maximum per tensor
        bits.append(b)
        xs.append(dev(torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16)))
    want = [orc.absmax_bf16(b) for b in bits]
    slots = torch.zeros(6, dtype=torch.float32, device="cuda")
    fp8.absmax_accumulate_many(xs, [slots[i:i + 1] for i in range(4)])
    torch.cuda.synchronize()
    got = slots.cpu().numpy()
    for i in range(4):
        assert_f32_equal(got[i], want[i], f"tensor {i} (n={sizes[i]})")
    assert got[4] == 0 and got[5] == 0
    # two tensors into one slot, a larger prior in another
    s2 = torch.tensor([0.0, 1e30], dtype=torch.float32, device="cuda")
    fp8.absmax_accumulate_many([xs[0], xs[3], xs[1]], [s2[0:1], s2[0:1], s2[1:2]])
    torch.cuda.synchronize()
    r = s2.cpu().numpy()
    assert_f32_equal(r[0], max(np.float32(want[0]), np.float32(want[3])), "shared slot")
    assert_f32_equal(r[1], np.float32(1e30), "larger prior")
    # eight tensors in one launch (the largest count), each into its own slot
    s8 = torch.zeros(8, dtype=torch.float32, device="cuda")
    xs8 = xs + xs[:3] + [xs[2]]
    fp8.absmax_accumulate_many(xs8, [s8[i:i + 1] for i in range(8)])
    torch.cuda.synchronize()
    r8 = s8.cpu().numpy()
    for i, k in enumerate([0, 1, 2, 3, 0, 1, 2, 2]):
        assert_f32_equal(r8[i], want[k], f"eight tensors, slot {i}")
    with pytest.raises(ValueError):
        fp8.absmax_accumulate_many(xs8 + xs[:1], [s8[i:i + 1] for i in range(8)] + [slots[0:1]])


def test_absmax_clear(fp8, orc):
    """fp8_absmax_clear sets exactly its slots to +0 (600 of them: three
    256-lane blocks, the last one partial) and leaves the neighbours alone; a
    statistic accumulated after it equals the tensor's fresh absmax."""
    say("absmax clear")
    buf = torch.full((700,), -3.5, dtype=torch.float32, device="cuda")   # sign bit set
    fp8.absmax_clear(buf[5:605])
    torch.cuda.synchronize()
    r = buf.cpu().numpy()
    assert (r[5:605] == 0).all() and not np.signbit(r[5:605]).any()
    assert (r[:5] == -3.5).all() and (r[605:] == -3.5).all()
    b = u16(workloads.draw(103, 0, (4097,), 2.0))
    x = dev(torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16))
    fp8.absmax(x, buf[7:8], accumulate=True)
    torch.cuda.synchronize()
    assert_f32_equal(buf[7:8].cpu().numpy()[0], orc.absmax_bf16(b), "accumulated after the clear")
    with pytest.raises(ValueError):
        fp8.absmax_clear(buf[:0])


def test_quantize_many(fp8, orc):
    """Up to 8 tensors in one launch, each bit-identical to its own fp8_quantize
    call and to the oracle: mixed formats, q only / qt only / both, ragged
    multiples of 16 spanning several 128 x 128 tiles, one input of 64 MiB
    (read non-temporally) next to small ones, a retained (stale) statistic;
    and the same bytes with the transposed copies marked as read later."""
    shapes = [(144, 272), (4096, 8192), (16, 16), (400, 1040), (272, 144), (1024, 2048), (128, 128), (48, 4112)]
    fmts = [E4M3, E5M2, E4M3, E5M2, E4M3, E4M3, E5M2, E4M3]
    want_q = [True, True, False, True, True, False, True, True]
    want_qt = [True, True, True, False, True, True, True, False]
    say("quantize many", len(shapes))
    xs, bits, amaxs = [], [], []
    for k, (r, c) in enumerate(shapes):
        x = workloads.draw(103, k, (r, c), 1.0 if fmts[k] == E4M3 else 1e-3)
        bits.append(u16(x))
        xs.append(dev(x))
        amaxs.append(fp8.absmax(xs[-1]))
    amaxs[3] = amaxs[3] * 0.25              # a stale statistic: some codes saturate
    qs, qts, scs, invs = fp8.quantize_many(xs, fmts, amaxs, want_q=want_q, want_qt=want_qt)
    torch.cuda.synchronize()
    for k, (r, c) in enumerate(shapes):
        what = f"tensor {k} {r}x{c} fmt {fmts[k]}"
        am = scalar(amaxs[k])
        s_ref, inv_ref = orc.scale(am, fmts[k])
        assert_f32_equal(scalar(scs[k]), s_ref, what + " scale")
        assert_f32_equal(scalar(invs[k]), inv_ref, what + " inv")
        q_ref, _ = orc.quantize(bits[k], fmts[k], s_ref)
        assert (qs[k] is not None) == want_q[k] and (qts[k] is not None) == want_qt[k]
        if want_q[k]:
            assert_codes_equal(u8(qs[k]), q_ref, fmts[k], what + " q")
        if want_qt[k]:
            assert_codes_equal(u8(qts[k]), q_ref.T.copy(), fmts[k], what + " qt")
        q1, qt1, _, _ = fp8.quantize(xs[k], fmts[k], amaxs[k], want_q=want_q[k], want_qt=want_qt[k])
        if want_q[k]:
            assert torch.equal(q1, qs[k]), what + " vs fp8_quantize"
        if want_qt[k]:
            assert torch.equal(qt1, qts[k]), what + " vs fp8_quantize (qt)"
    # the transposed copies marked as read later (non-temporal stores): every other
    # tensor (two launches, one per kind), then all of them (one launch) -- same bytes
    for later in ([k % 2 == 0 for k in range(len(shapes))], True):
        qs2, qts2, scs2, invs2 = fp8.quantize_many(xs, fmts, amaxs, want_q=want_q, want_qt=want_qt, qt_later=later)
        torch.cuda.synchronize()
        for k in range(len(shapes)):
            what = f"tensor {k} qt_later {later}"
            if want_q[k]:
                assert torch.equal(qs2[k], qs[k]), what + " q"
            if want_qt[k]:
                assert torch.equal(qts2[k], qts[k]), what + " qt"
            assert torch.equal(scs2[k], scs[k]) and torch.equal(invs2[k], invs[k]), what + " scales"
    with pytest.raises(fp8.Fp8Error):     # rows % 16 != 0 in one entry: refused before any launch
        fp8.quantize_many([xs[0], torch.zeros((8, 16), dtype=torch.bfloat16, device="cuda")], E4M3, amaxs[0])


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_scale_every_bf16_absmax(fp8, orc, fmt):
    say("scale sweep", fmt)
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    amax = torch.from_numpy(((bits.astype(np.uint32) << 16).view(np.float32)).copy()).cuda()
    x = torch.zeros((16, 16), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((16, 16), dtype=torch.uint8, device="cuda")
    sc = torch.empty(bits.size, dtype=torch.float32, device="cuda")
    inv = torch.empty(bits.size, dtype=torch.float32, device="cuda")
    for i in range(bits.size):
        fp8.quantize(x, fmt, amax[i:i + 1], q=q, scale=sc[i:i + 1], inv_scale=inv[i:i + 1])
    s_gpu, i_gpu = sc.cpu().numpy(), inv.cpu().numpy()
    a = amax.cpu().numpy()
    for i in range(0, bits.size, 1):
        s_ref, i_ref = orc.scale(a[i], fmt)
        if s_gpu[i].view(np.uint32) != np.float32(s_ref).view(np.uint32) or \
                i_gpu[i].view(np.uint32) != np.float32(i_ref).view(np.uint32):
            raise AssertionError(f"absmax {a[i]!r}: gpu ({s_gpu[i]!r}, {i_gpu[i]!r}) oracle ({s_ref!r}, {i_ref!r})")


RETAINED = [0.0, 1e-45, 1e-40, 1.1754944e-38, 1e-37, 1.3e-36, 2.0 ** -20, 0.5, 1.0, 3.0, 448.0, 1000.0,
            57344.0, 1.0e5, 3.3e38, np.finfo(np.float32).max, np.inf, np.nan]


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_every_bf16_pattern_under_retained_scales(fp8, orc, fmt):
    all_bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(4096, 16)
    x = dev(torch.from_numpy(all_bits.view(np.int16).copy()).view(torch.bfloat16))
    rng = np.random.default_rng(42)
    values = RETAINED + list(rng.uniform(1e-3, 1e3, 12))
    for a in values:
        say("retained", fmt, a)
        amax = torch.tensor([a], dtype=torch.float32, device="cuda")
        q, qt, s, inv = fp8.quantize(x, fmt, amax, want_q=True, want_qt=True)
        s_ref, inv_ref = orc.scale(np.float32(a), fmt)
        assert_f32_equal(scalar(s), s_ref, f"scale {a}")
        assert_f32_equal(scalar(inv), inv_ref, f"inv {a}")
        q_ref, _ = orc.quantize(all_bits, fmt, s_ref)
        assert_codes_equal(u8(q), q_ref, fmt, f"q absmax={a}")
        assert_codes_equal(u8(qt), q_ref.T.copy(), fmt, f"qt absmax={a}")
        q_only, _, _, _ = fp8.quantize(x, fmt, amax, want_q=True, want_qt=False)
        assert_codes_equal(u8(q_only), q_ref, fmt, f"q (flat kernel) absmax={a}")


SHAPES = [(1, 16), (3, 48), (16, 16), (48, 528), (64, 512), (80, 1040), (144, 4112), (130, 2064),
          (2048, 1008), (16, 65536)]


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("shape", SHAPES)
def test_quantize_shapes(fp8, orc, fmt, shape):
    rows, cols = shape
    say("quantize", fmt, shape)
    sigma = 1.0 if fmt == E4M3 else 1e-3
    x = workloads.draw(7, rows * 31 + cols, shape, sigma)
    bits = u16(x)
    xd = dev(x)
    amax = fp8.absmax(xd)
    want_qt = rows % 16 == 0
    q, qt, s, inv = fp8.quantize(xd, fmt, amax, want_q=True, want_qt=want_qt)
    am_ref = orc.absmax_bf16(bits)
    assert_f32_equal(scalar(amax), am_ref, "absmax")
    s_ref, inv_ref = orc.scale(am_ref, fmt)
    assert_f32_equal(scalar(s), s_ref, "scale")
    assert_f32_equal(scalar(inv), inv_ref, "inv")
    q_ref, _ = orc.quantize(bits, fmt, s_ref)
    assert_codes_equal(u8(q), q_ref, fmt, "q")
    if want_qt:
        assert_codes_equal(u8(qt), q_ref.T.copy(), fmt, "qt")
        _, qt_only, _, _ = fp8.quantize(xd, fmt, amax, want_q=False, want_qt=True)
        assert_codes_equal(u8(qt_only), q_ref.T.copy(), fmt, "qt only")


def test_quantize_rejects_bad_arguments(fp8):
    x = torch.zeros((16, 24), dtype=torch.bfloat16, device="cuda")
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    with pytest.raises(fp8.Fp8Error):
        fp8.quantize(x, E4M3, amax)          # cols % 16 != 0
    x = torch.zeros((8, 16), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fp8.Fp8Error):
        fp8.quantize(x, E4M3, amax, want_qt=True)   # rows % 16 != 0 with qt


def test_absmax_every_loop_region(fp8, orc):
    """One planted maximum at a time in each region of the single pass: the
    first vector, the last vector of the unrolled part, the remainder vectors
    past it, the last full vector and the ragged tail -- at lengths whose
    vector count is not a multiple of the unrolled step, for a full-chip grid
    (1024 lanes per CU) and for small grids."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stride = cus * 1024                                    # 16-byte vectors per full-grid step
    lengths = [8 * (2 * stride + stride // 2) + 5,         # one unrolled step, half a step of remainder
               8 * (4 * stride + 1) + 7,                   # two steps and one remainder vector
               8 * (3 * stride - 3),                       # one step, then most of another by remainders
               8 * 3000 + 3, 8 * 8193 + 1]                 # one- and two-block grids
    for n in lengths:
        nvec = n // 8
        base = u16(workloads.draw(103, n % 991, (n,), 1.0))
        xd = dev(torch.from_numpy(base.view(np.int16).copy()).view(torch.bfloat16))
        spots = sorted({0, min(nvec - 1, 2 * stride - 1) * 8 + 3, min(nvec - 1, 2 * stride) * 8 + 6,
                        (nvec - 1) * 8 + 1, n - 1})
        for p in spots:
            say("absmax region", n, p)
            b = base.copy()
            b[p] = 0xC580                                   # -4096: larger than every drawn value
            xd[p] = torch.tensor(-4096.0, dtype=torch.bfloat16)
            got = scalar(fp8.absmax(xd))
            assert_f32_equal(got, orc.absmax_bf16(b), f"absmax n={n} max at {p}")
            xd[p] = torch.from_numpy(base[p:p + 1].view(np.int16).copy()).view(torch.bfloat16).cuda()[0]
