"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, and rejects invalid arguments with the documented status codes before
touching the GPU (no kernel is launched here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8_precision.h")
LIB = os.path.join(ROOT, "fp8_precision_amd", "libfp8_precision.so")

OK, INVALID, UNSUPPORTED = 0, 1, 2


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:fp8_status|const char\*)\s+(fp8_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} not built: run `python fp8_precision_amd/build.py`")
    lib = ctypes.CDLL(LIB)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.fp8_absmax.argtypes = [vp, i64, vp, vp]
    lib.fp8_absmax_accumulate.argtypes = [vp, i64, vp, vp]
    lib.fp8_absmax_accumulate_many.argtypes = [i32, vp, vp, vp, vp]
    lib.fp8_quantize.argtypes = [vp, i64, i64, i32, vp, vp, vp, vp, vp, vp]
    lib.fp8_swiglu_requant.argtypes = [vp, i64, i64, vp, i32, vp, vp, vp, vp]
    lib.fp8_gemm_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp]
    lib.fp8_gemm_fwd_swiglu_absmax.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, vp]
    lib.fp8_gemm_dgrad.argtypes = [vp, i32, vp, vp, vp, vp, i64, i64, i64, vp]
    lib.fp8_gemm_wgrad.argtypes = [vp, i32, vp, vp, vp, vp, i64, i64, i64, vp]
    lib.fp8_last_error.restype = ctypes.c_char_p
    lib.fp8_status_string.restype = ctypes.c_char_p
    for f in ("fp8_absmax", "fp8_absmax_accumulate", "fp8_absmax_accumulate_many", "fp8_absmax_clear", "fp8_quantize", "fp8_swiglu_requant", "fp8_gemm_fwd",
              "fp8_gemm_fwd_swiglu_absmax", "fp8_gemm_dgrad", "fp8_gemm_wgrad"):
        getattr(lib, f).restype = i32
    return lib


def test_header_declares_the_hot_path():
    names = declared_functions()
    for want in ("fp8_absmax", "fp8_absmax_accumulate", "fp8_absmax_accumulate_many", "fp8_quantize", "fp8_swiglu_requant", "fp8_gemm_fwd", "fp8_gemm_dgrad",
                 "fp8_gemm_wgrad", "fp8_gemm_fwd_swiglu_absmax", "fp8_gemm_backward", "fp8_gemm_dgrad_mn", "fp8_gemm_wgrad_mn",
                 "fp8_gemm_backward_mn", "fp8_swiglu_backward", "fp8_quantize_many", "fp8_status_string", "fp8_last_error"):
        assert want in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in range(4):
        assert lib.fp8_status_string(s)
    assert b"unknown" in lib.fp8_status_string(99)


# Fake but well-aligned device addresses: validation rejects the call before any
# HIP call, so they are never dereferenced.
A16 = 0x10000000
B16 = 0x20000000
C16 = 0x30000000
D16 = 0x40000000
E16 = 0x50000000


def test_absmax_validation(lib):
    assert lib.fp8_absmax(None, 16, C16, None) == INVALID
    assert lib.fp8_absmax(A16, 16, None, None) == INVALID
    assert lib.fp8_absmax(A16, 0, C16, None) == INVALID          # empty input
    assert lib.fp8_absmax(A16, -5, C16, None) == INVALID
    assert lib.fp8_absmax(A16, 16, A16 + 8, None) == INVALID     # output inside x
    assert b"overlaps" in lib.fp8_last_error()
    assert lib.fp8_absmax(A16 + 2, 16, C16, None) == UNSUPPORTED  # misaligned x
    assert lib.fp8_absmax(A16, 16, C16 + 1, None) == UNSUPPORTED


def test_absmax_accumulate_validation(lib):
    f = lib.fp8_absmax_accumulate
    assert f(None, 16, C16, None) == INVALID
    assert f(A16, 16, None, None) == INVALID
    assert f(A16, 0, C16, None) == INVALID
    assert f(A16, 16, A16 + 4, None) == INVALID
    assert b"fp8_absmax_accumulate" in lib.fp8_last_error()
    assert f(A16 + 8, 16, C16, None) == UNSUPPORTED
    assert f(A16, 16, C16 + 2, None) == UNSUPPORTED


def test_quantize_validation(lib):
    q = lib.fp8_quantize
    assert q(None, 16, 16, 0, C16, B16, None, None, None, None) == INVALID
    assert q(A16, 16, 16, 0, None, B16, None, None, None, None) == INVALID
    assert q(A16, 16, 16, 0, C16, None, None, None, None, None) == INVALID     # no output
    assert q(A16, 16, 16, 2, C16, B16, None, None, None, None) == INVALID      # bad format
    assert q(A16, 0, 16, 0, C16, B16, None, None, None, None) == INVALID       # empty
    assert q(A16, 16, 0, 0, C16, B16, None, None, None, None) == INVALID
    assert q(A16, 16, 16, 0, C16, A16 + 64, None, None, None, None) == INVALID  # q inside x
    assert q(A16, 16, 16, 0, C16, B16, B16 + 128, None, None, None) == INVALID  # q and qt overlap
    assert q(A16, 16, 24, 0, C16, B16, None, None, None, None) == UNSUPPORTED  # cols % 16
    assert q(A16, 8, 16, 0, C16, None, D16, None, None, None) == UNSUPPORTED   # rows % 16 with qt
    assert q(A16, 16, 16, 0, C16, B16 + 8, None, None, None, None) == UNSUPPORTED  # misaligned q
    assert q(A16, 16, 16, 1, C16, B16, None, E16 + 2, None, None) == UNSUPPORTED   # misaligned scale


def test_swiglu_validation(lib):
    s = lib.fp8_swiglu_requant
    assert s(None, 16, 16, C16, 1, B16, None, None, None) == INVALID
    assert s(A16, 16, 16, None, 1, B16, None, None, None) == INVALID
    assert s(A16, 16, 16, C16, 1, None, None, None, None) == INVALID
    assert s(A16, 16, 16, C16, 3, B16, None, None, None) == INVALID          # compute_absmax in {0, 1, 2}
    assert s(A16, 16, 16, C16, -1, B16, None, None, None) == INVALID
    assert s(A16, 0, 16, C16, 1, B16, None, None, None) == INVALID
    assert s(A16, 16, 0, C16, 1, B16, None, None, None) == INVALID
    assert s(A16, 16, 16, A16 + 4, 1, B16, None, None, None) == INVALID       # absmax inside gu
    assert s(A16, 16, 24, C16, 1, B16, None, None, None) == UNSUPPORTED       # F % 16
    assert s(A16, 8, 16, C16, 0, None, D16, None, None) == UNSUPPORTED        # M % 16 with hqt
    assert s(A16, 16, 1 << 62, C16, 1, B16, None, None, None) == INVALID     # 2 F would overflow
    assert s(A16, 1 << 40, 1 << 40, C16, 1, B16, None, None, None) == INVALID


@pytest.mark.parametrize("entry", ["fwd", "dgrad", "wgrad"])
def test_gemm_validation(lib, entry):
    if entry == "fwd":
        call = lambda a, b, ia, ib, out, M, N, K: lib.fp8_gemm_fwd(a, b, ia, ib, out, M, N, K, None)
    elif entry == "dgrad":
        call = lambda a, b, ia, ib, out, M, N, K: lib.fp8_gemm_dgrad(a, 1, b, ia, ib, out, M, N, K, None)
    else:
        call = lambda a, b, ia, ib, out, M, N, K: lib.fp8_gemm_wgrad(a, 1, b, ia, ib, out, M, N, K, None)
    assert call(None, B16, C16, C16 + 4, D16, 128, 128, 128) == INVALID
    assert call(A16, B16, None, C16 + 4, D16, 128, 128, 128) == INVALID
    assert call(A16, B16, C16, C16 + 4, None, 128, 128, 128) == INVALID
    assert call(A16, B16, C16, C16 + 4, D16, 0, 128, 128) == INVALID
    assert call(A16, B16, C16, C16 + 4, A16, 128, 128, 128) == INVALID        # out aliases A
    assert call(A16, B16, C16, C16 + 4, D16, 136, 136, 136) == UNSUPPORTED    # not a multiple of 16 / 128
    # the reduction axis (K, N, M for fwd, dgrad, wgrad) must be a multiple of 128
    red = {"fwd": (128, 128, 192), "dgrad": (128, 192, 128), "wgrad": (192, 128, 128)}[entry]
    assert call(A16, B16, C16, C16 + 4, D16, *red) == UNSUPPORTED
    assert call(A16, B16, C16, C16 + 4, D16 + 4, 128, 128, 128) == UNSUPPORTED  # misaligned out
    assert call(A16 + 1, B16, C16, C16 + 4, D16, 128, 128, 128) == UNSUPPORTED
    # an operand of 2^31 bytes (A = 131072 rows of a 16384-byte reduction): 32-bit offsets
    big = {"fwd": (131072, 128, 16384), "dgrad": (131072, 16384, 128), "wgrad": (16384, 131072, 128)}[entry]
    far_a, far_b, far_out = 1 << 40, 2 << 40, 3 << 40
    assert call(far_a, far_b, C16, C16 + 4, far_out, *big) == UNSUPPORTED
    # dimensions whose products would overflow 64 bits are refused before any product is formed
    huge = 1 << 40
    for dims in ((huge, huge, huge), (16, huge, huge), (huge, 16, 128), (1 << 62, 1 << 62, 1 << 62)):
        assert call(far_a, far_b, C16, C16 + 4, far_out, *dims) == UNSUPPORTED


def test_backward_validation(lib):
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    f = lib.fp8_gemm_backward
    f.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, vp]
    f.restype = i32
    F16 = 0x60000000
    ok = (A16, B16, 1, C16, D16, E16, E16 + 4, E16 + 8, F16, F16 + (1 << 24), 256, 256, 256, None)
    bad = list(ok); bad[0] = None
    assert f(*bad) == INVALID
    bad = list(ok); bad[9] = F16 + 1024          # dw overlaps dx
    assert f(*bad) == INVALID
    bad = list(ok); bad[8] = B16                 # dx aliases dyqt
    assert f(*bad) == INVALID
    bad = list(ok); bad[2] = 5
    assert f(*bad) == INVALID
    bad = list(ok); bad[10] = 200                # M not a multiple of 16 / 128
    assert f(*bad) == UNSUPPORTED


@pytest.mark.parametrize("entry", ["dgrad_mn", "wgrad_mn"])
def test_gemm_mn_validation(lib, entry):
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    f = getattr(lib, "fp8_gemm_" + entry)
    f.argtypes = [vp, i32, vp, vp, vp, vp, i64, i64, i64, vp]
    f.restype = i32
    call = lambda a, b, ia, ib, out, M, N, K, fmt=1: f(a, fmt, b, ia, ib, out, M, N, K, None)
    assert call(None, B16, C16, C16 + 4, D16, 128, 128, 128) == INVALID
    assert call(A16, B16, C16, C16 + 4, None, 128, 128, 128) == INVALID
    assert call(A16, B16, C16, C16 + 4, D16, 128, 128, 128, fmt=3) == INVALID
    assert call(A16, B16, C16, C16 + 4, B16, 128, 128, 128) == INVALID       # out aliases B
    red = {"dgrad_mn": (128, 192, 128), "wgrad_mn": (192, 128, 128)}[entry]
    assert call(A16, B16, C16, C16 + 4, D16, *red) == UNSUPPORTED            # reduction % 128
    assert call(A16, B16, C16, C16 + 4, D16, 128, 128, 136) == UNSUPPORTED  # K % 16
    assert call(A16, B16 + 8, C16, C16 + 4, D16, 128, 128, 128) == UNSUPPORTED


def test_backward_mn_validation(lib):
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    f = lib.fp8_gemm_backward_mn
    f.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, vp]
    f.restype = i32
    F16 = 0x60000000
    ok = (A16, 1, C16, D16, E16, E16 + 4, E16 + 8, F16, F16 + (1 << 24), 256, 256, 256, None)
    bad = list(ok); bad[0] = None
    assert f(*bad) == INVALID
    bad = list(ok); bad[8] = F16 + 1024         # dw overlaps dx
    assert f(*bad) == INVALID
    bad = list(ok); bad[7] = C16                # dx aliases wq
    assert f(*bad) == INVALID
    bad = list(ok); bad[1] = 5
    assert f(*bad) == INVALID
    bad = list(ok); bad[9] = 200                # M not a multiple of 16 / 128
    assert f(*bad) == UNSUPPORTED


def test_swiglu_backward_validation(lib):
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    f = lib.fp8_swiglu_backward
    f.argtypes = [vp, vp, i64, i64, i32, vp, vp, vp, vp, vp, vp]
    f.restype = i32
    ok = (A16, B16, 16, 16, 1, C16, D16, None, None, None, None)
    bad = list(ok); bad[0] = None
    assert f(*bad) == INVALID
    bad = list(ok); bad[5] = None                 # absmax
    assert f(*bad) == INVALID
    bad = list(ok); bad[6] = None                 # neither q nor qt
    assert f(*bad) == INVALID
    bad = list(ok); bad[4] = 9
    assert f(*bad) == INVALID
    bad = list(ok); bad[6] = A16 + 32             # q inside gu
    assert f(*bad) == INVALID
    bad = list(ok); bad[3] = 24                   # F % 16
    assert f(*bad) == UNSUPPORTED
    bad = list(ok); bad[2] = 8; bad[7] = E16      # M % 16 with qt
    assert f(*bad) == UNSUPPORTED
    bad = list(ok); bad[1] = B16 + 8              # misaligned dh
    assert f(*bad) == UNSUPPORTED
    bad = list(ok); bad[3] = 1 << 62              # 2 F would overflow
    assert f(*bad) == INVALID


def test_bad_dy_format(lib):
    assert lib.fp8_gemm_dgrad(A16, 7, B16, C16, C16 + 4, D16, 128, 128, 128, None) == INVALID
    assert lib.fp8_gemm_wgrad(A16, -1, B16, C16, C16 + 4, D16, 128, 128, 128, None) == INVALID


def test_python_binding_imports_and_fails_loudly_without_gpu():
    import torch
    import fp8_precision_amd as fp8
    assert set(fp8.EXPORTED) <= set(declared_functions())
    x = torch.zeros(16, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        fp8.absmax(x)   # a CPU tensor is refused: there is no CPU path


def test_binding_refuses_tensors_on_two_devices():
    """Every call's tensors must share one device (the library acts on the
    current device, which the binding sets from them): a mix is refused before
    the entry point is called."""
    import torch
    from fp8_precision_amd import _lib as b
    called = []
    with pytest.raises(ValueError, match="one device"):
        b._run("fp8_absmax", lambda *a: called.append(a) or 0,
               (torch.empty(1), None, torch.empty(1, device="meta")), 0, 1, 0)
    assert not called


def test_gemm_fwd_swiglu_absmax_validation(lib):
    f = lib.fp8_gemm_fwd_swiglu_absmax
    # (xq, wq, inv_sx, inv_sw, gu, absmax_h, M, F, K)
    assert f(A16, B16, C16, C16 + 16, D16, None, 256, 128, 128, None) == INVALID       # null absmax_h
    assert f(None, B16, C16, C16 + 16, D16, E16, 256, 128, 128, None) == INVALID
    assert f(A16, B16, C16, C16 + 16, D16, E16, 256, 0, 128, None) == INVALID          # F = 0
    assert f(A16, B16, C16, C16 + 16, D16, D16 + 64, 256, 128, 128, None) == INVALID   # absmax_h inside gu
    assert b"overlaps" in lib.fp8_last_error()
    assert f(A16, B16, C16, C16 + 16, D16, E16, 256, 64, 128, None) == UNSUPPORTED     # F % 128
    assert f(A16, B16, C16, C16 + 16, D16, E16, 128, 128, 128, None) == UNSUPPORTED    # M < 256
    assert f(A16, B16, C16, C16 + 16, D16, E16, 256, 128, 100, None) == UNSUPPORTED    # K % 128
    assert f(A16, B16, C16, C16 + 16, D16, E16 + 2, 256, 128, 128, None) == UNSUPPORTED  # misaligned absmax_h


def test_absmax_accumulate_many_validation(lib):
    f = lib.fp8_absmax_accumulate_many

    def call(xs, ns, outs, count=None):
        k = len(xs)
        xa = (ctypes.c_void_p * k)(*xs)
        na = (ctypes.c_int64 * k)(*ns)
        oa = (ctypes.c_void_p * k)(*outs)
        return f(k if count is None else count, ctypes.cast(xa, ctypes.c_void_p), ctypes.cast(na, ctypes.c_void_p),
                 ctypes.cast(oa, ctypes.c_void_p), None)

    assert f(1, None, None, None, None) == INVALID
    assert call([A16, B16], [16, 16], [C16, C16 + 4], count=0) == INVALID
    assert call([A16, B16], [16, 16], [C16, C16 + 4], count=9) == INVALID
    assert call([A16, None], [16, 16], [C16, C16 + 4]) == INVALID
    assert call([A16, B16], [16, 16], [C16, None]) == INVALID
    assert call([A16, B16], [16, 0], [C16, C16 + 4]) == INVALID
    assert call([A16, B16], [16, 16], [C16, B16 + 8]) == INVALID        # an accumulator inside an input
    assert b"overlaps" in lib.fp8_last_error()
    assert call([A16, B16 + 2], [16, 16], [C16, C16 + 4]) == UNSUPPORTED
    assert call([A16, B16], [16, 16], [C16, C16 + 2]) == UNSUPPORTED


def test_quantize_many_validation(lib):
    f = lib.fp8_quantize_many
    f.restype = ctypes.c_int
    vp = ctypes.c_void_p

    def call(xs, rows, cols, fmts, ams, qs, qts, count=None):
        k = len(xs)
        P = lambda v: ctypes.cast((ctypes.c_void_p * k)(*v), vp)
        I = lambda v: ctypes.cast((ctypes.c_int64 * k)(*v), vp)
        F = lambda v: ctypes.cast((ctypes.c_int * k)(*v), vp)
        return f(k if count is None else count, P(xs), I(rows), I(cols), F(fmts), P(ams), P(qs), P(qts),
                 P([None] * k), P([None] * k), F([1] * k), None)

    ok = dict(xs=[A16, B16], rows=[16, 16], cols=[16, 32], fmts=[0, 1], ams=[C16, C16 + 4], qs=[D16, D16 + 256],
              qts=[E16, None])
    assert f(1, None, None, None, None, None, None, None, None, None, None, None) == INVALID
    assert call(**ok, count=0) == INVALID
    assert call(**ok, count=9) == INVALID
    assert call(**{**ok, "xs": [A16, None]}) == INVALID
    assert call(**{**ok, "qs": [D16, None], "qts": [E16, None]}) == INVALID          # tensor 1 has no output
    assert call(**{**ok, "fmts": [0, 2]}) == INVALID
    assert call(**{**ok, "rows": [16, 0]}) == INVALID
    assert call(**{**ok, "qs": [D16, D16 + 128]}) == INVALID                         # outputs overlap
    assert b"overlapping outputs" in lib.fp8_last_error()
    assert call(**{**ok, "qs": [D16, A16 + 64]}) == INVALID                          # an output inside an input
    assert b"overlaps an input" in lib.fp8_last_error()
    assert call(**{**ok, "rows": [16, 24]}) == UNSUPPORTED                           # rows % 16
    assert call(**{**ok, "cols": [16, 40]}) == UNSUPPORTED                           # cols % 16
    assert call(**{**ok, "xs": [A16, B16 + 2]}) == UNSUPPORTED                       # misaligned input


def test_stream_copy_validation(lib):
    f = lib.fp8_stream_copy
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    assert f(None, B16, 64, None) == INVALID
    assert f(A16, None, 64, None) == INVALID
    assert f(A16, B16, 0, None) == INVALID
    assert f(A16, B16, -16, None) == INVALID
    assert f(A16, A16 + 32, 64, None) == INVALID                    # overlapping
    assert b"overlap" in lib.fp8_last_error()
    assert f(A16, B16, 40, None) == UNSUPPORTED                     # not a multiple of 16
    assert f(A16 + 8, B16, 64, None) == UNSUPPORTED                 # misaligned source
    assert f(A16, B16 + 4, 64, None) == UNSUPPORTED                 # misaligned destination



def test_mx_quantize_validation(lib):
    f = lib.fp8_mx_quantize
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p]
    q, sc = B16, B16 + (1 << 20)
    assert f(None, 4, 128, 0, q, sc, None) == INVALID
    assert f(A16, 4, 128, 0, None, sc, None) == INVALID
    assert f(A16, 4, 128, 0, q, None, None) == INVALID
    assert f(A16, 4, 128, 2, q, sc, None) == INVALID                 # bad format
    assert f(A16, 0, 128, 0, q, sc, None) == INVALID                 # empty
    assert f(A16, 4, 128, 0, A16 + 64, sc, None) == INVALID          # q overlaps x
    assert b"overlap" in lib.fp8_last_error()
    assert f(A16, 4, 96, 0, q, sc, None) == UNSUPPORTED              # cols not a multiple of 128
    assert f(A16 + 2, 4, 128, 0, q, sc, None) == UNSUPPORTED         # misaligned input
    assert f(A16, 4, 128, 0, q + 8, sc, None) == UNSUPPORTED         # misaligned codes


def test_mx_gemm_validation(lib):
    f = lib.fp8_mx_gemm_fwd
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    X, SX, W, SW, Y = A16, A16 + (1 << 24), B16, B16 + (1 << 24), C16
    ok = (X, SX, 0, W, SW, Y, 512, 512, 256, None)
    bad = lambda **kw: f(*[kw.get(k, v) for k, v in zip(("x", "sx", "fmt", "w", "sw", "y", "M", "N", "K", "s"), ok)])
    assert bad(sx=None) == INVALID and bad(sw=None) == INVALID and bad(x=None) == INVALID
    assert bad(fmt=3) == INVALID
    assert bad(y=SX) == INVALID                                       # output over the scales
    assert b"overlaps" in lib.fp8_last_error()
    assert bad(M=128) == UNSUPPORTED and bad(N=240) == UNSUPPORTED    # below one tile
    assert bad(K=192) == UNSUPPORTED                                  # reduction not a multiple of 128
    assert bad(sx=SX + 2) == UNSUPPORTED                              # misaligned scales
    assert bad(x=X + 8) == UNSUPPORTED                                # misaligned codes


def test_mx_gemm_backward_validation(lib):
    f = lib.fp8_mx_gemm_backward
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int] + [ctypes.c_void_p] * 6 + [ctypes.c_int64] * 3 + [ctypes.c_void_p]
    G = 1 << 24
    keys = ("dyq", "sdy", "dyqt", "sdyt", "fmt", "wqt", "swt", "xqt", "sxt", "dx", "dw", "M", "N", "K", "s")
    ok = (A16, A16 + G, A16 + 2 * G, A16 + 3 * G, 1, B16, B16 + G, B16 + 2 * G, B16 + 3 * G, C16, D16,
          512, 768, 640, None)
    bad = lambda **kw: f(*[kw.get(k, v) for k, v in zip(keys, ok)])
    for k in ("dyq", "sdy", "dyqt", "sdyt", "wqt", "swt", "xqt", "sxt", "dx", "dw"):
        assert bad(**{k: None}) == INVALID, k
    assert bad(fmt=2) == INVALID
    assert bad(dw=C16 + 64) == INVALID                                # dx and dw overlap
    assert bad(dx=B16 + 3 * G) == INVALID                             # dx over the scales of X^T
    assert b"overlap" in lib.fp8_last_error()
    assert bad(M=128) == UNSUPPORTED and bad(K=240) == UNSUPPORTED    # below one tile
    assert bad(N=704) == UNSUPPORTED and bad(M=576) == UNSUPPORTED    # reductions not multiples of 128
    assert bad(swt=B16 + G + 2) == UNSUPPORTED                        # misaligned scales
    assert bad(xqt=B16 + 2 * G + 8) == UNSUPPORTED                    # misaligned codes


def test_mx_swiglu_validation(lib):
    f = lib.fp8_mx_swiglu_requant
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    hq, sc = B16, B16 + (1 << 20)
    assert f(None, 4, 128, hq, sc, None) == INVALID
    assert f(A16, 4, 128, None, sc, None) == INVALID
    assert f(A16, 0, 128, hq, sc, None) == INVALID
    assert f(A16, 4, 128, A16 + 256, sc, None) == INVALID            # hq over gu
    assert f(A16, 4, 96, hq, sc, None) == UNSUPPORTED                # F not a multiple of 128
    assert f(A16 + 2, 4, 128, hq, sc, None) == UNSUPPORTED           # misaligned gu


def test_mx_quantize_t_validation(lib):
    f = lib.fp8_mx_quantize_t
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p]
    qt, sc = B16, B16 + (1 << 20)
    assert f(None, 128, 128, 0, qt, sc, None) == INVALID
    assert f(A16, 128, 128, 5, qt, sc, None) == INVALID
    assert f(A16, 128, 128, 0, A16 + 512, sc, None) == INVALID       # qt over x
    assert f(A16, 64, 128, 0, qt, sc, None) == UNSUPPORTED           # rows not a multiple of 128
    assert f(A16, 128, 144, 0, qt, sc, None) == UNSUPPORTED          # cols not a multiple of 128
    assert f(A16, 128, 128, 0, qt, sc + 2, None) == UNSUPPORTED      # misaligned scales


def test_mx_quantize_both_validation(lib):
    f = lib.fp8_mx_quantize_both
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int] + [ctypes.c_void_p] * 5
    q, sq, qt, sqt = B16, B16 + (1 << 20), C16, C16 + (1 << 20)
    assert f(None, 128, 128, 0, q, sq, qt, sqt, None) == INVALID
    assert f(A16, 128, 128, 0, q, sq, None, sqt, None) == INVALID
    assert f(A16, 128, 128, 0, q, sq, q + 64, sqt, None) == INVALID    # qt over q
    assert f(A16, 128, 96, 0, q, sq, qt, sqt, None) == UNSUPPORTED
    assert f(A16, 128, 128, 0, q + 8, sq, qt, sqt, None) == UNSUPPORTED
    assert f(A16, 128, 128, 0, q, sq + 2, qt, sqt, None) == UNSUPPORTED     # misaligned scales
    assert f(A16, 128, 128, 0, q, sq, qt, sqt + 1, None) == UNSUPPORTED


def test_absmax_clear_validation(lib):
    f = lib.fp8_absmax_clear
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    assert f(None, 4, None) == INVALID
    assert f(A16, 0, None) == INVALID and f(A16, -1, None) == INVALID
    assert f(A16, (1 << 20) + 1, None) == INVALID
    assert b"count" in lib.fp8_last_error()
    assert f(A16 + 2, 4, None) == UNSUPPORTED                          # not 4-byte aligned
