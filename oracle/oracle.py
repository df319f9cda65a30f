"""numpy/ctypes binding of the C oracle (test infrastructure only).

Arrays in and out are numpy: bf16 tensors travel as ``uint16`` bit patterns,
FP8 tensors as ``uint8`` codes, fp32 as ``float32``.  Every function checks
shapes and dtypes and raises ``ValueError`` on a mismatch.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

E4M3 = 0
E5M2 = 1
FP8_MAX = {E4M3: 448.0, E5M2: 57344.0}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def lib_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        i64, f32, i32 = ctypes.c_int64, ctypes.c_float, ctypes.c_int
        vp = ctypes.c_void_p
        sig = {
            "oracle_bf16_to_f32": (f32, [ctypes.c_uint16]),
            "oracle_f32_to_bf16": (ctypes.c_uint16, [f32]),
            "oracle_encode": (ctypes.c_uint8, [f32, i32]),
            "oracle_decode": (f32, [ctypes.c_uint8, i32]),
            "oracle_absmax_bf16": (f32, [vp, i64]),
            "oracle_absmax_f32": (f32, [vp, i64]),
            "oracle_scale": (None, [f32, i32, vp, vp]),
            "oracle_quantize": (None, [vp, i64, i64, i32, f32, vp, vp]),
            "oracle_exp_neg": (f32, [f32]),
            "oracle_swiglu_one": (f32, [f32, f32]),
            "oracle_swiglu_h": (None, [vp, i64, i64, vp]),
            "oracle_swiglu_requant": (None, [vp, i64, i64, i32, vp, vp, vp, vp, vp]),
            "oracle_gemm": (None, [vp, i32, vp, i32, i64, i64, i64, f32, f32, vp, i64, vp, vp, vp]),
            "oracle_swiglu_grad_one": (None, [f32, f32, f32, vp, vp]),
            "oracle_swiglu_grad": (None, [vp, vp, i64, i64, vp]),
            "oracle_swiglu_backward": (None, [vp, vp, i64, i64, i32, vp, vp, vp, vp, vp, vp]),
            "oracle_mx_quantize": (None, [vp, i64, i64, i32, vp, vp]),
            "oracle_mx_gemm": (None, [vp, vp, i32, vp, vp, i32, i64, i64, i64, vp, i64, vp]),
            "oracle_mx_quantize_f32": (None, [vp, i64, i64, i32, vp, vp]),
            "oracle_mx_swiglu": (None, [vp, i64, i64, vp, vp]),
            "oracle_encode_vec": (None, [vp, i64, i32, vp]),
            "oracle_decode_vec": (None, [vp, i64, i32, vp]),
            "oracle_exp_neg_vec": (None, [vp, i64, vp]),
            "oracle_num_threads": (i32, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def _need(a, dtype, name):
    if not isinstance(a, np.ndarray) or a.dtype != dtype:
        raise ValueError(f"{name} must be a numpy {np.dtype(dtype)} array")
    if not a.flags.c_contiguous:
        raise ValueError(f"{name} must be C-contiguous")


def _fmt(fmt):
    if fmt not in (E4M3, E5M2):
        raise ValueError("fmt must be E4M3 (0) or E5M2 (1)")
    return fmt


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exact."""
    _need(bits, np.uint16, "bits")
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (the C routine, element by element)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    lib = _load()
    out = np.empty(x.shape, np.uint16)
    flat_in, flat_out = x.reshape(-1), out.reshape(-1)
    for i in range(flat_in.size):
        flat_out[i] = lib.oracle_f32_to_bf16(float(flat_in[i]))
    return out


def encode(v: np.ndarray, fmt: int) -> np.ndarray:
    """fp32 values -> OFP8 codes (RNE, saturating)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().oracle_encode_vec(_ptr(v), v.size, _fmt(fmt), _ptr(out))
    return out


def decode(c: np.ndarray, fmt: int) -> np.ndarray:
    """OFP8 codes -> fp32 values (exact)."""
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, np.float32)
    _load().oracle_decode_vec(_ptr(c), c.size, _fmt(fmt), _ptr(out))
    return out


def absmax_bf16(x: np.ndarray) -> np.float32:
    _need(x, np.uint16, "x")
    if x.size == 0:
        raise ValueError("absmax of an empty tensor is undefined")
    return np.float32(_load().oracle_absmax_bf16(_ptr(x), x.size))


def absmax_f32(x: np.ndarray) -> np.float32:
    _need(x, np.float32, "x")
    if x.size == 0:
        raise ValueError("absmax of an empty tensor is undefined")
    return np.float32(_load().oracle_absmax_f32(_ptr(x), x.size))


def scale(absmax, fmt: int) -> tuple[np.float32, np.float32]:
    """(scale, inverse scale) for a per-tensor absmax."""
    s = np.zeros(1, np.float32)
    inv = np.zeros(1, np.float32)
    _load().oracle_scale(float(np.float32(absmax)), _fmt(fmt), _ptr(s), _ptr(inv))
    return s[0], inv[0]


def quantize(x: np.ndarray, fmt: int, s, want_q: bool = True, want_qt: bool = False):
    """Quantise a bf16 [rows, cols] tensor (uint16 bits) with scale s.

    Returns (q [rows, cols] or None, qt [cols, rows] or None).
    """
    _need(x, np.uint16, "x")
    if x.ndim != 2:
        raise ValueError("x must be 2-D")
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8) if want_q else None
    qt = np.empty((cols, rows), np.uint8) if want_qt else None
    _load().oracle_quantize(_ptr(x), rows, cols, _fmt(fmt), float(np.float32(s)), _ptr(q), _ptr(qt))
    return q, qt


def exp_neg(g: np.ndarray) -> np.ndarray:
    """RN32(e^-g) element-wise, g float32."""
    g = np.ascontiguousarray(g, dtype=np.float32)
    out = np.empty(g.shape, np.float32)
    _load().oracle_exp_neg_vec(_ptr(g), g.size, _ptr(out))
    return out


def swiglu_h(gu: np.ndarray) -> np.ndarray:
    """fp32 h [M, F] from gu = [gate | up], bf16 bits [M, 2F]."""
    _need(gu, np.uint16, "gu")
    if gu.ndim != 2 or gu.shape[1] % 2:
        raise ValueError("gu must be [M, 2F]")
    M, F = gu.shape[0], gu.shape[1] // 2
    h = np.empty((M, F), np.float32)
    _load().oracle_swiglu_h(_ptr(gu), M, F, _ptr(h))
    return h


def swiglu_requant(gu: np.ndarray, absmax_h=None, want_hq: bool = True, want_hqt: bool = False):
    """SwiGLU then e4m3 requantisation.

    absmax_h None: forward mode, the absmax of h is computed.  Otherwise the
    given (retained) statistic is used and no reduction runs.
    Returns (hq or None, hqt or None, absmax_h, inv_scale_h).
    """
    _need(gu, np.uint16, "gu")
    if gu.ndim != 2 or gu.shape[1] % 2:
        raise ValueError("gu must be [M, 2F]")
    M, F = gu.shape[0], gu.shape[1] // 2
    am = np.array([0.0 if absmax_h is None else absmax_h], np.float32)
    inv = np.zeros(1, np.float32)
    hbuf = np.empty((M, F), np.float32)
    hq = np.empty((M, F), np.uint8) if want_hq else None
    hqt = np.empty((F, M), np.uint8) if want_hqt else None
    _load().oracle_swiglu_requant(_ptr(gu), M, F, 1 if absmax_h is None else 0, _ptr(am),
                                  _ptr(inv), _ptr(hbuf), _ptr(hq), _ptr(hqt))
    return hq, hqt, am[0], inv[0]



def swiglu_grad(gu: np.ndarray, dh: np.ndarray) -> np.ndarray:
    """The fp32 gradient [dg | du] ([M, 2F]) of gu = [gate | up] given dh = dL/dh (bf16 bits)."""
    _need(gu, np.uint16, "gu")
    _need(dh, np.uint16, "dh")
    M, F = gu.shape[0], gu.shape[1] // 2
    if gu.ndim != 2 or gu.shape[1] % 2 or dh.shape != (M, F):
        raise ValueError("gu must be [M, 2F] and dh [M, F]")
    out = np.empty((M, 2 * F), np.float32)
    _load().oracle_swiglu_grad(_ptr(gu), _ptr(dh), M, F, _ptr(out))
    return out


def swiglu_backward(gu: np.ndarray, dh: np.ndarray, fmt: int = E5M2, want_q: bool = True, want_qt: bool = False):
    """SwiGLU backward fused with the quantisation of [dg | du].

    Returns (q [M, 2F] or None, qt [2F, M] or None, absmax, scale, inv_scale).
    """
    _need(gu, np.uint16, "gu")
    _need(dh, np.uint16, "dh")
    M, F = gu.shape[0], gu.shape[1] // 2
    if gu.ndim != 2 or gu.shape[1] % 2 or dh.shape != (M, F):
        raise ValueError("gu must be [M, 2F] and dh [M, F]")
    am, sc, inv = (np.zeros(1, np.float32) for _ in range(3))
    buf = np.empty((M, 2 * F), np.float32)
    q = np.empty((M, 2 * F), np.uint8) if want_q else None
    qt = np.empty((2 * F, M), np.uint8) if want_qt else None
    _load().oracle_swiglu_backward(_ptr(gu), _ptr(dh), M, F, _fmt(fmt), _ptr(am), _ptr(sc), _ptr(inv), _ptr(buf),
                                   _ptr(q), _ptr(qt))
    return q, qt, am[0], sc[0], inv[0]


def swiglu_grad_one(g, u, d):
    """(dg, du) of one element pair, fp32."""
    dg, du = np.zeros(1, np.float32), np.zeros(1, np.float32)
    _load().oracle_swiglu_grad_one(np.float32(g), np.float32(u), np.float32(d), _ptr(dg), _ptr(du))
    return dg[0], du[0]


def gemm(a: np.ndarray, fmt_a: int, b: np.ndarray, fmt_b: int, da, db, rows=None) -> np.ndarray:
    """Y = bf16(RN32(sum_k dec(A[m,k]) dec(B[n,k]) * RN32(da*db))), bf16 bits.

    a: uint8 [M, K], b: uint8 [N, K].  rows: optional int64 row indices; then
    only those rows of Y are computed and returned as [len(rows), N].
    """
    _need(a, np.uint8, "a")
    _need(b, np.uint8, "b")
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError("a must be [M, K] and b [N, K]")
    M, K = a.shape
    N = b.shape[0]
    if rows is None:
        r_arr, nrows = None, M
    else:
        r_arr = np.ascontiguousarray(rows, dtype=np.int64)
        if r_arr.ndim != 1 or (r_arr.size and (r_arr.min() < 0 or r_arr.max() >= M)):
            raise ValueError("rows out of range")
        nrows = r_arr.size
    y = np.empty((nrows, N), np.uint16)
    a_dec = np.empty((nrows, K), np.float32)
    b_dec = np.empty((N, K), np.float32)
    _load().oracle_gemm(_ptr(a), _fmt(fmt_a), _ptr(b), _fmt(fmt_b), M, N, K,
                        float(np.float32(da)), float(np.float32(db)), _ptr(r_arr), nrows,
                        _ptr(a_dec), _ptr(b_dec), _ptr(y))
    return y


MX_BLOCK = 32


def mx_quantize(x: np.ndarray, fmt: int):
    """Block (MX) quantisation of a bf16 [rows, cols] tensor (uint16 bits, cols a
    multiple of 32): returns (codes uint8 [rows, cols], E8M0 scales uint8 [rows, cols / 32])."""
    _need(x, np.uint16, "x")
    if x.ndim != 2 or x.shape[1] % MX_BLOCK:
        raise ValueError("x must be 2-D with a multiple of 32 columns")
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    sc = np.empty((rows, cols // MX_BLOCK), np.uint8)
    _load().oracle_mx_quantize(_ptr(x), rows, cols, _fmt(fmt), _ptr(q), _ptr(sc))
    return q, sc


def mx_gemm(a: np.ndarray, sa: np.ndarray, fmt_a: int, b: np.ndarray, sb: np.ndarray, fmt_b: int,
            rows=None) -> np.ndarray:
    """Y = bf16(RN32(sum_k ldexp(dec(A[m,k]) dec(B[n,k]), ea + eb))) with per-block scales, bf16 bits.

    a: uint8 [M, K] and sa: uint8 [M, K / 32]; b: uint8 [N, K] and sb: uint8 [N, K / 32].
    rows: optional int64 row indices, as in gemm().
    """
    for t, n in ((a, "a"), (sa, "sa"), (b, "b"), (sb, "sb")):
        _need(t, np.uint8, n)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1] or a.shape[1] % MX_BLOCK:
        raise ValueError("a must be [M, K] and b [N, K], K a multiple of 32")
    M, K = a.shape
    N = b.shape[0]
    if sa.shape != (M, K // MX_BLOCK) or sb.shape != (N, K // MX_BLOCK):
        raise ValueError("scales must be [M, K / 32] and [N, K / 32]")
    if rows is None:
        r_arr, nrows = None, M
    else:
        r_arr = np.ascontiguousarray(rows, dtype=np.int64)
        if r_arr.ndim != 1 or (r_arr.size and (r_arr.min() < 0 or r_arr.max() >= M)):
            raise ValueError("rows out of range")
        nrows = r_arr.size
    y = np.empty((nrows, N), np.uint16)
    _load().oracle_mx_gemm(_ptr(a), _ptr(sa), _fmt(fmt_a), _ptr(b), _ptr(sb), _fmt(fmt_b), M, N, K,
                           _ptr(r_arr), nrows, _ptr(y))
    return y


def mx_quantize_f32(x: np.ndarray, fmt: int):
    """Block (MX) quantisation of an fp32 [rows, cols] tensor (cols a multiple of 32),
    the rule of mx_quantize: returns (codes [rows, cols], scales [rows, cols / 32])."""
    _need(x, np.float32, "x")
    if x.ndim != 2 or x.shape[1] % MX_BLOCK:
        raise ValueError("x must be 2-D with a multiple of 32 columns")
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    sc = np.empty((rows, cols // MX_BLOCK), np.uint8)
    _load().oracle_mx_quantize_f32(_ptr(x), rows, cols, _fmt(fmt), _ptr(q), _ptr(sc))
    return q, sc


def mx_swiglu(gu: np.ndarray):
    """The SwiGLU output of gu = [gate | up] (bf16 bits [M, 2F], F a multiple of 32),
    MX-quantised (E4M3) along F: returns (hq [M, F], scales [M, F / 32])."""
    _need(gu, np.uint16, "gu")
    if gu.ndim != 2 or gu.shape[1] % (2 * MX_BLOCK):
        raise ValueError("gu must be [M, 2F] with F a multiple of 32")
    M, F = gu.shape[0], gu.shape[1] // 2
    hq = np.empty((M, F), np.uint8)
    sc = np.empty((M, F // MX_BLOCK), np.uint8)
    _load().oracle_mx_swiglu(_ptr(gu), M, F, _ptr(hq), _ptr(sc))
    return hq, sc
