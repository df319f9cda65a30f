"""ctypes binding of ``libfp8_precision.so`` (the C ABI in include/fp8_precision.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  torch supplies device memory (tensors are passed by ``data_ptr()``)
and the stream (torch's current stream on the tensor's device).  If the
library is missing, importing this module raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

E4M3 = 0
E5M2 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8_precision.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python fp8_precision_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

_i64, _i32, _vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
_SIGS = {
    "fp8_status_string": (ctypes.c_char_p, [_i32]),
    "fp8_last_error": (ctypes.c_char_p, []),
    "fp8_absmax": (_i32, [_vp, _i64, _vp, _vp]),
    "fp8_absmax_accumulate": (_i32, [_vp, _i64, _vp, _vp]),
    "fp8_absmax_accumulate_many": (_i32, [ctypes.c_int, _vp, _vp, _vp, _vp]),
    "fp8_absmax_clear": (_i32, [_vp, _i64, _vp]),
    "fp8_quantize": (_i32, [_vp, _i64, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "fp8_quantize_many": (_i32, [ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "fp8_swiglu_requant": (_i32, [_vp, _i64, _i64, _vp, _i32, _vp, _vp, _vp, _vp]),
    "fp8_swiglu_backward": (_i32, [_vp, _vp, _i64, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "fp8_gemm_fwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "fp8_gemm_fwd_swiglu_absmax": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "fp8_gemm_dgrad": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "fp8_gemm_wgrad": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "fp8_gemm_backward": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "fp8_gemm_dgrad_mn": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "fp8_gemm_wgrad_mn": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "fp8_gemm_backward_mn": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "fp8_stream_copy": (_i32, [_vp, _vp, _i64, _vp]),
    "fp8_mx_quantize": (_i32, [_vp, _i64, _i64, _i32, _vp, _vp, _vp]),
    "fp8_mx_gemm_fwd": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "fp8_mx_gemm_backward": (_i32, [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "fp8_mx_swiglu_requant": (_i32, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "fp8_mx_quantize_t": (_i32, [_vp, _i64, _i64, _i32, _vp, _vp, _vp]),
    "fp8_mx_quantize_both": (_i32, [_vp, _i64, _i64, _i32, _vp, _vp, _vp, _vp, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


class Fp8Error(RuntimeError):
    def __init__(self, call: str, status: int):
        self.status = status
        detail = _lib.fp8_last_error().decode()
        super().__init__(f"{call} failed: {_lib.fp8_status_string(status).decode()} ({detail})")


def _check(call: str, status: int) -> None:
    if status != 0:
        raise Fp8Error(call, status)


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


def _run(call: str, fn, tensors, *args) -> None:
    """Call entry point ``fn`` with ``args`` and the stream.  Every tensor of the
    call must be on one device; that device is made current for the call (the
    library acts on the current HIP device) and its current stream is passed."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{call}: all tensors must be on one device (got {dev} and {t.device})")
    with torch.cuda.device(dev):
        _check(call, fn(*args, torch.cuda.current_stream(dev).cuda_stream))


def _dev_tensor(t, name, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _scalar_in(t, name):
    """An fp32 scalar input (absmax, inverse scale): a device tensor holding at least one value."""
    _dev_tensor(t, name, torch.float32)
    if t.numel() < 1:
        raise ValueError(f"{name} must hold at least one fp32")
    return t


def _scalar(t, name, device):
    if t is None:
        return torch.empty(1, dtype=torch.float32, device=device)
    _dev_tensor(t, name, torch.float32)
    if t.numel() < 1:
        raise ValueError(f"{name} must hold at least one fp32")
    return t


def absmax(x: torch.Tensor, out: torch.Tensor | None = None, accumulate: bool = False) -> torch.Tensor:
    """max |x| of a bf16 tensor, as a one-element fp32 device tensor.

    With ``accumulate`` the result is max(out, max |x|) (``out`` required,
    holding +0 or an earlier result): fp8_absmax_accumulate.
    """
    _dev_tensor(x, "x", torch.bfloat16)
    if accumulate:
        if out is None:
            raise ValueError("accumulate needs out")
        out = _scalar(out, "out", x.device)
        _run("fp8_absmax_accumulate", _lib.fp8_absmax_accumulate, (x, out), _ptr(x), x.numel(), _ptr(out))
        return out
    out = _scalar(out, "out", x.device)
    _run("fp8_absmax", _lib.fp8_absmax, (x, out), _ptr(x), x.numel(), _ptr(out))
    return out


def absmax_accumulate_many(xs, outs) -> None:
    """Running absmax of up to 8 bf16 tensors in one launch: outs[i] (fp32 [1]
    device tensors, +0 or an earlier result) become max(outs[i], max |xs[i]|)."""
    if len(xs) != len(outs) or not 1 <= len(xs) <= 8:
        raise ValueError("1 to 8 tensors, one output each")
    for x in xs:
        _dev_tensor(x, "x", torch.bfloat16)
    if any(o is None for o in outs):
        raise ValueError("every output is read and updated: pass a tensor holding +0 or an earlier result")
    outs = [_scalar_in(o, "out") for o in outs]
    k = len(xs)
    xp = (ctypes.c_void_p * k)(*[_ptr(x) for x in xs])
    ns = (ctypes.c_int64 * k)(*[x.numel() for x in xs])
    op = (ctypes.c_void_p * k)(*[_ptr(o) for o in outs])
    _run("fp8_absmax_accumulate_many", _lib.fp8_absmax_accumulate_many, list(xs) + outs,
         k, ctypes.cast(xp, _vp), ctypes.cast(ns, _vp), ctypes.cast(op, _vp))


def absmax_clear(stats: torch.Tensor) -> None:
    """Set every statistic of a contiguous fp32 device tensor to +0 (the start
    of the running absmax that the accumulating calls update), in one launch."""
    _dev_tensor(stats, "stats", torch.float32)
    if not 1 <= stats.numel() <= 1 << 20:
        raise ValueError("1 to 2^20 statistics")
    _run("fp8_absmax_clear", _lib.fp8_absmax_clear, (stats,), _ptr(stats), stats.numel())


def quantize(x: torch.Tensor, fmt: int, amax: torch.Tensor, want_q: bool = True, want_qt: bool = False,
             q: torch.Tensor | None = None, qt: torch.Tensor | None = None,
             scale: torch.Tensor | None = None, inv_scale: torch.Tensor | None = None):
    """Quantise a 2-D bf16 tensor with the scale of ``amax``.

    Returns (q uint8 [rows, cols] or None, qt uint8 [cols, rows] or None,
    scale fp32 [1], inv_scale fp32 [1]).
    """
    _dev_tensor(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    rows, cols = x.shape
    _scalar_in(amax, "amax")
    if want_q and q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if want_qt and qt is None:
        qt = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    for t, n in ((q, "q"), (qt, "qt")):
        if t is not None:
            _dev_tensor(t, n, torch.uint8)
            if t.numel() != rows * cols:
                raise ValueError(f"{n} has the wrong size")
    scale = _scalar(scale, "scale", x.device)
    inv_scale = _scalar(inv_scale, "inv_scale", x.device)
    _run("fp8_quantize", _lib.fp8_quantize, (x, amax, q, qt, scale, inv_scale),
         _ptr(x), rows, cols, int(fmt), _ptr(amax), _ptr(q), _ptr(qt), _ptr(scale), _ptr(inv_scale))
    return q, qt, scale, inv_scale


def quantize_many(xs, fmts, amaxs, want_q=True, want_qt=False, qs=None, qts=None, scales=None, inv_scales=None,
                  qt_later=False):
    """Quantise up to 8 2-D bf16 tensors in one launch, each exactly as ``quantize``.

    ``fmts``, ``amaxs``, ``want_q``, ``want_qt``, ``qt_later`` and the optional
    output lists are per tensor (a single value applies to all).  ``qt_later``:
    the transposed copy is read later (the backward pass), not by the next
    call, and is stored non-temporally (same bytes).  Returns lists
    (qs, qts, scales, inv_scales), None where an output was not asked for.
    """
    k = len(xs)
    if not 1 <= k <= 8:
        raise ValueError("1 to 8 tensors")
    per = lambda v: list(v) if isinstance(v, (list, tuple)) else [v] * k
    fmts, amaxs, want_q, want_qt, qt_later = per(fmts), per(amaxs), per(want_q), per(want_qt), per(qt_later)
    qs, qts = per(qs) if qs is not None else [None] * k, per(qts) if qts is not None else [None] * k
    scales = per(scales) if scales is not None else [None] * k
    inv_scales = per(inv_scales) if inv_scales is not None else [None] * k
    if any(len(v) != k for v in (fmts, amaxs, want_q, want_qt, qt_later, qs, qts, scales, inv_scales)):
        raise ValueError("one entry per tensor")
    rows, cols = [], []
    for i, x in enumerate(xs):
        _dev_tensor(x, "x", torch.bfloat16)
        if x.dim() != 2:
            raise ValueError("every x must be 2-D")
        r, c = x.shape
        rows.append(r)
        cols.append(c)
        _scalar_in(amaxs[i], "amax")
        if want_q[i] and qs[i] is None:
            qs[i] = torch.empty((r, c), dtype=torch.uint8, device=x.device)
        if want_qt[i] and qts[i] is None:
            qts[i] = torch.empty((c, r), dtype=torch.uint8, device=x.device)
        for t, n in ((qs[i], "q"), (qts[i], "qt")):
            if t is not None:
                _dev_tensor(t, n, torch.uint8)
                if t.numel() != r * c:
                    raise ValueError(f"{n} has the wrong size")
        scales[i] = _scalar(scales[i], "scale", x.device)
        inv_scales[i] = _scalar(inv_scales[i], "inv_scale", x.device)
    arr = lambda ts: (ctypes.c_void_p * k)(*[_ptr(t) for t in ts])
    xa, aa, qa, qta, sa, ia = arr(xs), arr(amaxs), arr(qs), arr(qts), arr(scales), arr(inv_scales)
    ra, ca = (ctypes.c_int64 * k)(*rows), (ctypes.c_int64 * k)(*cols)
    fa = (ctypes.c_int * k)(*[int(f) for f in fmts])
    la = (ctypes.c_int * k)(*[1 if v else 0 for v in qt_later])
    _run("fp8_quantize_many", _lib.fp8_quantize_many,
         list(xs) + list(amaxs) + qs + qts + scales + inv_scales,
         k, ctypes.cast(xa, _vp), ctypes.cast(ra, _vp), ctypes.cast(ca, _vp), ctypes.cast(fa, _vp),
         ctypes.cast(aa, _vp), ctypes.cast(qa, _vp), ctypes.cast(qta, _vp), ctypes.cast(sa, _vp),
         ctypes.cast(ia, _vp), ctypes.cast(la, _vp))
    return qs, qts, scales, inv_scales


def swiglu_requant(gu: torch.Tensor, absmax_h: torch.Tensor | None = None, compute_absmax: bool = True,
                   want_hq: bool = True, want_hqt: bool = False, hq: torch.Tensor | None = None,
                   hqt: torch.Tensor | None = None, inv_scale_h: torch.Tensor | None = None,
                   accumulate: bool = False):
    """SwiGLU of gu = [gate | up] (bf16 [M, 2F]) requantised to e4m3.

    compute_absmax True: absmax_h is computed (forward); with ``accumulate``
    it is max(absmax_h, max |h|) (absmax_h given, holding +0 or an earlier
    result).  False: the given retained absmax_h is used and no reduction runs
    (recomputation).  Returns (hq or None, hqt or None, absmax_h, inv_scale_h).
    """
    _dev_tensor(gu, "gu", torch.bfloat16)
    if gu.dim() != 2 or gu.shape[1] % 2:
        raise ValueError("gu must be [M, 2F]")
    M, F = gu.shape[0], gu.shape[1] // 2
    if not compute_absmax and absmax_h is None:
        raise ValueError("recomputation needs the retained absmax_h")
    if accumulate and (absmax_h is None or not compute_absmax):
        raise ValueError("accumulate needs compute_absmax and the absmax_h to update")
    absmax_h = _scalar(absmax_h, "absmax_h", gu.device)
    if want_hq and hq is None:
        hq = torch.empty((M, F), dtype=torch.uint8, device=gu.device)
    if want_hqt and hqt is None:
        hqt = torch.empty((F, M), dtype=torch.uint8, device=gu.device)
    for t, n in ((hq, "hq"), (hqt, "hqt")):
        if t is not None:
            _dev_tensor(t, n, torch.uint8)
            if t.numel() != M * F:
                raise ValueError(f"{n} has the wrong size")
    inv_scale_h = _scalar(inv_scale_h, "inv_scale_h", gu.device)
    _run("fp8_swiglu_requant", _lib.fp8_swiglu_requant, (gu, absmax_h, hq, hqt, inv_scale_h),
         _ptr(gu), M, F, _ptr(absmax_h), (2 if accumulate else 1) if compute_absmax else 0,
         _ptr(hq), _ptr(hqt), _ptr(inv_scale_h))
    return hq, hqt, absmax_h, inv_scale_h


def swiglu_backward(gu: torch.Tensor, dh: torch.Tensor, fmt: int = E5M2, want_q: bool = True, want_qt: bool = False,
                    absmax: torch.Tensor | None = None, q: torch.Tensor | None = None, qt: torch.Tensor | None = None,
                    scale: torch.Tensor | None = None, inv_scale: torch.Tensor | None = None):
    """Gradient of gu = [gate | up] (bf16 [M, 2F]) from dh (bf16 [M, F]), quantised with its own absmax.

    Returns (q uint8 [M, 2F] or None, qt uint8 [2F, M] or None, absmax, scale, inv_scale).
    """
    _dev_tensor(gu, "gu", torch.bfloat16)
    _dev_tensor(dh, "dh", torch.bfloat16)
    if gu.dim() != 2 or gu.shape[1] % 2:
        raise ValueError("gu must be [M, 2F]")
    M, F = gu.shape[0], gu.shape[1] // 2
    if tuple(dh.shape) != (M, F):
        raise ValueError("dh must be [M, F]")
    if want_q and q is None:
        q = torch.empty((M, 2 * F), dtype=torch.uint8, device=gu.device)
    if want_qt and qt is None:
        qt = torch.empty((2 * F, M), dtype=torch.uint8, device=gu.device)
    for t, n in ((q, "q"), (qt, "qt")):
        if t is not None:
            _dev_tensor(t, n, torch.uint8)
            if t.numel() != 2 * M * F:
                raise ValueError(f"{n} has the wrong size")
    absmax = _scalar(absmax, "absmax", gu.device)
    scale = _scalar(scale, "scale", gu.device)
    inv_scale = _scalar(inv_scale, "inv_scale", gu.device)
    _run("fp8_swiglu_backward", _lib.fp8_swiglu_backward, (gu, dh, absmax, q, qt, scale, inv_scale),
         _ptr(gu), _ptr(dh), M, F, int(fmt), _ptr(absmax), _ptr(q), _ptr(qt), _ptr(scale), _ptr(inv_scale))
    return q, qt, absmax, scale, inv_scale


def _out_bf16(out, shape, device):
    if out is None:
        return torch.empty(shape, dtype=torch.bfloat16, device=device)
    _dev_tensor(out, "out", torch.bfloat16)
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out must have shape {tuple(shape)}")
    return out


def gemm_fwd(xq, wq, inv_sx, inv_sw, out=None) -> torch.Tensor:
    """Y[M, N] = X[M, K] . W[N, K]^T (both e4m3), bf16 out."""
    _dev_tensor(xq, "xq", torch.uint8)
    _dev_tensor(wq, "wq", torch.uint8)
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("xq is [M, K] and wq must be [N, K]")
    _scalar_in(inv_sx, "inv_sx")
    _scalar_in(inv_sw, "inv_sw")
    out = _out_bf16(out, (M, N), xq.device)
    _run("fp8_gemm_fwd", _lib.fp8_gemm_fwd, (xq, wq, inv_sx, inv_sw, out),
         _ptr(xq), _ptr(wq), _ptr(inv_sx), _ptr(inv_sw), _ptr(out), M, N, K)
    return out


def gemm_fwd_swiglu_absmax(xq, wq, inv_sx, inv_sw, absmax_h, out=None) -> torch.Tensor:
    """gu[M, 2F] = X[M, K] . Wgu[2F, K]^T (e4m3), bf16 out, and absmax_h (fp32 [1],
    holding +0 or an earlier result) updated to max(absmax_h, max |silu(gate) * up|)."""
    _dev_tensor(xq, "xq", torch.uint8)
    _dev_tensor(wq, "wq", torch.uint8)
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K or N % 2:
        raise ValueError("xq is [M, K] and wq must be [2F, K]")
    _scalar_in(inv_sx, "inv_sx")
    _scalar_in(inv_sw, "inv_sw")
    if absmax_h is None:
        raise ValueError("absmax_h is read and updated: pass a tensor holding +0 or an earlier result")
    _scalar_in(absmax_h, "absmax_h")
    out = _out_bf16(out, (M, N), xq.device)
    _run("fp8_gemm_fwd_swiglu_absmax", _lib.fp8_gemm_fwd_swiglu_absmax, (xq, wq, inv_sx, inv_sw, out, absmax_h),
         _ptr(xq), _ptr(wq), _ptr(inv_sx), _ptr(inv_sw), _ptr(out), _ptr(absmax_h), M, N // 2, K)
    return out


def gemm_dgrad(dyq, dy_fmt, wqt, inv_sdy, inv_sw, out=None) -> torch.Tensor:
    """dX[M, K] = dY[M, N] . W[N, K], with W passed transposed as wqt [K, N]."""
    _dev_tensor(dyq, "dyq", torch.uint8)
    _dev_tensor(wqt, "wqt", torch.uint8)
    M, N = dyq.shape
    K = wqt.shape[0]
    if wqt.shape[1] != N:
        raise ValueError("dyq is [M, N] and wqt must be [K, N]")
    _scalar_in(inv_sdy, "inv_sdy")
    _scalar_in(inv_sw, "inv_sw")
    out = _out_bf16(out, (M, K), dyq.device)
    _run("fp8_gemm_dgrad", _lib.fp8_gemm_dgrad, (dyq, wqt, inv_sdy, inv_sw, out),
         _ptr(dyq), int(dy_fmt), _ptr(wqt), _ptr(inv_sdy), _ptr(inv_sw), _ptr(out), M, N, K)
    return out


def gemm_wgrad(dyqt, dy_fmt, xqt, inv_sdy, inv_sx, out=None) -> torch.Tensor:
    """dW[N, K] = dY[M, N]^T . X[M, K], with dY and X passed transposed ([N, M], [K, M])."""
    _dev_tensor(dyqt, "dyqt", torch.uint8)
    _dev_tensor(xqt, "xqt", torch.uint8)
    N, M = dyqt.shape
    K = xqt.shape[0]
    if xqt.shape[1] != M:
        raise ValueError("dyqt is [N, M] and xqt must be [K, M]")
    _scalar_in(inv_sdy, "inv_sdy")
    _scalar_in(inv_sx, "inv_sx")
    out = _out_bf16(out, (N, K), dyqt.device)
    _run("fp8_gemm_wgrad", _lib.fp8_gemm_wgrad, (dyqt, xqt, inv_sdy, inv_sx, out),
         _ptr(dyqt), int(dy_fmt), _ptr(xqt), _ptr(inv_sdy), _ptr(inv_sx), _ptr(out), M, N, K)
    return out


def gemm_backward(dyq, dyqt, dy_fmt, wqt, xqt, inv_sdy, inv_sw, inv_sx, dx=None, dw=None):
    """dgrad and wgrad of one linear in one launch: returns (dX [M, K], dW [N, K])."""
    for t, n in ((dyq, "dyq"), (dyqt, "dyqt"), (wqt, "wqt"), (xqt, "xqt")):
        _dev_tensor(t, n, torch.uint8)
    M, N = dyq.shape
    K = wqt.shape[0]
    if tuple(dyqt.shape) != (N, M) or wqt.shape[1] != N or tuple(xqt.shape) != (K, M):
        raise ValueError("expected dyq [M, N], dyqt [N, M], wqt [K, N], xqt [K, M]")
    for t, n in ((inv_sdy, "inv_sdy"), (inv_sw, "inv_sw"), (inv_sx, "inv_sx")):
        _scalar_in(t, n)
    dx = _out_bf16(dx, (M, K), dyq.device)
    dw = _out_bf16(dw, (N, K), dyq.device)
    _run("fp8_gemm_backward", _lib.fp8_gemm_backward, (dyq, dyqt, wqt, xqt, inv_sdy, inv_sw, inv_sx, dx, dw),
         _ptr(dyq), _ptr(dyqt), int(dy_fmt), _ptr(wqt), _ptr(xqt), _ptr(inv_sdy), _ptr(inv_sw), _ptr(inv_sx),
         _ptr(dx), _ptr(dw), M, N, K)
    return dx, dw


def gemm_dgrad_mn(dyq, dy_fmt, wq, inv_sdy, inv_sw, out=None) -> torch.Tensor:
    """dX[M, K] = dY[M, N] . W[N, K] on the untransposed wq [N, K]."""
    _dev_tensor(dyq, "dyq", torch.uint8)
    _dev_tensor(wq, "wq", torch.uint8)
    M, N = dyq.shape
    K = wq.shape[1]
    if wq.shape[0] != N:
        raise ValueError("dyq is [M, N] and wq must be [N, K]")
    _scalar_in(inv_sdy, "inv_sdy")
    _scalar_in(inv_sw, "inv_sw")
    out = _out_bf16(out, (M, K), dyq.device)
    _run("fp8_gemm_dgrad_mn", _lib.fp8_gemm_dgrad_mn, (dyq, wq, inv_sdy, inv_sw, out),
         _ptr(dyq), int(dy_fmt), _ptr(wq), _ptr(inv_sdy), _ptr(inv_sw), _ptr(out), M, N, K)
    return out


def gemm_wgrad_mn(dyq, dy_fmt, xq, inv_sdy, inv_sx, out=None) -> torch.Tensor:
    """dW[N, K] = dY[M, N]^T . X[M, K] on the untransposed dyq [M, N] and xq [M, K]."""
    _dev_tensor(dyq, "dyq", torch.uint8)
    _dev_tensor(xq, "xq", torch.uint8)
    M, N = dyq.shape
    K = xq.shape[1]
    if xq.shape[0] != M:
        raise ValueError("dyq is [M, N] and xq must be [M, K]")
    _scalar_in(inv_sdy, "inv_sdy")
    _scalar_in(inv_sx, "inv_sx")
    out = _out_bf16(out, (N, K), dyq.device)
    _run("fp8_gemm_wgrad_mn", _lib.fp8_gemm_wgrad_mn, (dyq, xq, inv_sdy, inv_sx, out),
         _ptr(dyq), int(dy_fmt), _ptr(xq), _ptr(inv_sdy), _ptr(inv_sx), _ptr(out), M, N, K)
    return out


def gemm_backward_mn(dyq, dy_fmt, wq, xq, inv_sdy, inv_sw, inv_sx, dx=None, dw=None):
    """dgrad and wgrad of one linear in one launch on the untransposed tensors: (dX [M, K], dW [N, K])."""
    for t, n in ((dyq, "dyq"), (wq, "wq"), (xq, "xq")):
        _dev_tensor(t, n, torch.uint8)
    M, N = dyq.shape
    K = wq.shape[1]
    if wq.shape[0] != N or tuple(xq.shape) != (M, K):
        raise ValueError("expected dyq [M, N], wq [N, K], xq [M, K]")
    for t, n in ((inv_sdy, "inv_sdy"), (inv_sw, "inv_sw"), (inv_sx, "inv_sx")):
        _scalar_in(t, n)
    dx = _out_bf16(dx, (M, K), dyq.device)
    dw = _out_bf16(dw, (N, K), dyq.device)
    _run("fp8_gemm_backward_mn", _lib.fp8_gemm_backward_mn, (dyq, wq, xq, inv_sdy, inv_sw, inv_sx, dx, dw),
         _ptr(dyq), int(dy_fmt), _ptr(wq), _ptr(xq), _ptr(inv_sdy), _ptr(inv_sw), _ptr(inv_sx), _ptr(dx), _ptr(dw),
         M, N, K)
    return dx, dw


def mx_quantize(x: torch.Tensor, fmt: int, q: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """Block (MX) quantisation of a 2-D bf16 tensor (cols a multiple of 128):
    returns (q uint8 [rows, cols], scales uint8 [cols / 128, rows, 4], E8M0: the
    scale of block b of row i at [b // 4, i, b % 4])."""
    _dev_tensor(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    rows, cols = x.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((cols // 128, rows, 4), dtype=torch.uint8, device=x.device)
    for t, n, size in ((q, "q", rows * cols), (scales, "scales", rows * (cols // 32))):
        _dev_tensor(t, n, torch.uint8)
        if t.numel() != size:
            raise ValueError(f"{n} has the wrong size")
    _run("fp8_mx_quantize", _lib.fp8_mx_quantize, (x, q, scales), _ptr(x), rows, cols, int(fmt), _ptr(q), _ptr(scales))
    return q, scales


def mx_quantize_t(x: torch.Tensor, fmt: int, qt: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """Block (MX) quantisation of x^T for a 2-D bf16 x [rows, cols] (both multiples of
    128): returns (qt uint8 [cols, rows], scales uint8 [rows / 128, cols, 4]) -- blocks
    of 32 consecutive rows of x per column."""
    _dev_tensor(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    rows, cols = x.shape
    if qt is None:
        qt = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows // 128, cols, 4), dtype=torch.uint8, device=x.device)
    for t, n, size in ((qt, "qt", rows * cols), (scales, "scales", rows * cols // 32)):
        _dev_tensor(t, n, torch.uint8)
        if t.numel() != size:
            raise ValueError(f"{n} has the wrong size")
    _run("fp8_mx_quantize_t", _lib.fp8_mx_quantize_t, (x, qt, scales), _ptr(x), rows, cols, int(fmt), _ptr(qt),
         _ptr(scales))
    return qt, scales


def mx_quantize_both(x: torch.Tensor, fmt: int, q=None, sq=None, qt=None, sqt=None):
    """Both block quantisations of x [rows, cols] (multiples of 128) in one read: the
    results of mx_quantize (q, sq) and of mx_quantize_t (qt, sqt)."""
    _dev_tensor(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    rows, cols = x.shape
    u8 = lambda *sh: torch.empty(sh, dtype=torch.uint8, device=x.device)
    q = u8(rows, cols) if q is None else q
    sq = u8(cols // 128, rows, 4) if sq is None else sq
    qt = u8(cols, rows) if qt is None else qt
    sqt = u8(rows // 128, cols, 4) if sqt is None else sqt
    for t, n, size in ((q, "q", rows * cols), (sq, "sq", rows * cols // 32), (qt, "qt", rows * cols),
                       (sqt, "sqt", rows * cols // 32)):
        _dev_tensor(t, n, torch.uint8)
        if t.numel() != size:
            raise ValueError(f"{n} has the wrong size")
    _run("fp8_mx_quantize_both", _lib.fp8_mx_quantize_both, (x, q, sq, qt, sqt), _ptr(x), rows, cols, int(fmt),
         _ptr(q), _ptr(sq), _ptr(qt), _ptr(sqt))
    return q, sq, qt, sqt


def mx_swiglu_requant(gu: torch.Tensor, hq: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """The SwiGLU output of gu = [gate | up] (bf16 [M, 2F], F a multiple of 128),
    block (MX) quantised to E4M3 along F: returns (hq uint8 [M, F], scales uint8
    [F / 128, M, 4])."""
    _dev_tensor(gu, "gu", torch.bfloat16)
    if gu.dim() != 2 or gu.shape[1] % 2:
        raise ValueError("gu must be [M, 2F]")
    M, F = gu.shape[0], gu.shape[1] // 2
    if hq is None:
        hq = torch.empty((M, F), dtype=torch.uint8, device=gu.device)
    if scales is None:
        scales = torch.empty((F // 128, M, 4), dtype=torch.uint8, device=gu.device)
    for t, n, size in ((hq, "hq", M * F), (scales, "scales", M * F // 32)):
        _dev_tensor(t, n, torch.uint8)
        if t.numel() != size:
            raise ValueError(f"{n} has the wrong size")
    _run("fp8_mx_swiglu_requant", _lib.fp8_mx_swiglu_requant, (gu, hq, scales), _ptr(gu), M, F, _ptr(hq),
         _ptr(scales))
    return hq, scales


def mx_gemm_fwd(xq, sx, wq, sw, x_fmt: int = E4M3, out=None) -> torch.Tensor:
    """Y[M, N] = bf16(sum_k dec(X) 2^ex dec(W) 2^ew) of block-scaled operands (from
    mx_quantize): xq uint8 [M, K] with sx uint8 [K / 128, M, 4], wq uint8 [N, K]
    (e4m3) with sw uint8 [K / 128, N, 4]."""
    for t, n in ((xq, "xq"), (sx, "sx"), (wq, "wq"), (sw, "sw")):
        _dev_tensor(t, n, torch.uint8)
    if xq.dim() != 2 or wq.dim() != 2 or xq.shape[1] != wq.shape[1]:
        raise ValueError("xq must be [M, K] and wq [N, K]")
    M, K = xq.shape
    N = wq.shape[0]
    if sx.numel() != M * (K // 32) or sw.numel() != N * (K // 32):
        raise ValueError("sx must hold M * K / 32 and sw N * K / 32 scales")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    _dev_tensor(out, "out", torch.bfloat16)
    if out.numel() != M * N:
        raise ValueError("out must be [M, N]")
    _run("fp8_mx_gemm_fwd", _lib.fp8_mx_gemm_fwd, (xq, sx, wq, sw, out), _ptr(xq), _ptr(sx), int(x_fmt), _ptr(wq),
         _ptr(sw), _ptr(out), M, N, K)
    return out


def mx_gemm_backward(dyq, sdy, dyqt, sdyt, wqt, swt, xqt, sxt, dy_fmt: int = E5M2, dx=None, dw=None):
    """Both backward products of a linear on block-scaled operands in one launch
    (fp8_mx_gemm_backward): dX [M, K] from dyq [M, N] (scales [N / 128, M, 4], from
    mx_quantize of dY) and wqt [K, N] (scales [N / 128, K, 4], mx_quantize_t of W);
    dW [N, K] from dyqt [N, M] (scales [M / 128, N, 4], mx_quantize_t of dY) and
    xqt [K, M] (scales [M / 128, K, 4], mx_quantize_t of X).  Returns (dx, dw)."""
    names = ("dyq", "sdy", "dyqt", "sdyt", "wqt", "swt", "xqt", "sxt")
    ts = (dyq, sdy, dyqt, sdyt, wqt, swt, xqt, sxt)
    for t, n in zip(ts, names):
        _dev_tensor(t, n, torch.uint8)
    if dyq.dim() != 2 or dyqt.dim() != 2 or wqt.dim() != 2 or xqt.dim() != 2:
        raise ValueError("codes must be 2-D")
    M, N = dyq.shape
    K = wqt.shape[0]
    if tuple(dyqt.shape) != (N, M) or tuple(wqt.shape) != (K, N) or tuple(xqt.shape) != (K, M):
        raise ValueError("expected dyq [M, N], dyqt [N, M], wqt [K, N], xqt [K, M]")
    for t, n, size in ((sdy, "sdy", M * N // 32), (sdyt, "sdyt", M * N // 32), (swt, "swt", K * N // 32),
                       (sxt, "sxt", K * M // 32)):
        if t.numel() != size:
            raise ValueError(f"{n} has the wrong size")
    if dx is None:
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dyq.device)
    if dw is None:
        dw = torch.empty((N, K), dtype=torch.bfloat16, device=dyq.device)
    for t, n, size in ((dx, "dx", M * K), (dw, "dw", N * K)):
        _dev_tensor(t, n, torch.bfloat16)
        if t.numel() != size:
            raise ValueError(f"{n} has the wrong size")
    _run("fp8_mx_gemm_backward", _lib.fp8_mx_gemm_backward, ts + (dx, dw), _ptr(dyq), _ptr(sdy), _ptr(dyqt),
         _ptr(sdyt), int(dy_fmt), _ptr(wqt), _ptr(swt), _ptr(xqt), _ptr(sxt), _ptr(dx), _ptr(dw), M, N, K)
    return dx, dw


def stream_copy(src: torch.Tensor, dst: torch.Tensor) -> torch.Tensor:
    """dst <- src byte for byte (fp8_stream_copy): the streaming-copy reference
    that the statistic and quantisation calls are measured against.  Both
    contiguous device tensors of the same byte size, a multiple of 16."""
    _dev_tensor(src, "src")
    _dev_tensor(dst, "dst")
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nb:
        raise ValueError("src and dst must hold the same number of bytes")
    _run("fp8_stream_copy", _lib.fp8_stream_copy, (src, dst), _ptr(src), _ptr(dst), nb)
    return dst
