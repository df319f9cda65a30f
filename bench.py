#!/usr/bin/env python3
"""Benchmark of the FP8 training hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input at the
shapes of one workload configuration (default layer7b: the 7B-class layer, M = 4096
tokens, d = 4096, ffn = 11008): for the QKV, O, gate/up and down linears,
forward and backward --

  forward:  absmax -> quantise to e4m3 (with the transposed copies the
            backward reads) for X and W -> FP8 GEMM -> bf16 Y; the gate/up
            output goes through the fused SwiGLU absmax + requantisation and
            the down linear consumes its e4m3 output.  The tensors ready at
            the start of the step (the four weights and the first linear's
            input) take their statistics in one launch and their
            quantisations in one launch;
  backward: absmax -> quantise dY to e5m2 (+ transposed copy) -> dgrad
            (dY . W) and wgrad (dY^T . X) FP8 GEMMs -> bf16.

--workload layer14b runs the 14B-class shapes (M = 8192, Student-t activations with
outlier channels); layer32b the 32B-class shapes (M = 16384) with the MLP block
recomputed in the backward from the retained absmax statistics.
--layout mn runs the same step without the transposed FP8 copies: the
quantise and SwiGLU calls write only the row-major codes and the backward
GEMMs read W, X, dY and h untransposed (fp8_gemm_backward_mn).

`value` is the step's GEMM work (2MNK summed over the GEMMs) divided by the
wall time of the whole step, quantisation included: effective FP8 TFLOP/s.
Inputs are resident in HBM before the timed region starts.

Besides the timed steps the line reports every call of the step (`breakdown`:
GEMM TFLOP/s, absmax / quantise / SwiGLU GB/s with their algorithmic bytes)
and `streaming`: the bytes-weighted GB/s of those streaming calls in the step,
the same calls timed one at a time with a cold Infinity Cache, each as % of the
8 TB/s HBM peak and against a plain copy kernel measured the same way.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload layer7b|layer14b|layer32b]
                       [--layout copies|mn] [--no-cold] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA peak
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E peak

# rocprofv3 kernel names of the library's kernels (format of A, format of B,
# edge tiles, layout set, half tiles, gate/up with the SwiGLU statistic,
# non-temporal output stores -- the backward products); a GEMM call whose last
# round is balanced runs a second launch of the half-tile instantiation
# ("bwd", format of dY, layout set): the dgrad + wgrad launches
GEMM_KERNEL = {"fwd": "fp8k::gemm_tn_kernel<0, 0, false, 0, false, false, false>",
               ("bwd", 1, 0): "fp8k::gemm_tn_kernel<1, 0, false, 0, false, false, true>",
               ("bwd", 1, 1): "fp8k::gemm_tn_kernel<1, 0, false, 1, false, false, true>",
               ("bwd", 0, 0): "fp8k::gemm_tn_kernel<0, 0, false, 0, false, false, true>",
               ("bwd", 0, 1): "fp8k::gemm_tn_kernel<0, 0, false, 1, false, false, true>",
               "gate_up": "fp8k::gemm_tn_kernel<0, 0, false, 0, false, true, false>"}


def half_tile_kernel(kernel):
    """The half-tile instantiation that balances the last round of `kernel`'s calls."""
    head, args = kernel[:-1].split("<", 1)
    a = [x.strip() for x in args.split(",")]
    a[4] = "true"
    return head + "<" + ", ".join(a) + ">"


def tail_launch(probs, kmajor, cus):
    """Whether a GEMM call also launches the half-tile kernel: the same rule as the
    library's launcher (K-major operands, no edge tiles, and the tiles past the
    last full round of `cus` workgroups fill at most half of it)."""
    if not kmajor or any(P < 256 or Q < 256 for P, Q, _, _ in probs):
        return False
    tail = sum(-(-P // 256) * -(-Q // 256) for P, Q, _, _ in probs) % cus
    return 0 < tail and 2 * tail <= cus
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_traffic_layer7b.txt")
GEMM_SOURCE = os.path.join(ROOT, "fp8_precision_amd", "csrc", "gemm.hip")


def gemm_code_hash():
    """SHA-256 (first 16 hex digits) of the GEMM source with its comments and
    whitespace removed: the key that ties the committed traffic counters to the
    kernel code they were taken on (a comment edit does not change it)."""
    import hashlib
    import re
    src = open(GEMM_SOURCE).read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return hashlib.sha256("".join(src.split()).encode()).hexdigest()[:16]


def measured_traffic(kernel, tail_fraction=0.0):
    """HBM bytes per call of `kernel` from the committed rocprofv3 PMC summary
    (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by a plain copy of known
    size; a call adds its half-tile launch's bytes, `tail_fraction` of the calls
    have one), or None when the summary is missing or the GEMM code changed
    since it was taken."""
    try:
        line = next(l for l in open(TRAFFIC_SUMMARY) if l.startswith("TRAFFIC_JSON "))
    except (OSError, StopIteration):
        return None
    data = json.loads(line[len("TRAFFIC_JSON "):])
    if gemm_code_hash() != data.get("gemm_code_sha256_16"):
        return None
    b = data["per_dispatch_bytes"].get(kernel)
    if b is None:
        return None
    if tail_fraction > 0:
        t = data["per_dispatch_bytes"].get(half_tile_kernel(kernel))
        if t is None:
            return None
        b += tail_fraction * t
    return int(b)


class Op:
    """One library call of the step, with its algorithmic work."""

    def __init__(self, name, fn, kind, work, kernel=None, meta=None):
        self.name, self.fn, self.kind, self.work, self.kernel = name, fn, kind, work, kernel
        self.meta = meta or {}


WORKLOADS = {
    "layer7b": "7B-class layer (d=4096, ffn=11008, QKV 4096->12288, M=4096 tokens): the four linears fwd+bwd, "
          "MLP forward chained through the fused SwiGLU requant",
    "layer14b": "14B-class layer (d=5120, ffn=13824, QKV 5120->7168, M=8192 tokens): the four linears fwd+bwd, "
          "Student-t(3) activations with 0.1% outlier channels x50, MLP forward chained through the SwiGLU requant",
    "layer32b": "32B-class layer (d=5120, ffn=27648, QKV 5120->7168, M=16384 tokens): the four linears fwd+bwd, "
          "MLP forward chained; backward recomputes the MLP block from the retained absmax statistics",
}


def build_step(fp8, dev, cfg_name="layer7b", layout="copies", swiglu_bwd=False, fused_absmax_h=False,
               quant_mode="pair", dy_fmt=None):
    """Inputs and the ordered list of calls of one layer step of a configuration.

    The step starts by clearing its buffer of per-tensor absmax statistics (one
    fill); every absmax then accumulates into its own slot.  With
    fused_absmax_h the SwiGLU statistic absmax_h comes out of the gate/up GEMM's
    epilogue (fp8_gemm_fwd_swiglu_absmax) and fp8_swiglu_requant runs without a
    reduction pass; by default (measured faster in this step) fp8_swiglu_requant
    takes it in its own pass.
    Forward (group_weights): the statistics of the four weights and of the QKV
    input in one launch, their quantisations in one launch; then for QKV, O and
    gate/up the FP8 GEMM, preceded (O, gate/up) by the absmax and quantisation
    of that linear's input.  Without group_weights each linear takes the
    statistics of its X and W in one launch and quantises them separately.
    The fused SwiGLU requant of the gate/up output feeds the down linear.
    Backward: absmax + e5m2 quantise of dY, then dgrad and wgrad in one launch.
    With recomputation (layer32b) the backward first re-quantises the retained bf16
    gate/up input with its retained absmax, reruns the gate/up GEMM and
    requantises the SwiGLU output with the retained absmax_h (no reduction), and
    the forward keeps no transposed copies for the MLP block.
    With swiglu_bwd the gate/up output gradient is not drawn: the down linear's
    dgrad output dH goes through the fused SwiGLU backward, whose e5m2
    d[gate | up] feeds the gate/up backward GEMMs.
    """
    mn = layout == "mn"
    cfg = workloads.CONFIGS[cfg_name]
    recompute = cfg.recompute
    M = cfg.M
    E4M3, E5M2 = fp8.E4M3, fp8.E5M2
    DY = E5M2 if dy_fmt is None else dy_fmt       # format of the output gradients
    ops = []
    bufs = {}
    f32 = lambda: torch.empty(1, dtype=torch.float32, device=dev)
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)
    bf = lambda *s: torch.empty(s, dtype=torch.bfloat16, device=dev)
    lin = {l.name: (i, l) for i, l in enumerate(cfg.linears)}
    gemm_fwd_kernel = GEMM_KERNEL["fwd"]
    # the step's per-tensor absmax statistics live in one buffer, cleared once at
    # the start of the step; each absmax accumulates into its slot
    stats = torch.empty(64, dtype=torch.float32, device=dev)
    ops.append(Op("clear statistics", lambda: fp8.absmax_clear(stats), "zero", 0))
    slots = iter(range(64))

    def quantize_op(tag, x, rows, cols, fmt, am, want_qt):
        sc, inv = f32(), f32()
        q, qt = u8(rows, cols), (u8(cols, rows) if want_qt else None)
        n = rows * cols
        ops.append(Op(f"quantize {tag}", lambda: fp8.quantize(x, fmt, am, q=q, qt=qt, scale=sc, inv_scale=inv),
                      "quantize", (4 if want_qt else 3) * n, meta={"rows": rows, "cols": cols, "fmt": fmt,
                                                                   "qt": want_qt}))
        return q, qt, inv

    def quant_pair_ops(name, x, w, L, want_xt, want_wt, pair_absmax=True, pair_quant=False):
        """A linear's input and weight: their statistics (in one launch, or two), then
        their quantisations (in one launch, or two)."""
        kx, kw = next(slots), next(slots)
        am_x, am_w = stats[kx:kx + 1], stats[kw:kw + 1]
        if pair_absmax:
            ops.append(Op(f"absmax X_{name}+W_{name}", lambda: fp8.absmax_accumulate_many([x, w], [am_x, am_w]),
                          "absmax", 2 * (M + L.N) * L.K, meta={"shapes": [(M, L.K), (L.N, L.K)]}))
        else:
            # the gate/up weight is streamed non-temporally: a shared launch would
            # stream X too and cost its quantisation the Infinity Cache (measured)
            for tag, t, am, r in (("X", x, am_x, M), ("W", w, am_w, L.N)):
                ops.append(Op(f"absmax {tag}_{name}", lambda t=t, am=am: fp8.absmax(t, am, accumulate=True),
                              "absmax", 2 * r * L.K, meta={"rows": r, "cols": L.K}))
        if not pair_quant:
            xq, xqt, inv_x = quantize_op(f"X_{name}", x, M, L.K, E4M3, am_x, want_xt)
            wq, wqt, inv_w = quantize_op(f"W_{name}", w, L.N, L.K, E4M3, am_w, want_wt)
            return xq, xqt, inv_x, am_x, wq, wqt, inv_w
        shp, want_t = [(M, L.K), (L.N, L.K)], [want_xt, want_wt]
        qs = [u8(r, c) for r, c in shp]
        qts = [u8(c, r) if t else None for (r, c), t in zip(shp, want_t)]
        scs, invs = [f32(), f32()], [f32(), f32()]
        # the transposed copies are for the backward pass: written non-temporally
        ops.append(Op(f"quantize X_{name}+W_{name}",
                      lambda: fp8.quantize_many([x, w], E4M3, [am_x, am_w], want_q=True, want_qt=want_t, qs=qs,
                                                qts=qts, scales=scs, inv_scales=invs, qt_later=True),
                      "quantize", sum((4 if t else 3) * r * c for (r, c), t in zip(shp, want_t)),
                      meta={"group": [{"rows": r, "cols": c, "fmt": E4M3, "qt": t} for (r, c), t in zip(shp, want_t)]}))
        return qs[0], qts[0], invs[0], am_x, qs[1], qts[1], invs[1]

    def quant_ops(tag, x, rows, cols, fmt, want_qt, qt_later=False):
        k = next(slots)
        am = stats[k:k + 1]
        ops.append(Op(f"absmax {tag}", lambda: fp8.absmax(x, am, accumulate=True), "absmax", 2 * rows * cols,
                      meta={"rows": rows, "cols": cols, "fmt": fmt}))
        if not (qt_later and want_qt):
            return quantize_op(tag, x, rows, cols, fmt, am, want_qt) + (am,)
        # a forward weight's transposed copy is for the backward pass: written non-temporally
        q, qt, sc, inv = u8(rows, cols), u8(cols, rows), f32(), f32()
        ops.append(Op(f"quantize {tag}", lambda: fp8.quantize_many([x], fmt, [am], want_q=True, want_qt=True, qs=[q],
                                                                   qts=[qt], scales=[sc], inv_scales=[inv],
                                                                   qt_later=True),
                      "quantize", 4 * rows * cols, meta={"rows": rows, "cols": cols, "fmt": fmt, "qt": True}))
        return q, qt, inv, am

    def gemm_fwd_op(tag, xq, wq, ix, iw, y, L, am_h=None):
        if am_h is None:
            fn = lambda: fp8.gemm_fwd(xq, wq, ix, iw, y)
        else:
            fn = lambda: fp8.gemm_fwd_swiglu_absmax(xq, wq, ix, iw, am_h, out=y)
        ops.append(Op(f"gemm_fwd {tag}", fn, "gemm", 2 * M * L.N * L.K,
                      GEMM_KERNEL["gate_up"] if am_h is not None else gemm_fwd_kernel,
                      {"probs": [(M, L.N, L.K, E4M3)], "kmajor": True, "swiglu_absmax": am_h is not None}))

    def swiglu_op(tag, gu, am_h, compute, want_hqt, F):
        hq, hqt, inv_h = u8(M, F), (u8(F, M) if want_hqt else None), f32()
        work = (4 * M * F if compute else 0) + (6 if want_hqt else 5) * M * F
        # a computed statistic accumulates into its (step-cleared) slot: no reset launch
        ops.append(Op(f"swiglu_requant {tag}", lambda: fp8.swiglu_requant(gu, am_h, compute, hq=hq, hqt=hqt,
                                                                         inv_scale_h=inv_h, accumulate=compute),
                      "swiglu", work, meta={"M": M, "F": F, "qt": want_hqt, "compute": compute}))
        return hq, hqt, inv_h

    # ---- forward
    fwd = {}
    # absmax_h of the SwiGLU output: from the gate/up GEMM's epilogue (one slot of
    # the step's statistics), or from the SwiGLU kernel's own reduction pass
    am_h = stats[63:64]
    names = ("qkv", "o", "gate_up", "down")
    xs = {n: workloads.draw_x(cfg, lin[n][0]).to(dev) for n in names[:3]}
    ws = {n: workloads.draw_w(cfg, lin[n][0]).to(dev) for n in names}
    for n in names:
        bufs[n] = (xs.get(n), ws[n])
    keep_xt = {n: not mn and not (recompute and n == "gate_up") for n in names[:3]}
    qd = {}      # (tensor tag) -> (q, qt, inv, absmax slot)
    group_weights = quant_mode == "step"
    if group_weights:
        # the tensors ready when the layer's step starts -- its four weights and the
        # first linear's input -- take their statistics in one launch and their
        # quantisations (with the transposed copies) in one launch
        tags = ["X_qkv"] + [f"W_{n}" for n in names]
        tens = [xs["qkv"]] + [ws[n] for n in names]
        shp = [(M, lin["qkv"][1].K)] + [(lin[n][1].N, lin[n][1].K) for n in names]
        want_t = [keep_xt["qkv"]] + [not mn] * 4
        ams = [stats[k:k + 1] for k in (next(slots) for _ in tags)]
        ops.append(Op("absmax [" + ", ".join(tags) + "]",
                      lambda: fp8.absmax_accumulate_many(tens, ams), "absmax", sum(2 * r * c for r, c in shp),
                      meta={"shapes": shp}))
        qs = [u8(r, c) for r, c in shp]
        qts = [u8(c, r) if t else None for (r, c), t in zip(shp, want_t)]
        scs, invs = [f32() for _ in tags], [f32() for _ in tags]
        ops.append(Op("quantize [" + ", ".join(tags) + "]",
                      lambda: fp8.quantize_many(tens, E4M3, ams, want_q=True, want_qt=want_t, qs=qs, qts=qts,
                                                scales=scs, inv_scales=invs, qt_later=True),
                      "quantize", sum((4 if t else 3) * r * c for (r, c), t in zip(shp, want_t)),
                      meta={"group": [{"rows": r, "cols": c, "fmt": E4M3, "qt": t} for (r, c), t in zip(shp, want_t)]}))
        for k, t in enumerate(tags):
            qd[t] = (qs[k], qts[k], invs[k], ams[k])
    for name in ("qkv", "o", "gate_up"):
        li, L = lin[name]
        x, w = xs[name], ws[name]
        if group_weights:
            if name != "qkv":
                xq, xqt, inv_x, am_x = quant_ops(f"X_{name}", x, M, L.K, E4M3, keep_xt[name], qt_later=True)
            else:
                xq, xqt, inv_x, am_x = qd["X_qkv"]
            wq, wqt, inv_w, _ = qd[f"W_{name}"]
        elif quant_mode == "pair":
            xq, xqt, inv_x, am_x, wq, wqt, inv_w = quant_pair_ops(name, x, w, L, keep_xt[name], not mn,
                                                                  pair_absmax=name != "gate_up", pair_quant=True)
        elif name != "gate_up":
            xq, xqt, inv_x, am_x, wq, wqt, inv_w = quant_pair_ops(name, x, w, L, keep_xt[name], not mn)
        else:
            # the gate/up weight is streamed non-temporally: a shared launch would
            # stream X too and cost its quantisation the Infinity Cache, for no
            # shorter statistics pass (measured)
            xq, xqt, inv_x, am_x = quant_ops(f"X_{name}", x, M, L.K, E4M3, keep_xt[name], qt_later=True)
            wq, wqt, inv_w, _ = quant_ops(f"W_{name}", w, L.N, L.K, E4M3, not mn, qt_later=True)
        y = bf(M, L.N)
        gemm_fwd_op(name, xq, wq, inv_x, inv_w, y, L, am_h if (name == "gate_up" and fused_absmax_h) else None)
        fwd[name] = {"x": x, "am_x": am_x, "xq": xq, "wq": wq, "xqt": xqt, "wqt": wqt, "inv_x": inv_x,
                     "inv_w": inv_w, "y": y}
    # SwiGLU requantisation of the gate/up output feeds the down linear
    li, L = lin["down"]
    F = L.K
    hq, hqt, inv_h = swiglu_op("fwd", fwd["gate_up"]["y"], am_h, not fused_absmax_h, not mn and not recompute, F)
    if group_weights:
        wq, wqt, inv_w, _ = qd["W_down"]
    else:
        wq, wqt, inv_w, _ = quant_ops("W_down", ws["down"], L.N, L.K, E4M3, not mn, qt_later=True)
    y = bf(M, L.N)
    gemm_fwd_op("down", hq, wq, inv_h, inv_w, y, L)
    fwd["down"] = {"xq": hq, "wq": wq, "xqt": hqt, "wqt": wqt, "inv_x": inv_h, "inv_w": inv_w, "y": y}

    # ---- backward
    gu2 = None
    if recompute:
        # MLP block recomputation from the retained bf16 input and absmax statistics: no reduction runs
        _, Lg = lin["gate_up"]
        g = fwd["gate_up"]
        xq, xqt, inv_x = quantize_op("X_gate_up (recompute)", g["x"], M, Lg.K, E4M3, g["am_x"], not mn)
        gu2 = bf(M, Lg.N)
        gemm_fwd_op("gate_up (recompute)", xq, g["wq"], inv_x, g["inv_w"], gu2, Lg)
        g.update({"xq": xq, "xqt": xqt, "inv_x": inv_x})
        hq2, hqt2, inv_h2 = swiglu_op("recompute", gu2, am_h, False, not mn, F)
        fwd["down"].update({"xq": hq2, "xqt": hqt2, "inv_x": inv_h2})
    gu_bwd = fwd["gate_up"]["y"] if not recompute else gu2
    order = ("down", "gate_up", "o", "qkv") if swiglu_bwd else ("qkv", "o", "gate_up", "down")
    dh = None
    for name in order:
        li, L = lin[name]
        f = fwd[name]
        if swiglu_bwd and name == "gate_up":
            # the MLP chain: dH (the down dgrad output) -> fused SwiGLU backward -> e5m2 d[gate | up]
            am, sc, inv_dy = f32(), f32(), f32()
            dyq, dyqt = u8(M, L.N), (None if mn else u8(L.N, M))
            Fh = L.N // 2
            ops.append(Op("swiglu_backward", lambda dyq=dyq, dyqt=dyqt, am=am, sc=sc, inv=inv_dy:
                          fp8.swiglu_backward(gu_bwd, dh, DY, q=dyq, qt=dyqt, absmax=am, scale=sc, inv_scale=inv),
                          "swiglu_bwd", (12 + (4 if not mn else 2)) * M * Fh,
                          meta={"M": M, "F": Fh, "qt": not mn}))
        else:
            dy = workloads.draw_dy(cfg, li).to(dev)
            bufs["dy_" + name] = dy
            dyq, dyqt, inv_dy, _ = quant_ops(f"dY_{name}", dy, M, L.N, DY, not mn)
        dx = bf(M, L.K)
        dw = bf(L.N, L.K)
        if name == "down":
            dh = dx
        # dgrad dX = dY . W and wgrad dW = dY^T . X in one launch
        if mn:
            fn = (lambda dyq=dyq, wq=f["wq"], xq=f["xq"], a=inv_dy, b=f["inv_w"], c=f["inv_x"], dx=dx, dw=dw:
                  fp8.gemm_backward_mn(dyq, DY, wq, xq, a, b, c, dx, dw))
        else:
            fn = (lambda dyq=dyq, dyqt=dyqt, wqt=f["wqt"], xqt=f["xqt"], a=inv_dy, b=f["inv_w"], c=f["inv_x"],
                  dx=dx, dw=dw: fp8.gemm_backward(dyq, dyqt, DY, wqt, xqt, a, b, c, dx, dw))
        ops.append(Op(f"gemm_backward {name}", fn, "gemm", 4 * M * L.N * L.K, GEMM_KERNEL[("bwd", DY, 1 if mn else 0)],
                      {"probs": [(M, L.K, L.N, DY), (L.N, L.K, M, DY)], "kmajor": not mn}))
    return ops, bufs


def run_step(ops):
    for op in ops:
        op.fn()


def time_steps(ops, steps, stream, instrument_kinds=("gemm",)):
    """Time `steps` steps; events bracket every call whose kind is listed."""
    evs = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        for op in ops:
            if op.kind in instrument_kinds:
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                op.fn()
                b.record(stream)
                evs.append((op, a, b))
            else:
                op.fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_op = {}
    for op, a, b in evs:
        per_op.setdefault(op.name, []).append(a.elapsed_time(b) * 1e-3)
    return wall, start.elapsed_time(end) * 1e-3, per_op


STREAM_KINDS = ("absmax", "quantize", "swiglu", "swiglu_bwd")
FLUSH_BYTES = 1 << 30               # a cold call follows a read of this many bytes


def time_stream_phases(ops, steps, stream):
    """The step's streaming phases -- each maximal run of consecutive absmax /
    quantise / SwiGLU calls between two GEMMs -- timed with one event pair per
    phase over `steps` steps: (seconds per step in streaming phases, bytes per
    step).  Fewer events than one pair per call, so less of their dispatch and
    completion overhead enters the figure."""
    phases, cur = [], []
    for op in ops:
        if op.kind in STREAM_KINDS:
            cur.append(op)
        elif cur:
            phases.append(cur)
            cur = []
    if cur:
        phases.append(cur)
    evs = []
    torch.cuda.synchronize()
    for _ in range(steps):
        k = 0
        for op in ops:
            if k < len(phases) and op is phases[k][0]:
                a = torch.cuda.Event(enable_timing=True)
                a.record(stream)
            op.fn()
            if k < len(phases) and op is phases[k][-1]:
                b = torch.cuda.Event(enable_timing=True)
                b.record(stream)
                evs.append((a, b))
                k += 1
    torch.cuda.synchronize()
    total = sum(a.elapsed_time(b) * 1e-3 for a, b in evs) / steps
    return total, sum(op.work for ph in phases for op in ph), len(phases)


def streaming_cold(fp8, ops, stream, dev, reps=20, warm=3):
    """Every absmax / quantise / SwiGLU call of the step timed on its own with a
    cold Infinity Cache (median of `reps`, each after a 1 GiB read: a read
    evicts the 256 MB cache without leaving dirty lines for the timed call to
    write back), and the library's streaming copy (fp8_stream_copy, 16-byte
    vectors at the launch shape where a copy is fastest on this chip) measured
    the same way as the achievable read+write reference; torch's copy_ is
    timed too, for context.  Calls that accumulate a statistic are idempotent,
    so repeating them is harmless."""
    flush = torch.ones(FLUSH_BYTES // 2, dtype=torch.bfloat16, device=dev)
    fam = torch.zeros(1, dtype=torch.float32, device=dev)

    def timed(fn):
        for _ in range(warm):
            fp8.absmax(flush, fam, accumulate=True)
            fn()
        pairs = []
        for _ in range(reps):
            fp8.absmax(flush, fam, accumulate=True)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            pairs.append((a, b))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) * 1e-3 for a, b in pairs]))

    src = torch.ones(1 << 27, dtype=torch.bfloat16, device=dev)          # 256 MiB
    dst = torch.empty_like(src)
    t_copy = timed(lambda: fp8.stream_copy(src, dst))
    copy_gbs = 2 * src.numel() * 2 / t_copy / 1e9
    t_torch = timed(lambda: dst.copy_(src))
    torch_copy_gbs = 2 * src.numel() * 2 / t_torch / 1e9
    del src, dst
    calls, tb, tt = [], 0, 0.0
    for op in ops:
        if op.kind not in STREAM_KINDS:
            continue
        t = timed(op.fn)
        gbs = op.work / t / 1e9
        calls.append({"call": op.name, "bytes": int(op.work), "us": round(t * 1e6, 2), "gbs": round(gbs, 1),
                      "pct_hbm": round(100 * gbs / HBM_PEAK_GBS, 1), "vs_copy": round(gbs / copy_gbs, 3)})
        tb += op.work
        tt += t
    del flush
    torch.cuda.empty_cache()
    agg = tb / tt / 1e9
    return copy_gbs, {"gbs": round(agg, 1), "pct_hbm": round(100 * agg / HBM_PEAK_GBS, 1),
                      "vs_copy": round(agg / copy_gbs, 3), "torch_copy_cold_gbs": round(torch_copy_gbs, 1),
                      "calls": calls}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(ops, gemm_rows):
    """The oracle, as it stands, on the same step: every absmax / quantise / SwiGLU
    call over its full tensor (random bf16 of the call's shape), every GEMM on
    `gemm_rows` and 2 * `gemm_rows` output rows, extrapolated linearly to all its
    rows (the two sizes separate the per-call cost of decoding B from the per-row
    cost).  Reported as the step's GEMM FLOP over the estimated step time.
    """
    import oracle
    oracle.build(force=False)
    threads = oracle.num_threads()
    rng = np.random.default_rng(0)
    gemm_est = gemm_spent = stream_s = 0.0
    stream_bytes = 0
    gemm_flop = 0.0
    t_start = time.perf_counter()

    def timed(fn):
        t = time.perf_counter()
        fn()
        return time.perf_counter() - t

    for op in ops:
        m = op.meta
        if op.kind == "gemm":
            for P, Q, R, fa in m["probs"]:
                b = rng.integers(0, 0x7E, (Q, R), dtype=np.uint8)
                times = []
                for r in (gemm_rows, 2 * gemm_rows):
                    a = rng.integers(0, 0x7E, (r, R), dtype=np.uint8)
                    times.append(timed(lambda: oracle.gemm(a, fa, b, 0, 1.0, 1.0)))
                gemm_spent += sum(times)
                per_row = max(times[1] - times[0], 0.0) / gemm_rows
                fixed = max(times[0] - per_row * gemm_rows, 0.0)
                gemm_est += fixed + per_row * P
                gemm_flop += 2.0 * P * Q * R
            if m.get("swiglu_absmax"):
                # the SwiGLU statistic this GEMM also produces: the oracle's reduction pass
                P, Q = m["probs"][0][:2]
                gu = rng.integers(0, 0x4080, (P, Q), dtype=np.uint16)
                stream_s += timed(lambda: oracle.swiglu_requant(gu, want_hq=False))
                stream_bytes += 2 * P * Q
                del gu
        elif op.kind == "absmax":
            for rows, cols in m.get("shapes", [(m.get("rows"), m.get("cols"))]):
                x = rng.integers(0, 0x3F80, (rows, cols), dtype=np.uint16)
                stream_s += timed(lambda: oracle.absmax_bf16(x))
                del x
            stream_bytes += op.work
        elif op.kind == "quantize":
            for g in m.get("group", [m]):
                x = rng.integers(0, 0x3F80, (g["rows"], g["cols"]), dtype=np.uint16)
                s_, _ = oracle.scale(np.float32(1.0), g["fmt"])
                stream_s += timed(lambda: oracle.quantize(x, g["fmt"], s_, want_q=True, want_qt=g["qt"]))
                del x
            stream_bytes += op.work
        elif op.kind == "swiglu_bwd":
            gu = rng.integers(0, 0x4080, (m["M"], 2 * m["F"]), dtype=np.uint16)
            dh = rng.integers(0, 0x3A80, (m["M"], m["F"]), dtype=np.uint16)
            stream_s += timed(lambda: oracle.swiglu_backward(gu, dh, 1, want_q=True, want_qt=m["qt"]))
            stream_bytes += op.work
            del gu, dh
        elif op.kind == "swiglu":
            gu = rng.integers(0, 0x4080, (m["M"], 2 * m["F"]), dtype=np.uint16)
            stream_s += timed(lambda: oracle.swiglu_requant(gu, absmax_h=None if m["compute"] else np.float32(8.0),
                                                            want_hq=True, want_hqt=m["qt"]))
            stream_bytes += op.work
            del gu
    spent = time.perf_counter() - t_start
    est = gemm_est + stream_s
    return {"value": round(gemm_flop / est / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "cpu_model": cpu_model(),
            "kind": "oracle",
            "streaming_full_s": round(stream_s, 3),
            "streaming_gbs": round(stream_bytes / stream_s / 1e9, 2) if stream_s > 0 else None,
            "gemm_sampled_s": round(gemm_spent, 3), "gemm_estimated_s": round(gemm_est, 2),
            "sample": (f"every absmax/quantise/SwiGLU call of the step over its full tensor ({stream_bytes / 1e9:.2f} GB "
                       f"in {stream_s:.2f} s); every GEMM on {gemm_rows} and {2 * gemm_rows} output rows "
                       f"({gemm_spent:.1f} s), extrapolated to all rows; {spent:.1f} s of CPU work in all (input "
                       f"generation included), estimated full step {est:.1f} s on {threads} threads")}


def step_shapes(fp8, dev, stream, cfg_name, steps=5, warmup=5):
    """The GEMM figures of another configuration's layer, measured inside that
    configuration's own step (the same construction as the headline's: its
    inputs drawn by workloads.py, every quantisation and SwiGLU call in place,
    so each GEMM reads operands the step has just written, as in training):
    `warmup` untimed steps, `steps` timed ones with no event inside, then as many
    with an event pair around every GEMM call for the per-call rates."""
    ops, _ = build_step(fp8, dev, cfg_name)
    torch.cuda.synchronize()
    for _ in range(warmup):
        run_step(ops)
    _, gpu_s, _ = time_steps(ops, steps, stream, instrument_kinds=())
    _, _, per = time_steps(ops, steps, stream)
    rows, tf, tt = [], 0.0, 0.0
    for op in ops:
        if op.kind != "gemm":
            continue
        t = float(np.mean(per[op.name]))
        rows.append({"call": op.name, "tflops": round(op.work / t / 1e12, 1),
                     "frac": round(op.work / t / 1e12 / FP8_PEAK_TFLOPS, 4), "us": round(t * 1e6, 1)})
        tf += op.work
        tt += t
    step_s = gpu_s / steps
    del ops
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"workload": WORKLOADS[cfg_name], "gemm_tflops": round(tf / tt / 1e12, 1),
            "frac": round(tf / tt / 1e12 / FP8_PEAK_TFLOPS, 4), "ms_per_step": round(step_s * 1e3, 4),
            "step_tflops": round(tf / step_s / 1e12, 1),
            "timing": f"inside the configuration's own step: {warmup} untimed steps, {steps} timed without events, "
                      f"then {steps} with an event pair around every GEMM call",
            "calls": rows}


def mx_layer(fp8, dev, cfg_name="layer7b", reps=10):
    """Block (MX) scaling next to the per-tensor path for each linear's forward and
    backward (the measured alternative, not the headline).  Per tensor: the
    statistics of X and W in one launch, their quantisation with the transposed
    copies in one launch, the forward GEMM; the statistic and e5m2 quantisation
    (with the transposed copy) of dY, the dgrad + wgrad launch.  MX: fp8_mx_quantize_both
    of X and of W (the forward blocking and, from the same read, the blocking along the
    backward reductions), the block-scaled forward; fp8_mx_quantize_both of dY (e5m2),
    the block-scaled dgrad + wgrad launch.  Inputs drawn by workloads.py; the two paths
    interleaved, `reps` rounds, an event pair around every call, medians."""
    cfg = workloads.CONFIGS[cfg_name]
    E4, E5 = fp8.E4M3, fp8.E5M2
    ev = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    u8 = lambda *sh: torch.empty(sh, dtype=torch.uint8, device=dev)
    f32 = lambda: torch.empty(1, dtype=torch.float32, device=dev)
    rows = []
    tot = {k: 0.0 for k in ("pt_qf", "pt_gf", "pt_qb", "pt_gb", "mx_qf", "mx_gf", "mx_qb", "mx_gb", "ff", "fb",
                            "bf", "bb")}
    for li, L in enumerate(cfg.linears):
        x = workloads.draw_x(cfg, li).to(dev)
        w = workloads.draw_w(cfg, li).to(dev)
        dy = workloads.draw_dy(cfg, li).to(dev)
        M, K, N = cfg.M, L.K, L.N
        stats = torch.zeros(3, dtype=torch.float32, device=dev)
        am = [stats[0:1], stats[1:2]]
        xq, wq, xqt, wqt = u8(M, K), u8(N, K), u8(K, M), u8(K, N)
        dyq, dyqt = u8(M, N), u8(N, M)
        sc = [f32() for _ in range(6)]
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        dw = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        mxq, mwq, mxt, mwt, mdq, mdt = u8(M, K), u8(N, K), u8(K, M), u8(K, N), u8(M, N), u8(N, M)
        sx, sw = u8(K // 128, M, 4), u8(K // 128, N, 4)
        sxt, swt = u8(M // 128, K, 4), u8(N // 128, K, 4)
        sdq, sdt = u8(N // 128, M, 4), u8(M // 128, N, 4)
        calls = {
            "pt_abs": lambda: fp8.absmax_accumulate_many([x, w], am),
            "pt_quant": lambda: fp8.quantize_many([x, w], E4, am, want_q=True, want_qt=True, qs=[xq, wq],
                                                  qts=[xqt, wqt], scales=[sc[0], sc[1]], inv_scales=[sc[2], sc[3]]),
            "pt_fwd": lambda: fp8.gemm_fwd(xq, wq, sc[2], sc[3], y),
            "pt_dyabs": lambda: fp8.absmax(dy, stats[2:3], accumulate=True),
            "pt_dyquant": lambda: fp8.quantize(dy, E5, stats[2:3], want_q=True, want_qt=True, q=dyq, qt=dyqt,
                                               scale=sc[4], inv_scale=sc[5]),
            "pt_bwd": lambda: fp8.gemm_backward(dyq, dyqt, E5, wqt, xqt, sc[5], sc[3], sc[2], dx, dw),
            # each tensor's two blockings from one read (the forward writes the backward's
            # operands, as the per-tensor forward writes its transposed copies)
            "mx_x": lambda: fp8.mx_quantize_both(x, E4, mxq, sx, mxt, sxt),
            "mx_w": lambda: fp8.mx_quantize_both(w, E4, mwq, sw, mwt, swt),
            "mx_fwd": lambda: fp8.mx_gemm_fwd(mxq, sx, mwq, sw, E4, out=y),
            "mx_dy": lambda: fp8.mx_quantize_both(dy, E5, mdq, sdq, mdt, sdt),
            "mx_bwd": lambda: fp8.mx_gemm_backward(mdq, sdq, mdt, sdt, mwt, swt, mxt, sxt, E5, dx=dx, dw=dw),
        }
        order = [["pt_abs", "pt_quant", "pt_fwd", "pt_dyabs", "pt_dyquant", "pt_bwd"],
                 ["mx_x", "mx_w", "mx_fwd", "mx_dy", "mx_bwd"]]
        t = {k: [] for k in calls}
        for r in range(reps + 2):
            for seq in order:
                fp8.absmax_clear(stats)
                pairs = []
                for k in seq:
                    a, b = ev()
                    a.record()
                    calls[k]()
                    b.record()
                    pairs.append((k, a, b))
                torch.cuda.synchronize()
                if r >= 2:
                    for k, a, b in pairs:
                        t[k].append(a.elapsed_time(b) * 1e-3)
        md = {k: float(np.median(v)) for k, v in t.items()}
        ff, fb = 2.0 * M * N * K, 4.0 * M * N * K
        v = {"pt_qf": md["pt_abs"] + md["pt_quant"], "pt_gf": md["pt_fwd"],
             "pt_qb": md["pt_dyabs"] + md["pt_dyquant"], "pt_gb": md["pt_bwd"],
             "mx_qf": md["mx_x"] + md["mx_w"], "mx_gf": md["mx_fwd"],
             "mx_qb": md["mx_dy"],
             "mx_gb": md["mx_bwd"], "ff": ff, "fb": fb,
             "bf": (M + N) * K, "bb": M * N}
        for k in tot:
            tot[k] += v[k]
        us = lambda k: round(v[k] * 1e6, 1)
        rows.append({"linear": L.name, "M": M, "N": N, "K": K,
                     "per_tensor": {"fwd_quantise_us": us("pt_qf"), "fwd_gemm_us": us("pt_gf"),
                                    "bwd_quantise_us": us("pt_qb"), "bwd_gemm_us": us("pt_gb")},
                     "mx": {"fwd_quantise_us": us("mx_qf"), "fwd_gemm_us": us("mx_gf"),
                            "bwd_quantise_us": us("mx_qb"), "bwd_gemm_us": us("mx_gb")}})
        del x, w, dy, xq, wq, xqt, wqt, dyq, dyqt, y, dx, dw, mxq, mwq, mxt, mwt, mdq, mdt
    # the SwiGLU requantisation between the gate/up and down products: the per-tensor
    # form (statistic pass + quantisation pass, hq only) against the MX form (one pass)
    F = cfg.linears[3].K
    gu = workloads.draw(cfg.seed, 99, (cfg.M, 2 * F), 1.0).to(dev)
    am_h = torch.zeros(1, dtype=torch.float32, device=dev)
    hq = torch.empty((cfg.M, F), dtype=torch.uint8, device=dev)
    inv_h = torch.empty(1, dtype=torch.float32, device=dev)
    mhq = torch.empty_like(hq)
    msc = torch.empty((F // 128, cfg.M, 4), dtype=torch.uint8, device=dev)
    sw_calls = {"pt": lambda: fp8.swiglu_requant(gu, am_h, 1, hq=hq, inv_scale_h=inv_h),
                "mx": lambda: fp8.mx_swiglu_requant(gu, hq=mhq, scales=msc)}
    sw_t = {k: [] for k in sw_calls}
    for r in range(reps + 2):
        for k, fn in sw_calls.items():
            a, b = ev()
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            if r >= 2:
                sw_t[k].append(a.elapsed_time(b) * 1e-3)
    sw_pt, sw_mx = float(np.median(sw_t["pt"])), float(np.median(sw_t["mx"]))
    n_h = cfg.M * F
    del gu, hq, mhq, msc
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    # algorithmic bytes per quantised element: per tensor, the statistic's 2-byte read,
    # then a 2-byte read and the code + transposed-copy writes; MX, one 2-byte read,
    # both blockings' codes and one scale byte per 32 codes of each
    epb = {"pt": 6.0, "mx": 4.0 + 2.0 / 32}
    gbs = lambda p, k, n: round(epb[p] * tot[n] / tot[p + k] / 1e9, 1)
    path = lambda p: {"fwd_quantise_us": round(tot[p + "_qf"] * 1e6, 1), "fwd_gemm_us": round(tot[p + "_gf"] * 1e6, 1),
                      "fwd_quantise_gbs": gbs(p, "_qf", "bf"),
                      "fwd_gemm_tflops": round(tot["ff"] / tot[p + "_gf"] / 1e12, 1),
                      "bwd_quantise_us": round(tot[p + "_qb"] * 1e6, 1), "bwd_gemm_us": round(tot[p + "_gb"] * 1e6, 1),
                      "bwd_quantise_gbs": gbs(p, "_qb", "bb"),
                      "bwd_gemm_tflops": round(tot["fb"] / tot[p + "_gb"] / 1e12, 1),
                      "total_us": round(sum(tot[p + k] for k in ("_qf", "_gf", "_qb", "_gb")) * 1e6
                                        + (sw_pt if p == "pt" else sw_mx) * 1e6, 1)}
    return {"workload": WORKLOADS[cfg_name] + ", forward and backward of each linear",
            "per_tensor": path("pt"),
            "mx": path("mx"),
            "swiglu": {"M": cfg.M, "F": F,
                       "per_tensor_us": round(sw_pt * 1e6, 1),
                       "per_tensor_gbs": round((4 + 5) * n_h / sw_pt / 1e9, 1),
                       "mx_us": round(sw_mx * 1e6, 1),
                       "mx_gbs": round((4 + 1 + 1 / 32) * n_h / sw_mx / 1e9, 1),
                       "note": "per tensor: the SwiGLU statistic pass, then the requantisation (hq only); MX: one "
                               "pass, block maxima local"},
            "timing": f"{reps} interleaved rounds, an event pair around every call, medians; total_us adds "
                      "the SwiGLU requantisation",
            "linears": rows}


def vs_hipblaslt(fp8, ops, dev, reps=10, rounds=3):
    """Every GEMM call of the step next to hipBLASLt (torch._scaled_mm, per-tensor
    scales, bf16 out) on the same FP8 operand bytes, timed interleaved (ours,
    hipBLASLt, ours, ...) so that neither runs at a different clock.  A
    backward call (dgrad + wgrad in one launch here) is compared with the two
    hipBLASLt products run back to back.  For context only."""
    dt = {fp8.E4M3: torch.float8_e4m3fn, fp8.E5M2: torch.float8_e5m2}

    def events(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        return a, b

    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    one = torch.ones((), dtype=torch.float32, device=dev)
    rows = []
    for op in ops:
        if op.kind != "gemm":
            continue
        calls = []
        for P, Q, R, fa in op.meta["probs"]:
            # operand codes of the step's kind: normal draws quantised with their own absmax
            a = torch.randn((P, R), generator=gen, device=dev, dtype=torch.bfloat16)
            b = torch.randn((Q, R), generator=gen, device=dev, dtype=torch.bfloat16)
            aq = fp8.quantize(a, fa, fp8.absmax(a))[0]
            bq = fp8.quantize(b, fp8.E4M3, fp8.absmax(b))[0]
            del a, b
            calls.append((aq, bq, fa, torch.empty((P, Q), dtype=torch.bfloat16, device=dev)))
        inv = torch.ones(1, dtype=torch.float32, device=dev)

        def ours():
            if len(calls) == 1:
                aq, bq, fa, y = calls[0]
                if fa == fp8.E4M3:
                    fp8.gemm_fwd(aq, bq, inv, inv, out=y)
                else:
                    fp8.gemm_dgrad(aq, fa, bq, inv, inv, out=y)
            else:
                # a backward call: dgrad (dY [M, N], W^T [K, N]) and wgrad (dY^T [N, M],
                # X^T [K, M]) in one launch
                (dyq, wqt, fa, dx), (dyqt, xqt, _, dw) = calls
                fp8.gemm_backward(dyq, dyqt, fa, wqt, xqt, inv, inv, inv, dx=dx, dw=dw)

        def theirs():
            for aq, bq, fa, y in calls:
                torch._scaled_mm(aq.view(dt[fa]), bq.view(torch.float8_e4m3fn).t(), scale_a=one, scale_b=one,
                                 out_dtype=torch.bfloat16, out=y)
        row = {"call": op.name, "gflop": round(op.work / 1e9, 1)}
        try:
            theirs()
        except Exception as ex:      # a format pair the vendor library does not take
            row["hipblaslt"] = f"n/a ({type(ex).__name__})"
            theirs = None
        ours()
        torch.cuda.synchronize()
        t_ours, t_theirs = [], []
        for _ in range(rounds):
            e1 = events(ours)
            e2 = events(theirs) if theirs else None
            torch.cuda.synchronize()
            t_ours.append(e1[0].elapsed_time(e1[1]) * 1e-3 / reps)
            if e2:
                t_theirs.append(e2[0].elapsed_time(e2[1]) * 1e-3 / reps)
        row["ours_tflops"] = round(op.work / float(np.median(t_ours)) / 1e12, 1)
        if t_theirs:
            row["hipblaslt_tflops"] = round(op.work / float(np.median(t_theirs)) / 1e12, 1)
        rows.append(row)
        del calls
        torch.cuda.empty_cache()
    return rows


def amd_smi_sampler():
    """A background sampler of the median graphics clock and the socket power
    (`amd-smi metric -c -p`); returns (start, stop) where stop() gives the
    (clock MHz, power W) samples taken meanwhile, or None without amd-smi."""
    import shutil
    import subprocess
    import threading
    exe = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    if not os.path.exists(exe):
        return None
    samples, stop_ev = [], threading.Event()

    def loop():
        while not stop_ev.is_set():
            try:
                r = subprocess.run([exe, "metric", "-c", "-p", "--json", "-g", "0"], capture_output=True, text=True,
                                   timeout=20)
                d = json.loads(r.stdout)
                g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
                clks = [v["clk"]["value"] for k, v in g["clock"].items()
                        if k.startswith("gfx_") and isinstance(v.get("clk"), dict)]
                pw = g["power"]["socket_power"]["value"]
                if clks:
                    samples.append((float(np.median(clks)), float(pw)))
            except Exception:   # a malformed or missing sample is skipped
                pass

    th = threading.Thread(target=loop, daemon=True)

    def stop():
        stop_ev.set()
        th.join(timeout=30)
        return samples
    return th.start, stop


def sustained_vs_hipblaslt(fp8, dev, shapes, seconds=2.0, rounds=2):
    """One forward GEMM shape at a time, this library and hipBLASLt alternately,
    each run back to back for `seconds` while amd-smi samples the clock and the
    socket power: TFLOP/s, and per GHz and per joule, under the power limit."""
    one = torch.ones((), dtype=torch.float32, device=dev)
    inv = torch.ones(1, dtype=torch.float32, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    rows = []
    for P, Q, R in shapes:
        a = torch.randn((P, R), generator=gen, device=dev, dtype=torch.bfloat16)
        b = torch.randn((Q, R), generator=gen, device=dev, dtype=torch.bfloat16)
        aq = fp8.quantize(a, fp8.E4M3, fp8.absmax(a))[0]
        bq = fp8.quantize(b, fp8.E4M3, fp8.absmax(b))[0]
        del a, b
        y = torch.empty((P, Q), dtype=torch.bfloat16, device=dev)
        fns = {"ours": lambda: fp8.gemm_fwd(aq, bq, inv, inv, out=y),
               "hipblaslt": lambda: torch._scaled_mm(aq.view(torch.float8_e4m3fn), bq.view(torch.float8_e4m3fn).t(),
                                                     scale_a=one, scale_b=one, out_dtype=torch.bfloat16, out=y)}
        flop = 2.0 * P * Q * R
        for _ in range(rounds):
            for name, fn in fns.items():
                for _ in range(20):
                    fn()
                torch.cuda.synchronize()
                sampler = amd_smi_sampler()
                if sampler:
                    sampler[0]()
                n, t0 = 0, time.perf_counter()
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record()
                while time.perf_counter() - t0 < seconds:
                    for _ in range(10):
                        fn()
                    n += 10
                    torch.cuda.synchronize()
                e.record()
                torch.cuda.synchronize()
                smp = sampler[1]() if sampler else []
                tf = flop / (s.elapsed_time(e) * 1e-3 / n) / 1e12
                row = {"shape": f"{P}x{Q}x{R}", "kernel": name, "tflops": round(tf, 1)}
                if smp:
                    mhz, w = float(np.median([x[0] for x in smp])), float(np.median([x[1] for x in smp]))
                    row.update({"gfx_mhz": round(mhz), "power_w": round(w), "tflops_per_ghz": round(tf / (mhz / 1e3), 1),
                                "gflop_per_joule": round(tf * 1e3 / w, 1), "samples": len(smp)})
                rows.append(row)
        del aq, bq, y
        torch.cuda.empty_cache()
    return rows


def sustained_clock(ops, seconds=4.0):
    """Median graphics clock and socket power while the step loops (outside the timed region).

    A background thread queries `amd-smi metric -c -p --json` (current clock of
    every graphics clock domain, socket power) while the main thread keeps the
    GPU busy with the step.  Returns None when amd-smi is not available.
    """
    sampler = amd_smi_sampler()
    if sampler is None:
        return None
    for _ in range(5):          # the clock ramps up under load
        run_step(ops)
    sampler[0]()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(20):
            run_step(ops)
        torch.cuda.synchronize()
    samples = sampler[1]()
    if not samples:
        return None
    c = float(np.median([x[0] for x in samples]))
    return {"gfx_mhz_median": round(c, 1), "socket_power_w_median": float(np.median([x[1] for x in samples])),
            "samples": len(samples), "source": "amd-smi metric -c -p while the step loops, after the timed region"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baseline", action="store_true",
                    help="also time the oracle for the layer14b / layer32b workloads (always done for layer7b unless disabled)")
    ap.add_argument("--layout", choices=("copies", "mn"), default="copies",
                    help="backward GEMM operands: transposed FP8 copies, or the untransposed tensors")
    ap.add_argument("--cpu-gemm-rows", type=int, default=128)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="layer7b",
                    help="layer7b: 7B-class layer (the headline); layer14b: 14B-class; layer32b: 32B-class with MLP recomputation")
    ap.add_argument("--fused-swiglu-absmax", action="store_true",
                    help="take the SwiGLU statistic in the gate/up GEMM's epilogue (fp8_gemm_fwd_swiglu_absmax) "
                         "instead of fp8_swiglu_requant's own reduction pass")
    ap.add_argument("--swiglu-backward", action="store_true",
                    help="chain the MLP backward: down dgrad -> fused SwiGLU backward -> gate/up backward "
                         "(instead of a drawn gate/up output gradient)")
    ap.add_argument("--breakdown", action="store_true",
                    help="accepted for compatibility: the per-call breakdown is always reported")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache per-call streaming measurement")
    ap.add_argument("--no-clock", action="store_true", help="skip the sustained-clock sampling (amd-smi)")
    ap.add_argument("--no-shapes", action="store_true",
                    help="skip the 14B- and 32B-class layer steps (their GEMM figures) reported with the layer7b "
                         "workload")
    ap.add_argument("--no-mx", action="store_true",
                    help="skip the block-scaled (MX) layer measurement reported with the layer7b workload")
    ap.add_argument("--quant-mode", choices=("pair", "linear", "step"), default="pair",
                    help="pair: each linear's X and W quantised in one launch (their statistics in one launch for "
                         "QKV and O); linear: X and W quantised in separate launches; step: the four weights and the "
                         "first input quantised together at the start of the step")
    ap.add_argument("--dy-format", choices=("e5m2", "e4m3"), default="e5m2",
                    help="format of the output gradients dY (e5m2: the default reading; e4m3: the all-E4M3 variant)")
    ap.add_argument("--mx-only", action="store_true",
                    help="only run the block-scaled (MX) layer comparison and print it as the JSON line (context, "
                         "not the metric)")
    ap.add_argument("--vs-hipblaslt", action="store_true",
                    help="only compare every GEMM call of the step with hipBLASLt (torch._scaled_mm) on the same "
                         "operand bytes, interleaved, and print that as the JSON line (context, not the metric)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the path has no multi-GPU code; "
              "its value is one GPU's throughput.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        sys.exit(2)
    import fp8_precision_amd as fp8

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    cfg = workloads.CONFIGS[args.workload]
    if args.mx_only:
        print(json.dumps({"mx_layer": mx_layer(fp8, dev, args.workload)}))
        return
    if args.vs_hipblaslt:
        ops, _ = build_step(fp8, dev, args.workload, "copies", False, False)
        for _ in range(3):
            run_step(ops)
        rows = vs_hipblaslt(fp8, ops, dev)
        sus = sustained_vs_hipblaslt(fp8, dev, [(4096, 12288, 4096), (4096, 4096, 11008), (4096, 4096, 4096)])
        print(json.dumps({"comparison": "hipBLASLt (torch._scaled_mm, per-tensor scales, bf16 out) vs this library, "
                                        "same FP8 operand bytes, interleaved, median of 3 rounds of 10 calls",
                          "workload": args.workload, "calls": rows,
                          "sustained": {"note": "forward shapes, each kernel back to back for 2 s, alternating, with "
                                                "amd-smi sampling the graphics clock and socket power",
                                        "runs": sus}}))
        return
    ops, bufs = build_step(fp8, dev, args.workload, args.layout, args.swiglu_backward,
                           args.fused_swiglu_absmax, args.quant_mode,
                           fp8.E4M3 if args.dy_format == "e4m3" else fp8.E5M2)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        run_step(ops)
    torch.cuda.synchronize()

    # the timed steps carry no per-call events: an event recorded between a GEMM
    # and its neighbours leaves the GPU idle for ~5.6 us (rocprofv3 trace), 16
    # times a step; per-call times come from the instrumented pass below
    wall, gpu_s, _ = time_steps(ops, args.steps, stream, instrument_kinds=())
    step_s = gpu_s / args.steps
    gemm_flop = sum(op.work for op in ops if op.kind == "gemm")
    value = gemm_flop / step_s / 1e12

    # every call of the step, in the step (a separate instrumented pass: events
    # around each call; the pipeline's legitimate cache reuse included)
    _, _, per_all = time_steps(ops, max(3, args.steps // 2), stream,
                               instrument_kinds=("gemm", "zero") + STREAM_KINDS)

    # dominant kernel: the GEMM kernel with the largest summed time in the step;
    # its figures are per library call (a call may add a half-tile tail launch)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    by_kernel = {}
    for op in ops:
        if op.kind != "gemm":
            continue
        d = by_kernel.setdefault(op.kernel, {"flop": 0.0, "time": 0.0, "launches": 0, "tail_launches": 0})
        ts = per_all[op.name]
        d["flop"] += op.work
        d["time"] += float(np.mean(ts))
        d["launches"] += 1
        d["tail_launches"] += tail_launch(op.meta["probs"], op.meta["kmajor"], cus)
    dom_name, dom = max(by_kernel.items(), key=lambda kv: kv[1]["time"])
    achieved = dom["flop"] / dom["time"] / 1e12
    gemm_time = sum(d["time"] for d in by_kernel.values())

    breakdown = []
    for op in ops:
        t = float(np.mean(per_all[op.name]))
        if op.kind == "zero":
            breakdown.append({"call": op.name, "us": round(t * 1e6, 2)})
            continue
        if op.kind == "gemm":
            breakdown.append({"call": op.name, "us": round(t * 1e6, 2), "rate": round(op.work / t / 1e12, 1),
                              "unit": "TFLOP/s"})
        else:
            breakdown.append({"call": op.name, "bytes": int(op.work), "us": round(t * 1e6, 2),
                              "rate": round(op.work / t / 1e9, 1), "unit": "GB/s"})
    qt = sum(float(np.mean(per_all[op.name])) for op in ops if op.kind in STREAM_KINDS)
    qb = sum(op.work for op in ops if op.kind in STREAM_KINDS)
    quant_gbs = qb / qt / 1e9
    ph_s, ph_b, n_ph = time_stream_phases(ops, max(3, args.steps // 2), stream)
    phase_gbs = ph_b / ph_s / 1e9
    copy_gbs, cold = (None, None) if args.no_cold else streaming_cold(fp8, ops, stream, dev)

    shapes = {}
    if args.workload == "layer7b" and not args.no_shapes:
        for other in ("layer14b", "layer32b"):
            shapes[other] = step_shapes(fp8, dev, stream, other)
    mx = mx_layer(fp8, dev) if args.workload == "layer7b" and not args.no_mx else None
    clock = None if args.no_clock else sustained_clock(ops)
    want_cpu = not args.no_cpu_baseline and (args.workload == "layer7b" or args.cpu_baseline)
    cpu = cpu_baseline(ops, args.cpu_gemm_rows) if want_cpu else None

    line = {
        "metric": "FP8 GEMM TFLOP/s + % of MI355X FP8 peak at 7B shapes; quant/absmax HBM GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.workload], "name": args.workload, "M": cfg.M,
                   "linears": {l.name: [l.K, l.N] for l in cfg.linears},
                   "gemm_launches": sum(1 for op in ops if op.kind == "gemm"),
                   "backward_operands": "untransposed (MN-major)" if args.layout == "mn" else "transposed copies",
                   "mlp_backward": "chained through the fused SwiGLU backward" if args.swiglu_backward
                   else "drawn output gradients",
                   "swiglu_absmax": ("gate/up GEMM epilogue" if args.fused_swiglu_absmax
                                     else "separate reduction pass"),
                   "dy_format": args.dy_format,
                   "quantisation_launches": {"pair": "X and W of a linear in one launch",
                                             "linear": "X and W of a linear in separate launches",
                                             "step": "the weights and the layer input in one launch at step start"
                                             }[args.quant_mode],
                   "gemm_gflop_per_step": round(gemm_flop / 1e9, 1)},
        "pct_fp8_peak": round(100 * value / FP8_PEAK_TFLOPS, 2),
        "gemm_only_tflops": round(gemm_flop / gemm_time / 1e12, 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(dom_name, dom["tail_launches"] / dom["launches"]),
                     "kernel": dom_name, "launches_per_step": dom["launches"],
                     "tail_launches_per_step": dom["tail_launches"],
                     "peak_at_sustained_clock": (round(FP8_PEAK_TFLOPS * clock["gfx_mhz_median"] / 2400.0, 1)
                                                 if clock else None),
                     "frac_at_sustained_clock": (round(achieved / (FP8_PEAK_TFLOPS * clock["gfx_mhz_median"] / 2400.0), 4)
                                                 if clock else None),
                     "avg_launch_us": round(dom["time"] / dom["launches"] * 1e6, 2),
                     "timing": "per library call (events around the call, in an instrumented pass after the timed steps), "
                               "including its tail launch if any"},
        "cpu_baseline": cpu,
        "sustained_clock": clock,
        "wall_s": round(wall, 3),
    }
    line["quant_absmax_swiglu_gbs"] = round(quant_gbs, 1)
    line["streaming"] = {
        "unit": "GB/s", "hbm_peak": HBM_PEAK_GBS, "copy_cold_gbs": round(copy_gbs, 1) if copy_gbs else None,
        "copy": "fp8_stream_copy, 256 MiB each way after a 1 GiB read (both directions counted)",
        "in_step_phases": {"gbs": round(phase_gbs, 1), "pct_hbm": round(100 * phase_gbs / HBM_PEAK_GBS, 1),
                           "vs_copy": round(phase_gbs / copy_gbs, 3) if copy_gbs else None, "bytes": int(ph_b),
                           "phases": n_ph, "note": "one event pair per run of consecutive streaming calls between "
                                                   "two GEMMs"},
        "in_step": {"gbs": round(quant_gbs, 1), "pct_hbm": round(100 * quant_gbs / HBM_PEAK_GBS, 1),
                    "vs_copy": round(quant_gbs / copy_gbs, 3) if copy_gbs else None,
                    "bytes": int(qb), "note": "bytes-weighted over the step's absmax/quantise/SwiGLU calls"},
        "cold": cold,
    }
    if shapes:
        line["shapes"] = shapes
    if mx:
        line["mx_layer"] = mx
    line["breakdown"] = breakdown
    print(json.dumps(line))


if __name__ == "__main__":
    main()
