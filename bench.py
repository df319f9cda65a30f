#!/usr/bin/env python3
"""Benchmark of the FP8 training hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input at
7B-class shapes (M = 4096 tokens, d = 4096, ffn = 11008): for the QKV, O,
gate/up and down linears, forward and backward --

  forward:  absmax -> quantise to e4m3 (with the transposed copies the
            backward reads) for X and W -> FP8 GEMM -> bf16 Y; the gate/up
            output goes through the fused SwiGLU absmax + requantisation and
            the down linear consumes its e4m3 output;
  backward: absmax -> quantise dY to e5m2 (+ transposed copy) -> dgrad
            (dY . W) and wgrad (dY^T . X) FP8 GEMMs -> bf16.

--layout mn runs the same step without the transposed FP8 copies: the
quantise and SwiGLU calls write only the row-major codes and the backward
GEMMs read W, X, dY and h untransposed (fp8_gemm_backward_mn).

`value` is the step's GEMM work (2MNK summed over the 12 GEMMs) divided by the
wall time of the whole step, quantisation included: effective FP8 TFLOP/s.
Inputs are resident in HBM before the timed region starts.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--layout copies|mn] [--no-cpu-baseline]
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

# rocprofv3 kernel names of the library's kernels
GEMM_KERNEL = {(0, 0, 0): "fp8k::gemm_tn_kernel<0, 0, false, 0>", (1, 0, 0): "fp8k::gemm_tn_kernel<1, 0, false, 0>",
               (1, 0, 1): "fp8k::gemm_tn_kernel<1, 0, false, 1>"}
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_traffic_layer7b.txt")
GEMM_SOURCE = os.path.join(ROOT, "fp8_precision_amd", "csrc", "gemm.hip")


def measured_traffic(kernel):
    """HBM bytes per dispatch of `kernel` from the committed rocprofv3 PMC summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by a plain copy of known size), or
    None when the summary is missing or the GEMM source changed since it was taken."""
    import hashlib
    try:
        line = next(l for l in open(TRAFFIC_SUMMARY) if l.startswith("TRAFFIC_JSON "))
    except (OSError, StopIteration):
        return None
    data = json.loads(line[len("TRAFFIC_JSON "):])
    if hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()[:16] != data["gemm_source_sha256_16"]:
        return None
    b = data["per_dispatch_bytes"].get(kernel)
    return None if b is None else int(b)


class Op:
    """One library call of the step, with its algorithmic work."""

    def __init__(self, name, fn, kind, work, kernel=None, meta=None):
        self.name, self.fn, self.kind, self.work, self.kernel = name, fn, kind, work, kernel
        self.meta = meta or {}


def build_layer7b(fp8, dev, layout="copies"):
    """Inputs and the ordered list of calls of one 7B-layer step."""
    mn = layout == "mn"
    cfg = workloads.CONFIGS["c3"]
    M = cfg.M
    E4M3, E5M2 = fp8.E4M3, fp8.E5M2
    ops = []
    bufs = {}
    f32 = lambda: torch.empty(1, dtype=torch.float32, device=dev)
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)
    bf = lambda *s: torch.empty(s, dtype=torch.bfloat16, device=dev)
    lin = {l.name: (i, l) for i, l in enumerate(cfg.linears)}

    def quant_ops(tag, x, rows, cols, fmt):
        am, sc, inv = f32(), f32(), f32()
        q, qt = u8(rows, cols), (None if mn else u8(cols, rows))
        n = rows * cols
        ops.append(Op(f"absmax {tag}", lambda: fp8.absmax(x, am), "absmax", 2 * n,
                      meta={"rows": rows, "cols": cols, "fmt": fmt}))
        ops.append(Op(f"quantize {tag}", lambda: fp8.quantize(x, fmt, am, q=q, qt=qt, scale=sc, inv_scale=inv),
                      "quantize", (3 if mn else 4) * n, meta={"rows": rows, "cols": cols, "fmt": fmt, "qt": not mn}))
        return q, qt, inv

    # ---- forward
    fwd = {}
    for name in ("qkv", "o", "gate_up"):
        li, L = lin[name]
        x = workloads.draw_x(cfg, li).to(dev)
        w = workloads.draw_w(cfg, li).to(dev)
        bufs[name] = (x, w)
        xq, xqt, inv_x = quant_ops(f"X_{name}", x, M, L.K, E4M3)
        wq, wqt, inv_w = quant_ops(f"W_{name}", w, L.N, L.K, E4M3)
        y = bf(M, L.N)
        ops.append(Op(f"gemm_fwd {name}", lambda xq=xq, wq=wq, ix=inv_x, iw=inv_w, y=y: fp8.gemm_fwd(xq, wq, ix, iw, y),
                      "gemm", 2 * M * L.N * L.K, GEMM_KERNEL[(0, 0, 0)], {"probs": [(M, L.N, L.K, E4M3)]}))
        fwd[name] = (xq, wq, xqt, wqt, inv_x, inv_w, y)
    # SwiGLU requantisation of the gate/up output feeds the down linear
    li, L = lin["down"]
    F = L.K
    gu = fwd["gate_up"][6]
    am_h, inv_h = f32(), f32()
    hq, hqt = u8(M, F), (None if mn else u8(F, M))
    ops.append(Op("swiglu_requant fwd", lambda: fp8.swiglu_requant(gu, am_h, True, hq=hq, hqt=hqt, inv_scale_h=inv_h),
                  "swiglu", 4 * M * F + (5 if mn else 6) * M * F, meta={"M": M, "F": F, "qt": not mn}))
    w = workloads.draw_w(cfg, li).to(dev)
    bufs["down"] = (None, w)
    wq, wqt, inv_w = quant_ops("W_down", w, L.N, L.K, E4M3)
    y = bf(M, L.N)
    ops.append(Op("gemm_fwd down", lambda: fp8.gemm_fwd(hq, wq, inv_h, inv_w, y), "gemm", 2 * M * L.N * L.K,
                  GEMM_KERNEL[(0, 0, 0)], {"probs": [(M, L.N, L.K, E4M3)]}))
    fwd["down"] = (hq, wq, hqt, wqt, inv_h, inv_w, y)

    # ---- backward
    for name in ("qkv", "o", "gate_up", "down"):
        li, L = lin[name]
        dy = workloads.draw_dy(cfg, li).to(dev)
        xq, wq, xqt, wqt, inv_x, inv_w, _ = fwd[name]
        dyq, dyqt, inv_dy = quant_ops(f"dY_{name}", dy, M, L.N, E5M2)
        dx = bf(M, L.K)
        dw = bf(L.N, L.K)
        # dgrad dX = dY . W and wgrad dW = dY^T . X in one launch
        if mn:
            fn = (lambda dyq=dyq, wq=wq, xq=xq, a=inv_dy, b=inv_w, c=inv_x, dx=dx, dw=dw:
                  fp8.gemm_backward_mn(dyq, E5M2, wq, xq, a, b, c, dx, dw))
        else:
            fn = (lambda dyq=dyq, dyqt=dyqt, wqt=wqt, xqt=xqt, a=inv_dy, b=inv_w, c=inv_x, dx=dx, dw=dw:
                  fp8.gemm_backward(dyq, dyqt, E5M2, wqt, xqt, a, b, c, dx, dw))
        ops.append(Op(f"gemm_backward {name}", fn, "gemm", 4 * M * L.N * L.K, GEMM_KERNEL[(1, 0, 1 if mn else 0)],
                      {"probs": [(M, L.K, L.N, E5M2), (L.N, L.K, M, E5M2)]}))
        bufs["dy_" + name] = dy
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


def cpu_baseline(ops, gemm_rows):
    """The oracle, as it stands, on a bounded sample of the same step, scaled to a full step.

    Sample: every absmax / quantise / SwiGLU call over its full tensor (random
    bf16 of the same shape); every GEMM on `gemm_rows` and 2 * `gemm_rows`
    output rows, extrapolated linearly to all its rows.
    """
    import oracle
    oracle.build(force=False)
    threads = oracle.num_threads()
    rng = np.random.default_rng(0)
    est = 0.0
    gemm_flop = 0.0
    t_start = time.perf_counter()
    for op in ops:
        m = op.meta
        if op.kind == "gemm":
            for P, Q, R, fa in m["probs"]:
                # two sample sizes separate the per-call cost (decoding B) from the per-row cost
                b = rng.integers(0, 0x7E, (Q, R), dtype=np.uint8)
                times = []
                for r in (gemm_rows, 2 * gemm_rows):
                    a = rng.integers(0, 0x7E, (r, R), dtype=np.uint8)
                    t = time.perf_counter()
                    oracle.gemm(a, fa, b, 0, 1.0, 1.0)
                    times.append(time.perf_counter() - t)
                per_row = max(times[1] - times[0], 0.0) / gemm_rows
                fixed = max(times[0] - per_row * gemm_rows, 0.0)
                est += fixed + per_row * P
                gemm_flop += 2.0 * P * Q * R
        elif op.kind == "absmax":
            x = rng.integers(0, 0x3F80, (m["rows"], m["cols"]), dtype=np.uint16)
            t = time.perf_counter()
            oracle.absmax_bf16(x)
            est += time.perf_counter() - t
        elif op.kind == "quantize":
            x = rng.integers(0, 0x3F80, (m["rows"], m["cols"]), dtype=np.uint16)
            t = time.perf_counter()
            s_, _ = oracle.scale(oracle.absmax_bf16(x), m["fmt"])
            oracle.quantize(x, m["fmt"], s_, want_q=True, want_qt=m["qt"])
            est += time.perf_counter() - t
        elif op.kind == "swiglu":
            gu = rng.integers(0, 0x4080, (m["M"], 2 * m["F"]), dtype=np.uint16)
            t = time.perf_counter()
            oracle.swiglu_requant(gu, want_hq=True, want_hqt=m["qt"])
            est += time.perf_counter() - t
    spent = time.perf_counter() - t_start
    return {"value": round(gemm_flop / est / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": (f"every absmax/quantise/SwiGLU call of the step over its full tensor, every GEMM on "
                       f"{gemm_rows} and {2 * gemm_rows} output rows extrapolated to all rows; {spent:.1f} s of CPU work, "
                       f"estimated full step {est:.1f} s on {threads} threads")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layout", choices=("copies", "mn"), default="copies",
                    help="backward GEMM operands: transposed FP8 copies, or the untransposed tensors")
    ap.add_argument("--cpu-gemm-rows", type=int, default=16)
    ap.add_argument("--breakdown", action="store_true", help="also time every call (separate pass)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); every box here has one GPU "
              "and this path has no multi-GPU code.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        sys.exit(2)
    import fp8_precision_amd as fp8

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    ops, bufs = build_layer7b(fp8, dev, args.layout)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        run_step(ops)
    torch.cuda.synchronize()

    wall, gpu_s, per_op = time_steps(ops, args.steps, stream)
    step_s = gpu_s / args.steps
    gemm_flop = sum(op.work for op in ops if op.kind == "gemm")
    value = gemm_flop / step_s / 1e12

    # dominant kernel: the GEMM kernel with the largest summed time in the step
    by_kernel = {}
    for op in ops:
        if op.kind != "gemm":
            continue
        d = by_kernel.setdefault(op.kernel, {"flop": 0.0, "time": 0.0, "launches": 0})
        ts = per_op[op.name]
        d["flop"] += op.work
        d["time"] += float(np.mean(ts))
        d["launches"] += 1
    dom_name, dom = max(by_kernel.items(), key=lambda kv: kv[1]["time"])
    achieved = dom["flop"] / dom["time"] / 1e12
    gemm_time = sum(d["time"] for d in by_kernel.values())

    breakdown = None
    if args.breakdown:
        _, _, per_all = time_steps(ops, max(3, args.steps // 2), stream,
                                   instrument_kinds=("gemm", "absmax", "quantize", "swiglu"))
        breakdown = []
        for op in ops:
            t = float(np.mean(per_all[op.name]))
            unit = "TFLOP/s" if op.kind == "gemm" else "GB/s"
            rate = op.work / t / (1e12 if op.kind == "gemm" else 1e9)
            breakdown.append({"call": op.name, "us": round(t * 1e6, 2), "rate": round(rate, 1), "unit": unit})
        qt = sum(float(np.mean(per_all[op.name])) for op in ops if op.kind != "gemm")
        qb = sum(op.work for op in ops if op.kind != "gemm")
        quant_gbs = qb / qt / 1e9
    else:
        quant_gbs = None

    cpu = None if args.no_cpu_baseline else cpu_baseline(ops, args.cpu_gemm_rows)

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
        "config": {"workload": "7B-class layer linears fwd+bwd with SwiGLU requant chain (c3 shapes + c2 MLP chain)",
                   "M": 4096, "d": 4096, "ffn": 11008, "qkv_out": 12288, "gemms": 12, "gemm_launches": 8,
                   "backward_operands": "untransposed (MN-major)" if args.layout == "mn" else "transposed copies",
                   "gemm_gflop_per_step": round(gemm_flop / 1e9, 1)},
        "pct_fp8_peak": round(100 * value / FP8_PEAK_TFLOPS, 2),
        "gemm_only_tflops": round(gemm_flop / gemm_time / 1e12, 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(dom_name),
                     "kernel": dom_name, "launches_per_step": dom["launches"],
                     "avg_launch_us": round(dom["time"] / dom["launches"] * 1e6, 2)},
        "cpu_baseline": cpu,
        "wall_s": round(wall, 3),
    }
    if quant_gbs is not None:
        line["quant_absmax_swiglu_gbs"] = round(quant_gbs, 1)
        line["breakdown"] = breakdown
    print(json.dumps(line))


if __name__ == "__main__":
    main()
