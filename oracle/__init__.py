"""CPU oracle for the FP8 training hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and it
shares no code with it.

A thin numpy/ctypes layer over ``fp8_oracle.c`` (plain C, OpenMP,
``-O2 -ffp-contract=off``, no fast-math).  What each function computes, and the
passage of "LLMQ: Efficient Lower-Precision Pretraining for Consumer GPUs" or
of the FastML report that it follows, is written in the C file next to it.
"""
from .oracle import (  # noqa: F401
    E4M3, E5M2, FP8_MAX, build, lib_path, num_threads,
    bf16_to_f32, f32_to_bf16, encode, decode, absmax_bf16, absmax_f32, scale,
    quantize, exp_neg, swiglu_h, swiglu_requant, gemm, swiglu_grad, swiglu_grad_one, swiglu_backward,
    MX_BLOCK, mx_quantize, mx_gemm, mx_quantize_f32, mx_swiglu,
)
