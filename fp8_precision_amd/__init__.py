"""MI355X (gfx950) FP8 training hot path: absmax, quantise, SwiGLU requant, FP8 GEMMs.

The compute runs in hand-written HIP kernels behind the C ABI declared in
``include/fp8_precision.h``; this package is the thin Python binding over it.
"""
from ._lib import (  # noqa: F401
    E4M3, E5M2, EXPORTED, LIB_PATH, Fp8Error,
    absmax, absmax_accumulate_many, absmax_clear, quantize, quantize_many, swiglu_requant, swiglu_backward, gemm_fwd, gemm_fwd_swiglu_absmax, gemm_dgrad, gemm_wgrad,
    gemm_backward,
    gemm_dgrad_mn, gemm_wgrad_mn, gemm_backward_mn, stream_copy, mx_quantize, mx_gemm_fwd,
    mx_swiglu_requant, mx_quantize_t, mx_quantize_both, mx_gemm_backward,
)
