// fp8_internal.hpp -- launchers behind the C ABI.  Arguments reaching these
// functions have already been validated by api.cpp; each launcher only
// enqueues kernels on `stream` and returns the launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8k {

// Number of compute units of the current device (cached per device).
int device_cu_count();

hipError_t launch_absmax_bf16(const void* x, int64_t n, float* absmax, hipStream_t stream);

hipError_t launch_quantize(const void* x, int64_t rows, int64_t cols, int fmt, const float* absmax,
                           uint8_t* q, uint8_t* qt, float* scale, float* inv_scale,
                           hipStream_t stream);

hipError_t launch_swiglu_requant(const void* gu, int64_t M, int64_t F, float* absmax_h,
                                 int compute_absmax, uint8_t* hq, uint8_t* hqt,
                                 float* inv_scale_h, hipStream_t stream);

// out[P, Q] = bf16(RN32(sum_r A[p, r] B[q, r] * RN32(*inv_a * *inv_b)))
hipError_t launch_gemm_tn(const uint8_t* A, int fmt_a, const uint8_t* B, int fmt_b,
                          const float* inv_a, const float* inv_b, void* out,
                          int64_t P, int64_t Q, int64_t R, hipStream_t stream);

}  // namespace fp8k
