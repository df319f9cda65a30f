// fp8_internal.hpp -- launchers behind the C ABI.  Arguments reaching these
// functions have already been validated by api.cpp; each launcher only
// enqueues kernels on `stream` and returns the launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>
#include <utility>

namespace fp8k {

// Enqueue kernel<<<grid, block, 0, stream>>>(args...) and return the status of
// this launch itself, so that an error left behind by unrelated earlier work
// (which hipGetLastError would report) is never taken for this call's.
template <typename... P, typename... A>
inline hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream, A&&... args)
{
    static_assert(sizeof...(P) == sizeof...(A), "one argument per kernel parameter");
    std::tuple<std::decay_t<P>...> vals(std::forward<A>(args)...);
    void* ptrs[sizeof...(P)];
    std::apply([&ptrs](auto&... v) {
        int i = 0;
        ((ptrs[i++] = static_cast<void*>(&v)), ...);
    }, vals);
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0, stream);
}

// Number of compute units of the current device (cached per device).
int device_cu_count();

// The SwiGLU s_g table (swiglu.hip): fp32 [2 signs][kSiluEHi - kSiluELo + 1 bf16
// exponents][128 mantissas], entry = s_g of the bf16 gate value with that sign,
// exponent and mantissa.  It is constant data of the code object (generated at
// build time); silu_table() returns its address on the current device.
constexpr int kSiluELo = 100;
constexpr int kSiluEHi = 133;
hipError_t silu_table(const float** table, hipStream_t stream);

hipError_t launch_absmax_bf16(const void* x, int64_t n, float* absmax, bool accumulate, hipStream_t stream);

// Running absmax of up to kMaxAbsTensors tensors in one launch (no reset).
constexpr int kMaxAbsTensors = 8;
hipError_t launch_absmax_many(int count, const void* const* x, const int64_t* n, float* const* absmax,
                              hipStream_t stream);
// count fp32 statistics set to +0 (count <= 2^20).
hipError_t launch_absmax_clear(float* absmax, int64_t count, hipStream_t stream);

// Block-scaled GEMM out[P, Q] = bf16(sum_r dec(A) 2^ea dec(B) 2^eb) of K-major
// operands A [P, R], B [Q, R] (B in E4M3) with E8M0 scales stored step-major,
// [R / 128][P][4] and [R / 128][Q][4]; P, Q >= 256.
hipError_t launch_gemm_mx(const uint8_t* A, const uint8_t* sa, int fmt_a, const uint8_t* B, const uint8_t* sb,
                          int fmt_b, void* out, int64_t P, int64_t Q, int64_t R, hipStream_t stream);

// Two independent block-scaled products in one launch (the dgrad and wgrad
// products of a linear, A in format fmt_a, B in E4M3), both outputs stored
// non-temporally; each problem as launch_gemm_mx.
hipError_t launch_gemm_mx_pair(const uint8_t* A0, const uint8_t* sa0, const uint8_t* B0, const uint8_t* sb0,
                               void* out0, int64_t P0, int64_t Q0, int64_t R0, const uint8_t* A1,
                               const uint8_t* sa1, const uint8_t* B1, const uint8_t* sb1, void* out1, int64_t P1,
                               int64_t Q1, int64_t R1, int fmt_a, hipStream_t stream);

// Transposed block (MX) quantisation: qt [cols, rows] = the codes of x^T with
// blocks of 32 along qt's rows (32 consecutive rows of a column of x), scales
// step-major [rows / 128][cols][4]; rows and cols multiples of 128.
hipError_t launch_mx_quantize_t(const void* x, int64_t rows, int64_t cols, int fmt, uint8_t* qt, uint8_t* scales,
                                hipStream_t stream);

// Both block quantisations of x in one read: q [rows, cols] (blocks along rows,
// scales sq [cols / 128][rows][4]) and qt [cols, rows] (blocks along columns,
// scales sqt [rows / 128][cols][4]); rows, cols multiples of 128.
hipError_t launch_mx_quantize_both(const void* x, int64_t rows, int64_t cols, int fmt, uint8_t* q, uint8_t* sq,
                                   uint8_t* qt, uint8_t* sqt, hipStream_t stream);

// The SwiGLU output of gu = [gate | up] ([M, 2F] bf16, F a multiple of 128),
// block (MX) quantised along F: E4M3 codes hq[M, F], scales step-major
// [F / 128][M][4].
hipError_t launch_mx_swiglu(const void* gu, int64_t M, int64_t F, uint8_t* hq, uint8_t* scales, hipStream_t stream);

// Block (MX) quantisation of a bf16 [rows, cols] tensor (cols a multiple of 128):
// codes q[rows, cols] and one E8M0 scale per 32 consecutive elements of a row,
// stored step-major: the scale of block b of row i at ((b / 4) rows + i) 4 + b % 4.
hipError_t launch_mx_quantize(const void* x, int64_t rows, int64_t cols, int fmt, uint8_t* q, uint8_t* scales,
                              hipStream_t stream);

hipError_t launch_quantize(const void* x, int64_t rows, int64_t cols, int fmt, const float* absmax,
                           uint8_t* q, uint8_t* qt, float* scale, float* inv_scale,
                           hipStream_t stream);

// Quantisation of up to kMaxQuantTensors tensors in one launch (the tile form,
// q and / or qt per tensor); the arrays are host arrays of count entries.
// qt_later (may be null): per tensor, nonzero when its qt is read later rather
// than by the next call, so it is stored non-temporally.
constexpr int kMaxQuantTensors = 8;
hipError_t launch_quantize_many(int count, const void* const* x, const int64_t* rows, const int64_t* cols,
                                const int* fmt, const float* const* absmax, uint8_t* const* q, uint8_t* const* qt,
                                float* const* scale, float* const* inv_scale, const int* qt_later,
                                hipStream_t stream);

hipError_t launch_swiglu_requant(const void* gu, int64_t M, int64_t F, float* absmax_h,
                                 int compute_absmax, uint8_t* hq, uint8_t* hqt,
                                 float* inv_scale_h, hipStream_t stream);

// SwiGLU backward: absmax of [dg | du], then its quantisation q [M, 2F] and / or qt [2F, M].
hipError_t launch_swiglu_backward(const void* gu, const void* dh, int64_t M, int64_t F, int fmt, float* absmax,
                                  uint8_t* q, uint8_t* qt, float* scale, float* inv_scale, hipStream_t stream);

// out[P, Q] = bf16(RN32(sum_r A[p, r] B[q, r] * RN32(*inv_a * *inv_b))).  Operand
// layouts: 0 = K-major (A[p, r] at A + p R + r), 1 = MN-major (A[p, r] at
// A + r P + p; B likewise with Q).  Compiled pairs (A, B): (0, 0), (0, 1), (1, 1).
// nt_out: the output is written with non-temporal stores (the backward products:
// their dX and dW then do not displace the operand panels the launch re-reads).
hipError_t launch_gemm_tn(const uint8_t* A, int fmt_a, int la, const uint8_t* B, int fmt_b, int lb,
                          const float* inv_a, const float* inv_b, void* out, int64_t P, int64_t Q, int64_t R,
                          bool nt_out, hipStream_t stream);

// Gate/up forward product with the SwiGLU statistic: out[M, 2F] = A[M, K] . B[2F, K]^T
// as launch_gemm_tn (e4m3 x e4m3, K-major), and *absmax_h = max(*absmax_h, max |h|)
// over h = s_g(gate) * up of the bf16 outputs (bit-pattern max).  M >= 256, F % 128 == 0.
hipError_t launch_gemm_gate_up(const uint8_t* A, const uint8_t* B, const float* inv_a, const float* inv_b, void* out,
                               float* absmax_h, int64_t M, int64_t F, int64_t K, hipStream_t stream);

// Two independent products of the same operand formats (and the same B layout) in one
// launch: the dgrad and wgrad products of a linear, both stored non-temporally.
hipError_t launch_gemm_tn_pair(const uint8_t* A0, int la0, const uint8_t* B0, int lb0, const float* ia0,
                               const float* ib0, void* out0, int64_t P0, int64_t Q0, int64_t R0, const uint8_t* A1,
                               int la1, const uint8_t* B1, int lb1, const float* ia1, const float* ib1, void* out1,
                               int64_t P1, int64_t Q1, int64_t R1, int fmt_a, int fmt_b, hipStream_t stream);

// dst[0, bytes) = src[0, bytes): the streaming-copy reference (bytes % 16 == 0, both 16-byte aligned).
hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

}  // namespace fp8k
