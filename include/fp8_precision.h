/*
 * fp8_precision.h -- C ABI of the MI355X (gfx950) FP8 training hot path.
 *
 * The operations are those of an 8-bit training pipeline with dynamic,
 * per-tensor ("just-in-time") absmax scaling:
 *
 *   absmax -> scale = fp8_max / absmax -> round-to-nearest-even saturating
 *   quantisation to OCP E4M3 (activations, weights) or E5M2 (output
 *   gradients) -> FP8 GEMMs (forward, dgrad, wgrad) with fp32 accumulation and
 *   a per-tensor descale to bf16; plus the SwiGLU nonlinearity fused with its
 *   requantisation, reusing a retained absmax during recomputation.
 *
 * Sources: "LLMQ: Efficient Lower-Precision Pretraining for Consumer GPUs"
 * (paperlayer.ai summary of arXiv 2512.15306), sections 1, 3.1, 4 and 5 /
 * Figure 2; "FastML periodic report" (EU CORDIS), the item on FP8 training
 * without delayed scaling.  The bit formats are those of the OCP 8-bit
 * floating point specification (OFP8).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every pointer argument is a DEVICE pointer owned by the caller.  The
 *    library allocates no device memory for any call and keeps no reference
 *    after the call returns.  It never synchronises the host.  The SwiGLU
 *    tables (s_g and its derivative per bf16 gate value) are constant data
 *    of the library's code object, so every call, the first included, can be
 *    recorded under stream capture.
 *  - All work is enqueued on `stream` (0 = the null stream).  Inputs must stay
 *    valid until the stream reaches the work.
 *  - absmax, scale and inverse-scale values stay in device memory as fp32
 *    scalars; they are passed by pointer, never copied to the host.
 *  - bf16 tensors are raw 16-bit patterns, row-major; FP8 tensors are bytes,
 *    row-major, in the format named by the call.
 *  - Every tensor pointer must be 16-byte aligned.  fp32 scalar pointers must
 *    be 4-byte aligned.
 *  - Return value: FP8_OK, or an error code; on error nothing was enqueued
 *    (except FP8_ERR_HIP, reported after a launch failed).  Arguments are
 *    checked on the host before anything is launched.  fp8_last_error()
 *    gives a message for the calling thread's last failure.
 *  - Calls are thread-safe.  The device a pointer lives on must be the
 *    current HIP device.
 *  - NaN inputs give NaN codes (0x7F or 0xFF); which sign a NaN code carries
 *    is not specified.  Infinite inputs saturate to +-max.
 */
#ifndef FP8_PRECISION_H
#define FP8_PRECISION_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fp8_status {
    FP8_OK = 0,
    FP8_ERR_INVALID = 1,      /* null pointer, size <= 0, overlapping in/out, bad enum */
    FP8_ERR_UNSUPPORTED = 2,  /* misaligned pointer or a dimension outside the kernel's constraints */
    FP8_ERR_HIP = 3           /* the HIP runtime reported an error at launch */
} fp8_status;

/* OCP OFP8 formats.  E4M3: bias 7, no infinity, NaN S.1111.111, max 448.
 * E5M2: bias 15, infinity S.11111.00, max 57344. */
typedef enum fp8_fmt { FP8_E4M3 = 0, FP8_E5M2 = 1 } fp8_fmt;

/* Static text for a status code. */
const char* fp8_status_string(fp8_status s);

/* Detail message of the calling thread's most recent failed call ("" if none). */
const char* fp8_last_error(void);

/*
 * absmax of a bf16 tensor: *absmax = max over i < n of |x[i]| (fp32, exact).
 * This is the per-tensor statistic of dynamic tensor-level scaling (LLMQ
 * summary, section 1; FastML report: the scale is taken just in time from
 * the current tensor, not from a history).  A NaN anywhere gives a NaN, an
 * infinity gives +inf.  The result does not depend on launch order.
 *
 *   x       bf16 [n], 16-byte aligned
 *   n       number of elements, n >= 1
 *   absmax  one fp32 in device memory (written)
 */
fp8_status fp8_absmax(const void* x, int64_t n, float* absmax, hipStream_t stream);

/*
 * Running absmax: *absmax = max(*absmax, max over i < n of |x[i]|), the same
 * reduction as fp8_absmax without resetting the accumulator first, for a
 * statistic gathered over several calls (a tensor held in pieces) or a set of
 * statistics that the caller clears together once per step (one fill instead
 * of one per tensor).  The maximum is taken on the fp32 bit patterns, so the
 * NaN / infinity rules of fp8_absmax hold across calls; *absmax must start as
 * +0 or as an earlier result (its sign bit clear).  Calls that accumulate into
 * one location may run in any order or concurrently.
 *
 *   x       bf16 [n], 16-byte aligned
 *   n       number of elements, n >= 1
 *   absmax  one fp32 in device memory (read and updated)
 */
fp8_status fp8_absmax_accumulate(const void* x, int64_t n, float* absmax, hipStream_t stream);

/*
 * The running absmax of several tensors in one launch: for i < count,
 *   *absmax[i] = max(*absmax[i], max over j < n[i] of |x[i][j]|)
 * exactly as count calls of fp8_absmax_accumulate (the same statistic as
 * fp8_absmax, per tensor), but sharing the fixed cost of a launch -- for the
 * tensors that are ready together, such as a linear's input and weight
 * (LLMQ summary, section 1: every operand of an FP8 product gets its own
 * just-in-time statistic).
 *
 *   count      1 .. 8
 *   x, n       host arrays of count bf16 device pointers (16-byte aligned) and
 *              element counts (>= 1); read during the call
 *   absmax     host array of count device fp32 pointers (read and updated; each
 *              starts as +0 or an earlier result; two may be the same slot)
 */
fp8_status fp8_absmax_accumulate_many(int count, const void* const* x, const int64_t* n,
                                      float* const* absmax, hipStream_t stream);

/*
 * Sets count running statistics to +0, the start value of the running absmax
 * that fp8_absmax_accumulate and fp8_absmax_accumulate_many fold tensors into
 * (FastML report, FP8 training without delayed scaling: each scale comes from
 * the statistic of the current tensor, so a step's statistics start afresh
 * rather than carrying an amax history over).  One launch for a step's whole
 * set of statistics; stream-ordered like every other call.
 *
 *   absmax  fp32 [count] in device memory, 4-byte aligned (written)
 *   count   1 .. 2^20
 */
fp8_status fp8_absmax_clear(float* absmax, int64_t count, hipStream_t stream);

/*
 * Quantise a bf16 [rows, cols] tensor with the scale of its absmax:
 *   s      = fp8_max / absmax  (one fp32 division; 1 when absmax == 0; held at
 *            FLT_MAX if the division overflows)
 *   q[i,j] = encode_fmt(RN32(x[i,j] * s))   round to nearest even, saturating
 * and optionally its transposed copy qt[j,i] = q[i,j], the operand layout the
 * backward GEMMs read (LLMQ summary, section 4: backward-pass transposes and
 * the extra transpose/quantisation buffers of FP8).
 *
 *   x          bf16 [rows, cols]
 *   fmt        FP8_E4M3 or FP8_E5M2 (gradients: LLMQ summary, section 5 / Fig. 2)
 *   absmax     fp32 scalar: fresh from fp8_absmax or a retained statistic
 *   q          u8 [rows, cols] or NULL
 *   qt         u8 [cols, rows] or NULL (at least one of q, qt)
 *   scale      fp32 scalar out (s) or NULL
 *   inv_scale  fp32 scalar out (RN32(1 / s)), the GEMM descale factor, or NULL
 * Constraints: cols % 16 == 0; if qt is given, rows % 16 == 0 as well.
 */
fp8_status fp8_quantize(const void* x, int64_t rows, int64_t cols, fp8_fmt fmt,
                        const float* absmax, uint8_t* q, uint8_t* qt,
                        float* scale, float* inv_scale, hipStream_t stream);

/*
 * Several quantisations in one launch: for i < count, exactly the bytes of
 *   fp8_quantize(x[i], rows[i], cols[i], fmt[i], absmax[i], q[i], qt[i],
 *                scale[i], inv_scale[i], stream)
 * (same scale, codes and transposed copy), with the fixed cost of a launch
 * paid once -- for tensors that are ready together, such as the weights of a
 * layer and its input at the start of a step (LLMQ summary, section 1: every
 * operand gets its own just-in-time scale; section 4: the quantisation passes
 * and transposes are overhead of FP8 training).
 *
 *   count              1 .. 8
 *   x, rows, cols, fmt, absmax, q, qt, scale, inv_scale
 *                      host arrays of count entries, read during the call: the
 *                      device pointers and sizes of each tensor, as for
 *                      fp8_quantize (q[i] or qt[i] may be NULL, not both;
 *                      scale[i] and inv_scale[i] may be NULL)
 *   qt_later           host array of count entries, or NULL (all 0): nonzero
 *                      when tensor i's qt is read later -- in the forward pass,
 *                      the copies the backward products use -- rather than by
 *                      the next call; such a qt is written with non-temporal
 *                      stores, leaving the Infinity Cache to q, which the next
 *                      GEMM reads (the bytes are the same either way; tensors
 *                      of the two kinds go to separate launches)
 * Constraints: every rows[i] and cols[i] a multiple of 16.  Inputs (x, absmax)
 * may be shared between entries; no output may overlap an input or another
 * output.
 */
fp8_status fp8_quantize_many(int count, const void* const* x, const int64_t* rows, const int64_t* cols,
                             const fp8_fmt* fmt, const float* const* absmax, uint8_t* const* q,
                             uint8_t* const* qt, float* const* scale, float* const* inv_scale,
                             const int* qt_later, hipStream_t stream);

/*
 * SwiGLU fused with its E4M3 requantisation.  gu = [gate | up] is the bf16
 * [M, 2F] output of the gate/up GEMM; for i < M, j < F
 *   g = gu[i, j], u = gu[i, F + j]
 *   h = RN32(RN32(g / RN32(1 + RN32(e^-g))) * u)       (silu(g) * u, fp32)
 *   hq[i, j] = encode_e4m3(RN32(h * s_h)),  s_h = 448 / absmax_h
 * compute_absmax = 1 (forward): absmax_h = max |h| is computed and written.
 * compute_absmax = 2 (forward, running statistic): as 1 without resetting
 *   *absmax_h first: it becomes max(*absmax_h, max |h|) (bit-pattern max; the
 *   caller clears it, e.g. with the other statistics of a step -- see
 *   fp8_absmax_accumulate), and quantisation uses that value.
 * compute_absmax = 0 (recomputation): *absmax_h is the retained statistic and
 * is only read; no global reduction runs, and the bytes equal the forward's
 * for the same gu (LLMQ summary, section 3.1: the forward's statistic is
 * reused, so the recomputed SwiGLU output is requantised in the pass that
 * evaluates it and the tensor is never reduced a second time).
 *
 *   gu           bf16 [M, 2F]
 *   absmax_h     fp32 scalar (written when compute_absmax = 1, updated when 2, read when 0)
 *   hq           u8 [M, F] or NULL
 *   hqt          u8 [F, M] (transpose of hq) or NULL (at least one of hq, hqt)
 *   inv_scale_h  fp32 scalar out (RN32(1 / s_h)) or NULL
 * Constraints: F % 16 == 0; if hqt is given, M % 16 == 0.
 * Cache policy (same bytes either way): in the forward forms (compute_absmax
 * 1 or 2) hqt is written with non-temporal stores -- the backward pass reads
 * it, not the down projection's forward GEMM that reads hq next; in the
 * recomputation form (0) the backward product that follows reads hqt, and it
 * is written with ordinary stores.
 */
fp8_status fp8_swiglu_requant(const void* gu, int64_t M, int64_t F, float* absmax_h,
                              int compute_absmax, uint8_t* hq, uint8_t* hqt,
                              float* inv_scale_h, hipStream_t stream);

/*
 * SwiGLU backward fused with the quantisation of its output: the gradient of
 * gu = [gate | up] given dh, the gradient of h = silu(g) * u, is formed and
 * quantised for the gate/up backward GEMMs (the step downstream of the
 * requantised SwiGLU of the LLMQ summary, section 3.1; E5M2 gradients,
 * section 5 / Fig. 2).  For i < M, j < F, with g = gu[i, j], u = gu[i, F + j],
 * d = dh[i, j] and every step one fp32 operation:
 *   E = RN32(e^-g), t = 1 + E, sig = 1 / t, s = g / t            (silu(g))
 *   ds = sig * (1 + g * (1 - sig))                                 (silu'(g), in that order)
 *   du = d * s,  dg = (d * u) * ds
 *   dgu = [dg | du] (fp32 [M, 2F], never stored)
 *   *absmax = max |dgu| (fresh, as for any gradient), s_q = fp8_max / absmax
 *   q[i, c] = encode_fmt(RN32(dgu[i, c] * s_q)),  qt[c, i] = q[i, c]
 *
 *   gu         bf16 [M, 2F] (the forward's or the recomputed gate/up output)
 *   dh         bf16 [M, F]
 *   fmt        FP8_E5M2 (gradients) or FP8_E4M3
 *   absmax     fp32 scalar out
 *   q          u8 [M, 2F] or NULL;  qt  u8 [2F, M] or NULL (at least one) -- the
 *              operands of fp8_gemm_dgrad (q) and fp8_gemm_wgrad (qt) of gate/up
 *   scale, inv_scale  fp32 scalars out, each may be NULL
 * Constraints: F % 16 == 0; if qt is given, M % 16 == 0.  gu and dh may alias;
 * no output may overlap another buffer.
 */
fp8_status fp8_swiglu_backward(const void* gu, const void* dh, int64_t M, int64_t F, fp8_fmt fmt,
                               float* absmax, uint8_t* q, uint8_t* qt, float* scale, float* inv_scale,
                               hipStream_t stream);

/*
 * FP8 GEMMs with fp32 accumulation and per-tensor descale (LLMQ summary,
 * section 2: low-precision matrix products on the matrix units; section 4:
 * large models are dominated by these products).  Every call computes
 *   out[p, q] = bf16_RNE( RN32( (sum over r of dec(A[p, r]) * dec(B[q, r]))
 *                               * RN32(inv_a * inv_b) ) )
 * with both operands contiguous along the reduction index r, fp32
 * accumulation (each FP8 product is exact in fp32) and the output written
 * (never accumulated into).  The order of the fp32 sum is not specified, but
 * a given shape always produces the same bytes (no atomics).
 *
 * fp8_gemm_fwd:   Y[M, N]  = X[M, K] . W[N, K]^T      A = xq  (e4m3) [M, K], B = wq  (e4m3) [N, K]
 * fp8_gemm_dgrad: dX[M, K] = dY[M, N] . W[N, K]       A = dyq (dy_fmt) [M, N], B = wqt (e4m3) [K, N]
 * fp8_gemm_wgrad: dW[N, K] = dY[M, N]^T . X[M, K]     A = dyqt (dy_fmt) [N, M], B = xqt (e4m3) [K, M]
 *
 *   inv_*   fp32 scalars: the inverse scales written by fp8_quantize /
 *           fp8_swiglu_requant for the two operands
 *   dy_fmt  FP8_E5M2 (default reading of the pages) or FP8_E4M3
 * Constraints: every dimension >= 16 and a multiple of 16; the reduction
 * length (K, N and M respectively) a multiple of 128; each FP8 operand smaller
 * than 2^31 bytes and each output dimension below 2^30 (operand offsets are
 * 32-bit); anything else returns FP8_ERR_UNSUPPORTED.
 * Cache policy of the output (bytes and results are the same either way):
 * fp8_gemm_fwd writes Y with ordinary stores, so the statistic or SwiGLU pass
 * that reads it next finds it in the 256 MiB Infinity Cache -- unless Y is
 * 256 MiB or more while X and W together are at most 256 MiB, when Y is stored
 * non-temporally (it could not stay cached, and would push out the operands);
 * every backward product (dgrad, wgrad, and the pair and MN-major forms below)
 * stores dX / dW non-temporally, so the outputs do not displace the operand
 * panels that the rest of the launch re-reads.
 */
fp8_status fp8_gemm_fwd(const uint8_t* xq, const uint8_t* wq, const float* inv_sx,
                        const float* inv_sw, void* y, int64_t M, int64_t N, int64_t K,
                        hipStream_t stream);
fp8_status fp8_gemm_dgrad(const uint8_t* dyq, fp8_fmt dy_fmt, const uint8_t* wqt,
                          const float* inv_sdy, const float* inv_sw, void* dx,
                          int64_t M, int64_t N, int64_t K, hipStream_t stream);
fp8_status fp8_gemm_wgrad(const uint8_t* dyqt, fp8_fmt dy_fmt, const uint8_t* xqt,
                          const float* inv_sdy, const float* inv_sx, void* dw,
                          int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * The gate/up forward GEMM with the SwiGLU statistic taken in its epilogue
 * (LLMQ summary, section 3.1: the forward produces the absmax of the SwiGLU
 * output that quantisation -- and, later, recomputation -- uses; computing it
 * where [gate | up] is produced saves the separate read pass over that
 * tensor):
 *   gu[M, 2F] = X[M, K] . Wgu[2F, K]^T   exactly as fp8_gemm_fwd (same bytes)
 *   *absmax_h = max(*absmax_h, max over m, j of |h[m, j]|),
 *   h[m, j]   = RN32(s_g(gu[m, j]) * gu[m, F + j])  on the bf16 values of gu,
 * with s_g and the NaN / infinity rules of fp8_swiglu_requant, so the result
 * equals that call's computed absmax_h on this gu.  Like fp8_absmax_accumulate,
 * absmax_h is read and updated: it must start as +0 (or an earlier result);
 * fp8_swiglu_requant then runs with compute_absmax = 0 on it.
 *
 *   xq   e4m3 [M, K],  wq  e4m3 [2F, K]: gate rows 0 .. F-1, up rows F .. 2F-1
 *   inv_sx, inv_sw   fp32 inverse scales of the operands
 *   gu   bf16 [M, 2F] (written),  absmax_h  one fp32 (read and updated)
 * Constraints: those of fp8_gemm_fwd with N = 2F, plus F % 128 == 0 and
 * M >= 256.  No buffer may overlap gu or absmax_h.
 */
fp8_status fp8_gemm_fwd_swiglu_absmax(const uint8_t* xq, const uint8_t* wq, const float* inv_sx,
                                      const float* inv_sw, void* gu, float* absmax_h, int64_t M,
                                      int64_t F, int64_t K, hipStream_t stream);

/*
 * Both backward products of one linear in a single launch: dgrad
 * dX[M, K] = dY[M, N] . W[N, K] and wgrad dW[N, K] = dY[M, N]^T . X[M, K] are
 * independent, so one persistent launch runs both tile sets, longest
 * reduction first (LLMQ summary, section 4: the backward pass and its
 * transposed operands; large models are dominated by these products).  The
 * operands are those of fp8_gemm_dgrad (dyq, wqt) and fp8_gemm_wgrad (dyqt,
 * xqt) and both outputs are bit-identical to those two calls; the launch
 * pays the per-launch costs (first-stage fill, last-round epilogue) once.
 *
 *   dyq [M, N], dyqt [N, M]  (dy_fmt);  wqt [K, N], xqt [K, M]  (e4m3)
 *   dx  bf16 [M, K],  dw bf16 [N, K]  (must not overlap each other or any input)
 * Constraints: those of fp8_gemm_dgrad and fp8_gemm_wgrad.
 */
fp8_status fp8_gemm_backward(const uint8_t* dyq, const uint8_t* dyqt, fp8_fmt dy_fmt,
                             const uint8_t* wqt, const uint8_t* xqt,
                             const float* inv_sdy, const float* inv_sw, const float* inv_sx,
                             void* dx, void* dw, int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * The backward products on the untransposed FP8 tensors: the operands the
 * transposed copies would hold are read in their stored layout instead
 * (row-major along the product's output index, "MN-major"), staged through
 * LDS and fed to the matrix instructions with gfx950's transposing LDS reads.
 * The quantise and SwiGLU calls then need no qt / hqt outputs for the
 * backward pass (LLMQ summary, section 4: backward-pass transposes and the
 * extra transpose/quantisation buffers are overhead of FP8 training).  The
 * results are bit-identical to fp8_gemm_dgrad / fp8_gemm_wgrad /
 * fp8_gemm_backward on the transposed copies.
 *
 * fp8_gemm_dgrad_mn:  dX[M, K] = dY[M, N] . W[N, K]      dyq (dy_fmt) [M, N], wq (e4m3) [N, K]
 * fp8_gemm_wgrad_mn:  dW[N, K] = dY[M, N]^T . X[M, K]    dyq (dy_fmt) [M, N], xq (e4m3) [M, K]
 * fp8_gemm_backward_mn: both, in one launch (outputs must not overlap each
 *                     other or any input)
 *
 *   inv_*   fp32 scalars as for the calls above
 * Constraints: those of fp8_gemm_dgrad / fp8_gemm_wgrad (every dimension a
 * multiple of 16 and >= 16; the reduction length, N for dgrad and M for
 * wgrad, a multiple of 128).
 */
fp8_status fp8_gemm_dgrad_mn(const uint8_t* dyq, fp8_fmt dy_fmt, const uint8_t* wq,
                             const float* inv_sdy, const float* inv_sw, void* dx,
                             int64_t M, int64_t N, int64_t K, hipStream_t stream);
fp8_status fp8_gemm_wgrad_mn(const uint8_t* dyq, fp8_fmt dy_fmt, const uint8_t* xq,
                             const float* inv_sdy, const float* inv_sx, void* dw,
                             int64_t M, int64_t N, int64_t K, hipStream_t stream);
fp8_status fp8_gemm_backward_mn(const uint8_t* dyq, fp8_fmt dy_fmt, const uint8_t* wq, const uint8_t* xq,
                                const float* inv_sdy, const float* inv_sw, const float* inv_sx,
                                void* dx, void* dw, int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * Block (MX) scaling -- the alternative to one scale per tensor that the LLMQ
 * summary (section 2) says needs native hardware support (gfx950 has
 * block-scaled matrix instructions).  The pages define no format; these calls
 * follow the OCP Microscaling (MX) formats specification v1.0 (section 6.3).
 *
 * fp8_mx_quantize: every 32 consecutive elements of a row of the bf16
 * [rows, cols] tensor x share one scale 2^e,
 *   e = floor(log2(max |x| over the block)) - emax   (emax = 8 for E4M3, 15 for E5M2)
 * clamped to [-127, 127] (-127 for an all-zero block), and
 *   q[i, j]           = encode_fmt(x[i, j] * 2^-e)   (exact product; nearest even, saturating)
 *   scales[i, j / 32] = e + 127                      (an E8M0 byte)
 * A block holding a NaN or an infinity gets scales = 255 (NaN) and the unscaled
 * encodings.  One pass: no statistic call comes first.
 *
 *   x       bf16 [rows, cols], 16-byte aligned
 *   fmt     FP8_E4M3 or FP8_E5M2
 *   q       u8 [rows, cols], 16-byte aligned
 *   scales  u8, rows * cols / 32 bytes, stored step-major as [cols / 128][rows][4]:
 *           the scale of block b (elements 32 b .. 32 b + 31) of row i is at
 *           ((b / 4) * rows + i) * 4 + b % 4, so the four scales of one
 *           128-element reduction step of every row lie together, in the order
 *           fp8_mx_gemm_fwd reads them
 * Constraints: cols % 128 == 0 and rows * cols / 32 < 2^32 (else
 * FP8_ERR_UNSUPPORTED); buffers must not overlap.
 */
fp8_status fp8_mx_quantize(const void* x, int64_t rows, int64_t cols, fp8_fmt fmt, uint8_t* q,
                           uint8_t* scales, hipStream_t stream);

/*
 * fp8_mx_quantize_t: the block (MX) quantisation of x^T, for a backward
 * product whose reduction runs over x's rows (dgrad reads W^T with blocks
 * along N, wgrad reads dY^T and X^T with blocks along M).  The blocks must lie
 * along the reduction, so this is a second quantisation of x (its own scales),
 * not a transpose of fp8_mx_quantize's codes:
 *   qt[j, i] = encode_fmt(x[i, j] * 2^-e), blocks of 32 consecutive i for one j
 *   scales: block b of qt row j at ((b / 4) * cols + j) * 4 + b % 4  ([rows / 128][cols][4])
 * with the rule of fp8_mx_quantize for e, saturation and non-finite blocks.
 *
 *   x       bf16 [rows, cols], 16-byte aligned
 *   fmt     FP8_E4M3 or FP8_E5M2
 *   qt      u8 [cols, rows], 16-byte aligned
 *   scales  u8, rows * cols / 32 bytes, 4-byte aligned
 * Constraints: rows % 128 == 0 and cols % 128 == 0 (else FP8_ERR_UNSUPPORTED);
 * buffers must not overlap.
 */
fp8_status fp8_mx_quantize_t(const void* x, int64_t rows, int64_t cols, fp8_fmt fmt, uint8_t* qt,
                             uint8_t* scales, hipStream_t stream);

/*
 * fp8_mx_quantize_both: fp8_mx_quantize and fp8_mx_quantize_t of the same x
 * from one read of it -- the forward operand (blocks along rows) and the
 * backward operand (blocks along columns, of x^T), each with its own scales;
 * the bytes of the two calls.
 *
 *   x        bf16 [rows, cols], 16-byte aligned
 *   q, sq    u8 [rows, cols] (16-byte aligned) and [cols / 128][rows][4] (4-byte aligned)
 *   qt, sqt  u8 [cols, rows] (16-byte aligned) and [rows / 128][cols][4] (4-byte aligned)
 * Constraints: rows % 128 == 0 and cols % 128 == 0 (else FP8_ERR_UNSUPPORTED);
 * buffers must not overlap.
 */
fp8_status fp8_mx_quantize_both(const void* x, int64_t rows, int64_t cols, fp8_fmt fmt, uint8_t* q,
                                uint8_t* sq, uint8_t* qt, uint8_t* sqt, hipStream_t stream);

/*
 * fp8_mx_swiglu_requant: the SwiGLU output h = silu(g) * u of gu = [gate | up]
 * (each element exactly as fp8_swiglu_requant evaluates it, never rounded to
 * bf16), block-quantised to E4M3 along the feature axis by the rule of
 * fp8_mx_quantize (the block maximum over the 32 fp32 values of h).  One pass:
 * a block's maximum is local, so no statistic pass over [gate | up] comes first
 * (LLMQ summary, section 3.1: the per-tensor form needs the retained statistic).
 *
 *   gu      bf16 [M, 2F], 16-byte aligned
 *   hq      u8 [M, F] E4M3 codes, 16-byte aligned
 *   scales  u8, M * F / 32 bytes, step-major [F / 128][M][4] as for fp8_mx_quantize
 * Constraints: F % 128 == 0 (else FP8_ERR_UNSUPPORTED); buffers must not overlap.
 */
fp8_status fp8_mx_swiglu_requant(const void* gu, int64_t M, int64_t F, uint8_t* hq, uint8_t* scales,
                                 hipStream_t stream);

/*
 * fp8_mx_gemm_fwd: the forward product of block-scaled operands,
 *   Y[m, n] = bf16_RNE( RN32( sum_k dec(X[m, k]) 2^ex(m, k / 32) dec(W[n, k]) 2^ew(n, k / 32) ) )
 * with fp32 accumulation and no per-tensor factor (each 2^e is the E8M0 scale
 * of the 32-element block holding the code; a NaN scale gives NaN).  The
 * block scales are applied by the matrix instruction itself.
 *
 *   xq, sx   codes [M, K] (x_fmt: FP8_E4M3 or FP8_E5M2) and scales [K / 128][M][4]
 *            from fp8_mx_quantize of X
 *   wq, sw   codes [N, K] (E4M3) and scales [K / 128][N][4] from fp8_mx_quantize of W
 *   y        bf16 [M, N]
 * Constraints: those of fp8_gemm_fwd, and M >= 256, N >= 256; scales 4-byte
 * aligned; y may not overlap any input.
 */
fp8_status fp8_mx_gemm_fwd(const uint8_t* xq, const uint8_t* sx, fp8_fmt x_fmt, const uint8_t* wq,
                           const uint8_t* sw, void* y, int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * fp8_mx_gemm_backward: both backward products of a linear on block-scaled
 * operands, in one launch (as fp8_gemm_backward does for per-tensor scales):
 *   dX[m, k] = bf16_RNE( RN32( sum_n dec(dY[m, n]) 2^e(dY; m, n / 32) dec(W[n, k]) 2^e(W^T; k, n / 32) ) )
 *   dW[n, k] = bf16_RNE( RN32( sum_m dec(dY[m, n]) 2^e(dY^T; n, m / 32) dec(X[m, k]) 2^e(X^T; k, m / 32) ) )
 * each block along its product's reduction (LLMQ summary, section 4: the
 * backward pass needs its operands along the other dimension; the MX block
 * rule of fp8_mx_quantize).  Each output equals what fp8_mx_gemm_fwd computes
 * from the same operands, bit for bit; dX and dW are written with
 * non-temporal stores.
 *
 *   dyq, sdy    codes [M, N] (dy_fmt) and scales [N / 128][M][4]: fp8_mx_quantize of dY
 *   dyqt, sdyt  codes [N, M] (dy_fmt) and scales [M / 128][N][4]: fp8_mx_quantize_t of dY
 *   wqt, swt    codes [K, N] (E4M3) and scales [N / 128][K][4]: fp8_mx_quantize_t of W [N, K]
 *   xqt, sxt    codes [K, M] (E4M3) and scales [M / 128][K][4]: fp8_mx_quantize_t of X [M, K]
 *   dx          bf16 [M, K];  dw  bf16 [N, K]
 * Constraints: M, N, K >= 256, M and N multiples of 128, K a multiple of 16
 * (else FP8_ERR_UNSUPPORTED); codes and outputs 16-byte aligned, scales 4-byte
 * aligned; dx and dw overlap neither each other nor any input (else
 * FP8_ERR_INVALID).
 */
fp8_status fp8_mx_gemm_backward(const uint8_t* dyq, const uint8_t* sdy, const uint8_t* dyqt, const uint8_t* sdyt,
                                fp8_fmt dy_fmt, const uint8_t* wqt, const uint8_t* swt, const uint8_t* xqt,
                                const uint8_t* sxt, void* dx, void* dw, int64_t M, int64_t N, int64_t K,
                                hipStream_t stream);

/*
 * Measurement reference, not a step of the FP8 method: a plain device copy
 * dst[0, bytes) = src[0, bytes), built like the streaming kernels above
 * (16-byte vectors, non-temporal loads, the launch shape at which a copy
 * reaches its highest measured rate on this chip).  The bandwidth of the
 * statistic and quantisation calls is reported as a fraction of what this
 * copy reaches on the same machine.
 *
 *   src, dst  device buffers of `bytes` bytes, 16-byte aligned, not overlapping
 *   bytes     > 0 and a multiple of 16 (else FP8_ERR_INVALID / FP8_ERR_UNSUPPORTED)
 */
fp8_status fp8_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* FP8_PRECISION_H */
