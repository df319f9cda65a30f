// api.cpp -- the C ABI of the FP8 hot path: argument checks, then launches.
//
// Every entry point validates its arguments on the host before enqueuing
// anything; see include/fp8_precision.h for the contract of each call.
#include "fp8_precision.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "fp8_internal.hpp"

namespace {

thread_local std::string t_last_error;

fp8_status fail(fp8_status st, const char* what)
{
    t_last_error = what;
    return st;
}

fp8_status fail(fp8_status st, const std::string& what)
{
    t_last_error = what;
    return st;
}

fp8_status fail_hip(const char* call, hipError_t e)
{
    char buf[256];
    std::snprintf(buf, sizeof(buf), "%s: HIP error %d (%s)", call, (int)e, hipGetErrorString(e));
    t_last_error = buf;
    return FP8_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte ranges [p, p + n) and [q, q + m) overlap.
bool overlap(const void* p, int64_t n, const void* q, int64_t m)
{
    if (!p || !q || n <= 0 || m <= 0) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + (uintptr_t)m && b < a + (uintptr_t)n;
}

struct Range {
    const void* p;
    int64_t n;
};

// True if any two of the ranges overlap.
template <int N>
bool any_overlap(const Range (&r)[N])
{
    for (int i = 0; i < N; ++i)
        for (int j = i + 1; j < N; ++j)
            if (overlap(r[i].p, r[i].n, r[j].p, r[j].n)) return true;
    return false;
}

bool mul_ok(int64_t a, int64_t b, int64_t limit) { return a > 0 && b > 0 && a <= limit / b; }

constexpr int64_t kMaxElems = (int64_t)1 << 40;

}  // namespace

namespace fp8k {

int device_cu_count()
{
    static std::mutex mu;
    static int cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lk(mu);
    if (cache[dev] == 0) {
        int cu = 0;
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
            cu = 256;
        cache[dev] = cu;
    }
    return cache[dev];
}

}  // namespace fp8k

extern "C" {

const char* fp8_status_string(fp8_status s)
{
    switch (s) {
    case FP8_OK: return "ok";
    case FP8_ERR_INVALID: return "invalid argument";
    case FP8_ERR_UNSUPPORTED: return "unsupported argument (alignment or shape constraint)";
    case FP8_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* fp8_last_error(void) { return t_last_error.c_str(); }

static fp8_status absmax_common(const char* name, const void* x, int64_t n, float* absmax, bool accumulate,
                                hipStream_t stream)
{
    t_last_error.clear();
    const std::string f(name);
    if (!x || !absmax) return fail(FP8_ERR_INVALID, f + ": null pointer");
    if (n <= 0 || n > kMaxElems) return fail(FP8_ERR_INVALID, f + ": n must be in [1, 2^40]");
    if (overlap(x, 2 * n, absmax, 4)) return fail(FP8_ERR_INVALID, f + ": absmax overlaps x");
    if (!aligned(x, 16) || !aligned(absmax, 4))
        return fail(FP8_ERR_UNSUPPORTED, f + ": x must be 16-byte and absmax 4-byte aligned");
    hipError_t e = fp8k::launch_absmax_bf16(x, n, absmax, accumulate, stream);
    if (e != hipSuccess) return fail_hip(name, e);
    return FP8_OK;
}

fp8_status fp8_absmax(const void* x, int64_t n, float* absmax, hipStream_t stream)
{
    return absmax_common("fp8_absmax", x, n, absmax, false, stream);
}

fp8_status fp8_absmax_accumulate(const void* x, int64_t n, float* absmax, hipStream_t stream)
{
    return absmax_common("fp8_absmax_accumulate", x, n, absmax, true, stream);
}

fp8_status fp8_absmax_accumulate_many(int count, const void* const* x, const int64_t* n, float* const* absmax,
                                      hipStream_t stream)
{
    t_last_error.clear();
    const char* name = "fp8_absmax_accumulate_many";
    if (!x || !n || !absmax) return fail(FP8_ERR_INVALID, "fp8_absmax_accumulate_many: null array");
    if (count < 1 || count > fp8k::kMaxAbsTensors)
        return fail(FP8_ERR_INVALID, "fp8_absmax_accumulate_many: count must be in [1, 8]");
    for (int i = 0; i < count; ++i) {
        if (!x[i] || !absmax[i]) return fail(FP8_ERR_INVALID, "fp8_absmax_accumulate_many: null pointer");
        if (n[i] <= 0 || n[i] > kMaxElems)
            return fail(FP8_ERR_INVALID, "fp8_absmax_accumulate_many: every n must be in [1, 2^40]");
        if (!aligned(x[i], 16) || !aligned(absmax[i], 4))
            return fail(FP8_ERR_UNSUPPORTED, "fp8_absmax_accumulate_many: x 16-byte and absmax 4-byte aligned");
    }
    // an accumulator may be shared (the max is order-free), but none may lie inside an input
    for (int i = 0; i < count; ++i)
        for (int j = 0; j < count; ++j)
            if (overlap(x[j], 2 * n[j], absmax[i], 4))
                return fail(FP8_ERR_INVALID, "fp8_absmax_accumulate_many: an absmax overlaps an input");
    hipError_t e = fp8k::launch_absmax_many(count, x, n, absmax, stream);
    if (e != hipSuccess) return fail_hip(name, e);
    return FP8_OK;
}

fp8_status fp8_absmax_clear(float* absmax, int64_t count, hipStream_t stream)
{
    t_last_error.clear();
    if (!absmax) return fail(FP8_ERR_INVALID, "fp8_absmax_clear: null pointer");
    if (count < 1 || count > ((int64_t)1 << 20)) return fail(FP8_ERR_INVALID, "fp8_absmax_clear: count must be in [1, 2^20]");
    if (!aligned(absmax, 4)) return fail(FP8_ERR_UNSUPPORTED, "fp8_absmax_clear: absmax must be 4-byte aligned");
    hipError_t e = fp8k::launch_absmax_clear(absmax, count, stream);
    if (e != hipSuccess) return fail_hip("fp8_absmax_clear", e);
    return FP8_OK;
}

fp8_status fp8_quantize(const void* x, int64_t rows, int64_t cols, fp8_fmt fmt, const float* absmax,
                        uint8_t* q, uint8_t* qt, float* scale, float* inv_scale, hipStream_t stream)
{
    t_last_error.clear();
    if (!x || !absmax) return fail(FP8_ERR_INVALID, "fp8_quantize: null x or absmax");
    if (!q && !qt) return fail(FP8_ERR_INVALID, "fp8_quantize: at least one of q, qt is required");
    if (fmt != FP8_E4M3 && fmt != FP8_E5M2) return fail(FP8_ERR_INVALID, "fp8_quantize: bad format");
    if (!mul_ok(rows, cols, kMaxElems)) return fail(FP8_ERR_INVALID, "fp8_quantize: bad shape");
    const int64_t n = rows * cols;
    const Range r[] = {{x, 2 * n}, {absmax, 4}, {q, q ? n : 0}, {qt, qt ? n : 0},
                       {scale, scale ? 4 : 0}, {inv_scale, inv_scale ? 4 : 0}};
    if (any_overlap(r)) return fail(FP8_ERR_INVALID, "fp8_quantize: overlapping buffers");
    if (cols % 16) return fail(FP8_ERR_UNSUPPORTED, "fp8_quantize: cols must be a multiple of 16");
    if (qt && rows % 16) return fail(FP8_ERR_UNSUPPORTED, "fp8_quantize: rows must be a multiple of 16 with qt");
    if (qt && (rows + 127) / 128 > 65535) return fail(FP8_ERR_UNSUPPORTED, "fp8_quantize: too many rows for qt");
    if (!aligned(x, 16) || (q && !aligned(q, 16)) || (qt && !aligned(qt, 16)) || !aligned(absmax, 4) ||
        (scale && !aligned(scale, 4)) || (inv_scale && !aligned(inv_scale, 4)))
        return fail(FP8_ERR_UNSUPPORTED, "fp8_quantize: misaligned pointer");
    hipError_t e = fp8k::launch_quantize(x, rows, cols, (int)fmt, absmax, q, qt, scale, inv_scale, stream);
    if (e != hipSuccess) return fail_hip("fp8_quantize", e);
    return FP8_OK;
}

fp8_status fp8_quantize_many(int count, const void* const* x, const int64_t* rows, const int64_t* cols,
                             const fp8_fmt* fmt, const float* const* absmax, uint8_t* const* q, uint8_t* const* qt,
                             float* const* scale, float* const* inv_scale, const int* qt_later, hipStream_t stream)
{
    t_last_error.clear();
    const std::string f("fp8_quantize_many");
    if (!x || !rows || !cols || !fmt || !absmax || !q || !qt || !scale || !inv_scale)
        return fail(FP8_ERR_INVALID, f + ": null array");
    if (count < 1 || count > fp8k::kMaxQuantTensors) return fail(FP8_ERR_INVALID, f + ": count must be in [1, 8]");
    std::vector<Range> in, out;
    int64_t tiles = 0;
    int fm[fp8k::kMaxQuantTensors];
    for (int i = 0; i < count; ++i) {
        const std::string t = f + ": tensor " + std::to_string(i);
        if (!x[i] || !absmax[i]) return fail(FP8_ERR_INVALID, t + ": null x or absmax");
        if (!q[i] && !qt[i]) return fail(FP8_ERR_INVALID, t + ": at least one of q, qt is required");
        if (fmt[i] != FP8_E4M3 && fmt[i] != FP8_E5M2) return fail(FP8_ERR_INVALID, t + ": bad format");
        if (!mul_ok(rows[i], cols[i], kMaxElems)) return fail(FP8_ERR_INVALID, t + ": bad shape");
        if (rows[i] % 16 || cols[i] % 16)
            return fail(FP8_ERR_UNSUPPORTED, t + ": rows and cols must be multiples of 16");
        if (!aligned(x[i], 16) || (q[i] && !aligned(q[i], 16)) || (qt[i] && !aligned(qt[i], 16)) ||
            !aligned(absmax[i], 4) || (scale[i] && !aligned(scale[i], 4)) || (inv_scale[i] && !aligned(inv_scale[i], 4)))
            return fail(FP8_ERR_UNSUPPORTED, t + ": misaligned pointer");
        const int64_t n = rows[i] * cols[i];
        tiles += ((rows[i] + 127) / 128) * ((cols[i] + 127) / 128);
        in.push_back({x[i], 2 * n});
        in.push_back({absmax[i], 4});
        out.push_back({q[i], q[i] ? n : 0});
        out.push_back({qt[i], qt[i] ? n : 0});
        out.push_back({scale[i], scale[i] ? 4 : 0});
        out.push_back({inv_scale[i], inv_scale[i] ? 4 : 0});
        fm[i] = (int)fmt[i];
    }
    if (tiles > 0x7FFFFFFF) return fail(FP8_ERR_UNSUPPORTED, f + ": too many tiles for one launch");
    // inputs may be shared (they are only read); no output may overlap an input or another output
    for (size_t a = 0; a < out.size(); ++a) {
        for (size_t b = a + 1; b < out.size(); ++b)
            if (overlap(out[a].p, out[a].n, out[b].p, out[b].n)) return fail(FP8_ERR_INVALID, f + ": overlapping outputs");
        for (const Range& r : in)
            if (overlap(out[a].p, out[a].n, r.p, r.n)) return fail(FP8_ERR_INVALID, f + ": an output overlaps an input");
    }
    hipError_t e = fp8k::launch_quantize_many(count, x, rows, cols, fm, absmax, q, qt, scale, inv_scale, qt_later,
                                              stream);
    if (e != hipSuccess) return fail_hip("fp8_quantize_many", e);
    return FP8_OK;
}

fp8_status fp8_swiglu_requant(const void* gu, int64_t M, int64_t F, float* absmax_h, int compute_absmax,
                              uint8_t* hq, uint8_t* hqt, float* inv_scale_h, hipStream_t stream)
{
    t_last_error.clear();
    if (!gu || !absmax_h) return fail(FP8_ERR_INVALID, "fp8_swiglu_requant: null gu or absmax_h");
    if (!hq && !hqt) return fail(FP8_ERR_INVALID, "fp8_swiglu_requant: at least one of hq, hqt is required");
    if (compute_absmax < 0 || compute_absmax > 2)
        return fail(FP8_ERR_INVALID, "fp8_swiglu_requant: compute_absmax must be 0, 1 or 2");
    if (F <= 0 || F > kMaxElems || !mul_ok(M, 2 * F, kMaxElems))
        return fail(FP8_ERR_INVALID, "fp8_swiglu_requant: bad shape");
    const int64_t n = M * F;
    const Range r[] = {{gu, 4 * n}, {absmax_h, 4}, {hq, hq ? n : 0}, {hqt, hqt ? n : 0},
                       {inv_scale_h, inv_scale_h ? 4 : 0}};
    if (any_overlap(r)) return fail(FP8_ERR_INVALID, "fp8_swiglu_requant: overlapping buffers");
    if (F % 16) return fail(FP8_ERR_UNSUPPORTED, "fp8_swiglu_requant: F must be a multiple of 16");
    if (hqt && M % 16) return fail(FP8_ERR_UNSUPPORTED, "fp8_swiglu_requant: M must be a multiple of 16 with hqt");
    if (!aligned(gu, 16) || (hq && !aligned(hq, 16)) || (hqt && !aligned(hqt, 16)) || !aligned(absmax_h, 4) ||
        (inv_scale_h && !aligned(inv_scale_h, 4)))
        return fail(FP8_ERR_UNSUPPORTED, "fp8_swiglu_requant: misaligned pointer");
    hipError_t e = fp8k::launch_swiglu_requant(gu, M, F, absmax_h, compute_absmax, hq, hqt, inv_scale_h, stream);
    if (e != hipSuccess) return fail_hip("fp8_swiglu_requant", e);
    return FP8_OK;
}

fp8_status fp8_swiglu_backward(const void* gu, const void* dh, int64_t M, int64_t F, fp8_fmt fmt, float* absmax,
                               uint8_t* q, uint8_t* qt, float* scale, float* inv_scale, hipStream_t stream)
{
    t_last_error.clear();
    if (!gu || !dh || !absmax) return fail(FP8_ERR_INVALID, "fp8_swiglu_backward: null gu, dh or absmax");
    if (!q && !qt) return fail(FP8_ERR_INVALID, "fp8_swiglu_backward: at least one of q, qt is required");
    if (fmt != FP8_E4M3 && fmt != FP8_E5M2) return fail(FP8_ERR_INVALID, "fp8_swiglu_backward: bad format");
    if (F <= 0 || F > kMaxElems || !mul_ok(M, 2 * F, kMaxElems))
        return fail(FP8_ERR_INVALID, "fp8_swiglu_backward: bad shape");
    const int64_t n = M * F;
    const Range r[] = {{gu, 4 * n}, {dh, 2 * n}, {absmax, 4}, {q, q ? 2 * n : 0}, {qt, qt ? 2 * n : 0},
                       {scale, scale ? 4 : 0}, {inv_scale, inv_scale ? 4 : 0}};
    // the two inputs may alias each other; no output may alias anything
    for (int i = 2; i < 7; ++i)
        for (int j = 0; j < 7; ++j)
            if (i != j && overlap(r[i].p, r[i].n, r[j].p, r[j].n))
                return fail(FP8_ERR_INVALID, "fp8_swiglu_backward: overlapping buffers");
    if (F % 16) return fail(FP8_ERR_UNSUPPORTED, "fp8_swiglu_backward: F must be a multiple of 16");
    if (qt && M % 16) return fail(FP8_ERR_UNSUPPORTED, "fp8_swiglu_backward: M must be a multiple of 16 with qt");
    if (!aligned(gu, 16) || !aligned(dh, 16) || (q && !aligned(q, 16)) || (qt && !aligned(qt, 16)) ||
        !aligned(absmax, 4) || (scale && !aligned(scale, 4)) || (inv_scale && !aligned(inv_scale, 4)))
        return fail(FP8_ERR_UNSUPPORTED, "fp8_swiglu_backward: misaligned pointer");
    hipError_t e = fp8k::launch_swiglu_backward(gu, dh, M, F, (int)fmt, absmax, q, qt, scale, inv_scale, stream);
    if (e != hipSuccess) return fail_hip("fp8_swiglu_backward", e);
    return FP8_OK;
}

// Shared checks of the three GEMM calls, in the TN form out[P, Q] = A[P, R] . B[Q, R]^T.
// The block-scaled call passes need_inv = false (it has no per-tensor factors).
static fp8_status gemm_common(const char* name, const uint8_t* A, int fmt_a, const uint8_t* B, const float* inv_a,
                              const float* inv_b, void* out, int64_t P, int64_t Q, int64_t R, hipStream_t stream,
                              bool need_inv = true)
{
    char msg[160];
    if (!A || !B || (need_inv && (!inv_a || !inv_b)) || !out) {
        std::snprintf(msg, sizeof(msg), "%s: null pointer", name);
        return fail(FP8_ERR_INVALID, msg);
    }
    if (fmt_a != FP8_E4M3 && fmt_a != FP8_E5M2) {
        std::snprintf(msg, sizeof(msg), "%s: bad operand format", name);
        return fail(FP8_ERR_INVALID, msg);
    }
    if (P <= 0 || Q <= 0 || R <= 0) {
        std::snprintf(msg, sizeof(msg), "%s: dimensions must be positive", name);
        return fail(FP8_ERR_INVALID, msg);
    }
    // bound each dimension before forming any product (P * R, 2 * P * Q stay far below 2^63)
    if (P >= ((int64_t)1 << 30) || Q >= ((int64_t)1 << 30) || R >= ((int64_t)1 << 31)) {
        std::snprintf(msg, sizeof(msg), "%s: operand larger than 2 GiB", name);
        return fail(FP8_ERR_UNSUPPORTED, msg);
    }
    const Range r[] = {{A, P * R}, {B, Q * R}, {inv_a, need_inv ? 4 : 0}, {inv_b, need_inv ? 4 : 0},
                       {out, 2 * P * Q}};
    // the two inputs may alias each other (e.g. A == B); the output may alias nothing
    for (int i = 0; i < 4; ++i)
        if (overlap(r[i].p, r[i].n, r[4].p, r[4].n)) {
            std::snprintf(msg, sizeof(msg), "%s: output overlaps an input", name);
            return fail(FP8_ERR_INVALID, msg);
        }
    if (P % 16 || Q % 16 || R % 128 || P < 16 || Q < 16) {
        std::snprintf(msg, sizeof(msg), "%s: output dimensions must be multiples of 16, the reduction a multiple of 128",
                      name);
        return fail(FP8_ERR_UNSUPPORTED, msg);
    }
    if (P * R >= ((int64_t)1 << 31) || Q * R >= ((int64_t)1 << 31) || P >= ((int64_t)1 << 30) ||
        Q >= ((int64_t)1 << 30) || ((P + 255) / 256) * ((Q + 255) / 256) >= ((int64_t)1 << 31)) {
        std::snprintf(msg, sizeof(msg), "%s: operand larger than 2 GiB", name);
        return fail(FP8_ERR_UNSUPPORTED, msg);
    }
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(out, 16) || (need_inv && (!aligned(inv_a, 4) || !aligned(inv_b, 4)))) {
        std::snprintf(msg, sizeof(msg), "%s: misaligned pointer", name);
        return fail(FP8_ERR_UNSUPPORTED, msg);
    }
    (void)stream;
    return FP8_OK;
}

fp8_status fp8_gemm_fwd(const uint8_t* xq, const uint8_t* wq, const float* inv_sx, const float* inv_sw, void* y,
                        int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    t_last_error.clear();
    fp8_status st = gemm_common("fp8_gemm_fwd", xq, FP8_E4M3, wq, inv_sx, inv_sw, y, M, N, K, stream);
    if (st != FP8_OK) return st;
    // Y is stored non-temporally when it is too large to stay in the 256 MiB Infinity
    // Cache for the pass that reads it next while the operands are small enough to
    // stay there: then ordinary stores would only push out the operand panels the
    // launch keeps re-reading.  Measured on MI355X: the 14B-class gate/up forward
    // (453 MB out, 183 MB in) 9.6% faster, the step 1.6% shorter; with operands that
    // do not fit either (the 32B-class gate/up forward, 367 MB in) non-temporal
    // stores were 1% slower, and below 256 MiB of output (every 7B-class forward)
    // the next pass reads Y from the cache.
    const int64_t cache_bytes = (int64_t)256 << 20;
    const bool nt = 2 * M * N >= cache_bytes && (M + N) * K <= cache_bytes;
    hipError_t e = fp8k::launch_gemm_tn(xq, 0, 0, wq, 0, 0, inv_sx, inv_sw, y, M, N, K, nt, stream);
    if (e != hipSuccess) return fail_hip("fp8_gemm_fwd", e);
    return FP8_OK;
}

fp8_status fp8_gemm_fwd_swiglu_absmax(const uint8_t* xq, const uint8_t* wq, const float* inv_sx,
                                      const float* inv_sw, void* gu, float* absmax_h, int64_t M, int64_t F,
                                      int64_t K, hipStream_t stream)
{
    t_last_error.clear();
    const char* name = "fp8_gemm_fwd_swiglu_absmax";
    if (!absmax_h) return fail(FP8_ERR_INVALID, "fp8_gemm_fwd_swiglu_absmax: null absmax_h");
    if (F <= 0 || F > ((int64_t)1 << 29)) return fail(FP8_ERR_INVALID, "fp8_gemm_fwd_swiglu_absmax: bad F");
    fp8_status st = gemm_common(name, xq, FP8_E4M3, wq, inv_sx, inv_sw, gu, M, 2 * F, K, stream);
    if (st != FP8_OK) return st;
    const Range r[] = {{xq, M * K}, {wq, 2 * F * K}, {inv_sx, 4}, {inv_sw, 4}, {gu, 2 * M * 2 * F}};
    for (const Range& x : r)
        if (overlap(x.p, x.n, absmax_h, 4))
            return fail(FP8_ERR_INVALID, "fp8_gemm_fwd_swiglu_absmax: absmax_h overlaps another buffer");
    if (!aligned(absmax_h, 4)) return fail(FP8_ERR_UNSUPPORTED, "fp8_gemm_fwd_swiglu_absmax: misaligned absmax_h");
    if (F % 128 || M < 256)
        return fail(FP8_ERR_UNSUPPORTED, "fp8_gemm_fwd_swiglu_absmax: needs F % 128 == 0 and M >= 256");
    hipError_t e = fp8k::launch_gemm_gate_up(xq, wq, inv_sx, inv_sw, gu, absmax_h, M, F, K, stream);
    if (e != hipSuccess) return fail_hip(name, e);
    return FP8_OK;
}

fp8_status fp8_gemm_dgrad(const uint8_t* dyq, fp8_fmt dy_fmt, const uint8_t* wqt, const float* inv_sdy,
                          const float* inv_sw, void* dx, int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    t_last_error.clear();
    fp8_status st = gemm_common("fp8_gemm_dgrad", dyq, (int)dy_fmt, wqt, inv_sdy, inv_sw, dx, M, K, N, stream);
    if (st != FP8_OK) return st;
    hipError_t e = fp8k::launch_gemm_tn(dyq, (int)dy_fmt, 0, wqt, 0, 0, inv_sdy, inv_sw, dx, M, K, N, true, stream);
    if (e != hipSuccess) return fail_hip("fp8_gemm_dgrad", e);
    return FP8_OK;
}

fp8_status fp8_gemm_wgrad(const uint8_t* dyqt, fp8_fmt dy_fmt, const uint8_t* xqt, const float* inv_sdy,
                          const float* inv_sx, void* dw, int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    t_last_error.clear();
    fp8_status st = gemm_common("fp8_gemm_wgrad", dyqt, (int)dy_fmt, xqt, inv_sdy, inv_sx, dw, N, K, M, stream);
    if (st != FP8_OK) return st;
    hipError_t e = fp8k::launch_gemm_tn(dyqt, (int)dy_fmt, 0, xqt, 0, 0, inv_sdy, inv_sx, dw, N, K, M, true, stream);
    if (e != hipSuccess) return fail_hip("fp8_gemm_wgrad", e);
    return FP8_OK;
}

fp8_status fp8_gemm_backward(const uint8_t* dyq, const uint8_t* dyqt, fp8_fmt dy_fmt, const uint8_t* wqt,
                             const uint8_t* xqt, const float* inv_sdy, const float* inv_sw, const float* inv_sx,
                             void* dx, void* dw, int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    t_last_error.clear();
    fp8_status st = gemm_common("fp8_gemm_backward (dgrad)", dyq, (int)dy_fmt, wqt, inv_sdy, inv_sw, dx, M, K, N, stream);
    if (st != FP8_OK) return st;
    st = gemm_common("fp8_gemm_backward (wgrad)", dyqt, (int)dy_fmt, xqt, inv_sdy, inv_sx, dw, N, K, M, stream);
    if (st != FP8_OK) return st;
    const Range outs[] = {{dx, 2 * M * K}, {dw, 2 * N * K}};
    const Range ins[] = {{dyq, M * N}, {dyqt, M * N}, {wqt, K * N}, {xqt, K * M},
                         {inv_sdy, 4}, {inv_sw, 4}, {inv_sx, 4}};
    if (overlap(dx, 2 * M * K, dw, 2 * N * K))
        return fail(FP8_ERR_INVALID, "fp8_gemm_backward: dx and dw overlap");
    for (const Range& o : outs)
        for (const Range& i : ins)
            if (overlap(o.p, o.n, i.p, i.n)) return fail(FP8_ERR_INVALID, "fp8_gemm_backward: an output overlaps an input");
    hipError_t e = fp8k::launch_gemm_tn_pair(dyq, 0, wqt, 0, inv_sdy, inv_sw, dx, M, K, N, dyqt, 0, xqt, 0, inv_sdy,
                                             inv_sx, dw, N, K, M, (int)dy_fmt, 0, stream);
    if (e != hipSuccess) return fail_hip("fp8_gemm_backward", e);
    return FP8_OK;
}

// ---- the same products on the untransposed FP8 tensors (MN-major operands)

fp8_status fp8_gemm_dgrad_mn(const uint8_t* dyq, fp8_fmt dy_fmt, const uint8_t* wq, const float* inv_sdy,
                             const float* inv_sw, void* dx, int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    t_last_error.clear();
    fp8_status st = gemm_common("fp8_gemm_dgrad_mn", dyq, (int)dy_fmt, wq, inv_sdy, inv_sw, dx, M, K, N, stream);
    if (st != FP8_OK) return st;
    hipError_t e = fp8k::launch_gemm_tn(dyq, (int)dy_fmt, 0, wq, 0, 1, inv_sdy, inv_sw, dx, M, K, N, true, stream);
    if (e != hipSuccess) return fail_hip("fp8_gemm_dgrad_mn", e);
    return FP8_OK;
}

fp8_status fp8_gemm_wgrad_mn(const uint8_t* dyq, fp8_fmt dy_fmt, const uint8_t* xq, const float* inv_sdy,
                             const float* inv_sx, void* dw, int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    t_last_error.clear();
    fp8_status st = gemm_common("fp8_gemm_wgrad_mn", dyq, (int)dy_fmt, xq, inv_sdy, inv_sx, dw, N, K, M, stream);
    if (st != FP8_OK) return st;
    hipError_t e = fp8k::launch_gemm_tn(dyq, (int)dy_fmt, 1, xq, 0, 1, inv_sdy, inv_sx, dw, N, K, M, true, stream);
    if (e != hipSuccess) return fail_hip("fp8_gemm_wgrad_mn", e);
    return FP8_OK;
}

fp8_status fp8_gemm_backward_mn(const uint8_t* dyq, fp8_fmt dy_fmt, const uint8_t* wq, const uint8_t* xq,
                                const float* inv_sdy, const float* inv_sw, const float* inv_sx, void* dx, void* dw,
                                int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    t_last_error.clear();
    fp8_status st = gemm_common("fp8_gemm_backward_mn (dgrad)", dyq, (int)dy_fmt, wq, inv_sdy, inv_sw, dx, M, K, N,
                                stream);
    if (st != FP8_OK) return st;
    st = gemm_common("fp8_gemm_backward_mn (wgrad)", dyq, (int)dy_fmt, xq, inv_sdy, inv_sx, dw, N, K, M, stream);
    if (st != FP8_OK) return st;
    const Range outs[] = {{dx, 2 * M * K}, {dw, 2 * N * K}};
    const Range ins[] = {{dyq, M * N}, {wq, K * N}, {xq, K * M}, {inv_sdy, 4}, {inv_sw, 4}, {inv_sx, 4}};
    if (overlap(dx, 2 * M * K, dw, 2 * N * K))
        return fail(FP8_ERR_INVALID, "fp8_gemm_backward_mn: dx and dw overlap");
    for (const Range& o : outs)
        for (const Range& i : ins)
            if (overlap(o.p, o.n, i.p, i.n))
                return fail(FP8_ERR_INVALID, "fp8_gemm_backward_mn: an output overlaps an input");
    hipError_t e = fp8k::launch_gemm_tn_pair(dyq, 0, wq, 1, inv_sdy, inv_sw, dx, M, K, N, dyq, 1, xq, 1, inv_sdy,
                                             inv_sx, dw, N, K, M, (int)dy_fmt, 0, stream);
    if (e != hipSuccess) return fail_hip("fp8_gemm_backward_mn", e);
    return FP8_OK;
}

fp8_status fp8_mx_quantize(const void* x, int64_t rows, int64_t cols, fp8_fmt fmt, uint8_t* q, uint8_t* scales,
                           hipStream_t stream)
{
    t_last_error.clear();
    if (!x || !q || !scales) return fail(FP8_ERR_INVALID, "fp8_mx_quantize: null pointer");
    if (fmt != FP8_E4M3 && fmt != FP8_E5M2) return fail(FP8_ERR_INVALID, "fp8_mx_quantize: bad format");
    if (!mul_ok(rows, cols, kMaxElems)) return fail(FP8_ERR_INVALID, "fp8_mx_quantize: bad shape");
    const int64_t n = rows * cols;
    const Range r[] = {{x, 2 * n}, {q, n}, {scales, n / 32}};
    if (any_overlap(r)) return fail(FP8_ERR_INVALID, "fp8_mx_quantize: overlapping buffers");
    if (cols % 128) return fail(FP8_ERR_UNSUPPORTED, "fp8_mx_quantize: cols must be a multiple of 128");
    if (n / 32 >= ((int64_t)1 << 32)) return fail(FP8_ERR_UNSUPPORTED, "fp8_mx_quantize: more than 2^32 blocks");
    if (!aligned(x, 16) || !aligned(q, 16)) return fail(FP8_ERR_UNSUPPORTED, "fp8_mx_quantize: misaligned pointer");
    hipError_t e = fp8k::launch_mx_quantize(x, rows, cols, (int)fmt, q, scales, stream);
    if (e != hipSuccess) return fail_hip("fp8_mx_quantize", e);
    return FP8_OK;
}

fp8_status fp8_mx_quantize_t(const void* x, int64_t rows, int64_t cols, fp8_fmt fmt, uint8_t* qt, uint8_t* scales,
                             hipStream_t stream)
{
    t_last_error.clear();
    if (!x || !qt || !scales) return fail(FP8_ERR_INVALID, "fp8_mx_quantize_t: null pointer");
    if (fmt != FP8_E4M3 && fmt != FP8_E5M2) return fail(FP8_ERR_INVALID, "fp8_mx_quantize_t: bad format");
    if (!mul_ok(rows, cols, kMaxElems)) return fail(FP8_ERR_INVALID, "fp8_mx_quantize_t: bad shape");
    const int64_t n = rows * cols;
    const Range r[] = {{x, 2 * n}, {qt, n}, {scales, n / 32}};
    if (any_overlap(r)) return fail(FP8_ERR_INVALID, "fp8_mx_quantize_t: overlapping buffers");
    if (rows % 128 || cols % 128) return fail(FP8_ERR_UNSUPPORTED, "fp8_mx_quantize_t: rows and cols must be multiples of 128");
    if (!aligned(x, 16) || !aligned(qt, 16) || !aligned(scales, 4))
        return fail(FP8_ERR_UNSUPPORTED, "fp8_mx_quantize_t: misaligned pointer");
    hipError_t e = fp8k::launch_mx_quantize_t(x, rows, cols, (int)fmt, qt, scales, stream);
    if (e != hipSuccess) return fail_hip("fp8_mx_quantize_t", e);
    return FP8_OK;
}

fp8_status fp8_mx_quantize_both(const void* x, int64_t rows, int64_t cols, fp8_fmt fmt, uint8_t* q, uint8_t* sq,
                                uint8_t* qt, uint8_t* sqt, hipStream_t stream)
{
    t_last_error.clear();
    if (!x || !q || !sq || !qt || !sqt) return fail(FP8_ERR_INVALID, "fp8_mx_quantize_both: null pointer");
    if (fmt != FP8_E4M3 && fmt != FP8_E5M2) return fail(FP8_ERR_INVALID, "fp8_mx_quantize_both: bad format");
    if (!mul_ok(rows, cols, kMaxElems)) return fail(FP8_ERR_INVALID, "fp8_mx_quantize_both: bad shape");
    const int64_t n = rows * cols;
    const Range r[] = {{x, 2 * n}, {q, n}, {sq, n / 32}, {qt, n}, {sqt, n / 32}};
    if (any_overlap(r)) return fail(FP8_ERR_INVALID, "fp8_mx_quantize_both: overlapping buffers");
    if (rows % 128 || cols % 128) return fail(FP8_ERR_UNSUPPORTED, "fp8_mx_quantize_both: rows and cols must be multiples of 128");
    if (n / 32 >= ((int64_t)1 << 31)) return fail(FP8_ERR_UNSUPPORTED, "fp8_mx_quantize_both: tensor too large");
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(qt, 16) || !aligned(sq, 4) || !aligned(sqt, 4))
        return fail(FP8_ERR_UNSUPPORTED, "fp8_mx_quantize_both: misaligned pointer");
    hipError_t e = fp8k::launch_mx_quantize_both(x, rows, cols, (int)fmt, q, sq, qt, sqt, stream);
    if (e != hipSuccess) return fail_hip("fp8_mx_quantize_both", e);
    return FP8_OK;
}

fp8_status fp8_mx_swiglu_requant(const void* gu, int64_t M, int64_t F, uint8_t* hq, uint8_t* scales,
                                 hipStream_t stream)
{
    t_last_error.clear();
    if (!gu || !hq || !scales) return fail(FP8_ERR_INVALID, "fp8_mx_swiglu_requant: null pointer");
    if (M <= 0 || F <= 0 || !mul_ok(M, 2 * F, kMaxElems)) return fail(FP8_ERR_INVALID, "fp8_mx_swiglu_requant: bad shape");
    const Range r[] = {{gu, 4 * M * F}, {hq, M * F}, {scales, M * F / 32}};
    if (any_overlap(r)) return fail(FP8_ERR_INVALID, "fp8_mx_swiglu_requant: overlapping buffers");
    if (F % 128) return fail(FP8_ERR_UNSUPPORTED, "fp8_mx_swiglu_requant: F must be a multiple of 128");
    if (!aligned(gu, 16) || !aligned(hq, 16)) return fail(FP8_ERR_UNSUPPORTED, "fp8_mx_swiglu_requant: misaligned pointer");
    hipError_t e = fp8k::launch_mx_swiglu(gu, M, F, hq, scales, stream);
    if (e != hipSuccess) return fail_hip("fp8_mx_swiglu_requant", e);
    return FP8_OK;
}

fp8_status fp8_mx_gemm_fwd(const uint8_t* xq, const uint8_t* sx, fp8_fmt x_fmt, const uint8_t* wq, const uint8_t* sw,
                           void* y, int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    t_last_error.clear();
    const char* name = "fp8_mx_gemm_fwd";
    if (!sx || !sw) return fail(FP8_ERR_INVALID, "fp8_mx_gemm_fwd: null scales");
    fp8_status st = gemm_common(name, xq, (int)x_fmt, wq, nullptr, nullptr, y, M, N, K, stream, false);
    if (st != FP8_OK) return st;
    if (overlap(sx, M * (K / 32), y, 2 * M * N) || overlap(sw, N * (K / 32), y, 2 * M * N))
        return fail(FP8_ERR_INVALID, "fp8_mx_gemm_fwd: output overlaps the scales");
    if (M < 256 || N < 256) return fail(FP8_ERR_UNSUPPORTED, "fp8_mx_gemm_fwd: M and N must be at least 256");
    if (!aligned(sx, 4) || !aligned(sw, 4)) return fail(FP8_ERR_UNSUPPORTED, "fp8_mx_gemm_fwd: misaligned scales");
    hipError_t e = fp8k::launch_gemm_mx(xq, sx, (int)x_fmt, wq, sw, 0, y, M, N, K, stream);
    if (e != hipSuccess) return fail_hip(name, e);
    return FP8_OK;
}

fp8_status fp8_mx_gemm_backward(const uint8_t* dyq, const uint8_t* sdy, const uint8_t* dyqt, const uint8_t* sdyt,
                                fp8_fmt dy_fmt, const uint8_t* wqt, const uint8_t* swt, const uint8_t* xqt,
                                const uint8_t* sxt, void* dx, void* dw, int64_t M, int64_t N, int64_t K,
                                hipStream_t stream)
{
    t_last_error.clear();
    const char* name = "fp8_mx_gemm_backward";
    if (!sdy || !sdyt || !swt || !sxt) return fail(FP8_ERR_INVALID, "fp8_mx_gemm_backward: null scales");
    fp8_status st = gemm_common("fp8_mx_gemm_backward (dgrad)", dyq, (int)dy_fmt, wqt, nullptr, nullptr, dx, M, K, N,
                                stream, false);
    if (st != FP8_OK) return st;
    st = gemm_common("fp8_mx_gemm_backward (wgrad)", dyqt, (int)dy_fmt, xqt, nullptr, nullptr, dw, N, K, M, stream,
                     false);
    if (st != FP8_OK) return st;
    if (M < 256 || N < 256 || K < 256)
        return fail(FP8_ERR_UNSUPPORTED, "fp8_mx_gemm_backward: M, N and K must be at least 256");
    if (!aligned(sdy, 4) || !aligned(sdyt, 4) || !aligned(swt, 4) || !aligned(sxt, 4))
        return fail(FP8_ERR_UNSUPPORTED, "fp8_mx_gemm_backward: misaligned scales");
    if (overlap(dx, 2 * M * K, dw, 2 * N * K)) return fail(FP8_ERR_INVALID, "fp8_mx_gemm_backward: dx and dw overlap");
    const Range outs[] = {{dx, 2 * M * K}, {dw, 2 * N * K}};
    const Range ins[] = {{dyq, M * N},       {dyqt, M * N},       {wqt, K * N},       {xqt, K * M},
                         {sdy, M * N / 32}, {sdyt, M * N / 32}, {swt, K * N / 32}, {sxt, K * M / 32}};
    for (const Range& o : outs)
        for (const Range& i : ins)
            if (overlap(o.p, o.n, i.p, i.n))
                return fail(FP8_ERR_INVALID, "fp8_mx_gemm_backward: an output overlaps an input");
    hipError_t e = fp8k::launch_gemm_mx_pair(dyq, sdy, wqt, swt, dx, M, K, N, dyqt, sdyt, xqt, sxt, dw, N, K, M,
                                             (int)dy_fmt, stream);
    if (e != hipSuccess) return fail_hip(name, e);
    return FP8_OK;
}

fp8_status fp8_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream)
{
    t_last_error.clear();
    if (!src || !dst) return fail(FP8_ERR_INVALID, "fp8_stream_copy: null pointer");
    if (bytes <= 0 || bytes > 2 * kMaxElems) return fail(FP8_ERR_INVALID, "fp8_stream_copy: bytes must be in [1, 2^41]");
    if (bytes % 16 != 0 || !aligned(src, 16) || !aligned(dst, 16))
        return fail(FP8_ERR_UNSUPPORTED, "fp8_stream_copy: bytes a multiple of 16, both buffers 16-byte aligned");
    if (overlap(src, bytes, dst, bytes)) return fail(FP8_ERR_INVALID, "fp8_stream_copy: src and dst overlap");
    hipError_t e = fp8k::launch_stream_copy(src, dst, bytes, stream);
    if (e != hipSuccess) return fail_hip("fp8_stream_copy", e);
    return FP8_OK;
}

}  // extern "C"
