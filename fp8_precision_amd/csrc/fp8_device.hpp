// fp8_device.hpp -- device-side helpers shared by the gfx950 kernels.
//
// bf16 unpacking, the per-tensor scale, and the OFP8 encoder built on the
// hardware convert.  Measured on gfx950: v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32
// round to nearest even but do not saturate (an E4M3 overflow gives NaN, an
// E5M2 overflow gives infinity), so values are first clamped to +-max with
// v_med3_f32.  v_med3_f32 replaces a NaN operand by a bound, so a NaN is passed
// to the convert unclamped, which then yields a NaN code.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8k {

constexpr float kMaxE4M3 = 448.0f;
constexpr float kMaxE5M2 = 57344.0f;
constexpr float kFltMax = 3.40282346638528859812e+38f;

template <int FMT> struct Fmt;
template <> struct Fmt<0> { static constexpr float max = kMaxE4M3; };
template <> struct Fmt<1> { static constexpr float max = kMaxE5M2; };

// The two bf16 halves of a 32-bit word, as fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Per-tensor scale from an absmax: s = RN32(fp8_max / absmax), 1 when absmax is
// zero, FLT_MAX when the quotient overflows; inv = RN32(1 / s).  Both quotients
// are formed in binary64 and rounded once to binary32, which gives the
// correctly rounded binary32 quotient (53 >= 2 * 24 + 2).
__device__ __forceinline__ void tensor_scale(float absmax, float fp8_max, float& s, float& inv)
{
    if (absmax == 0.0f) {
        s = 1.0f;
    } else {
        s = (float)((double)fp8_max / (double)absmax);
        if (s == __builtin_inff()) s = kFltMax;
    }
    inv = (float)(1.0 / (double)s);
}

template <int FMT>
__device__ __forceinline__ float saturate(float v)
{
    float c = __builtin_amdgcn_fmed3f(v, -Fmt<FMT>::max, Fmt<FMT>::max);
    return __builtin_isnan(v) ? v : c;
}

// Encode two values into bytes 0-1 (HI = false) or 2-3 (HI = true) of `old`.
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t cvt2(float a, float b, uint32_t old)
{
    if (FMT == 0) return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(saturate<0>(a), saturate<0>(b), (int)old, HI);
    return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(saturate<1>(a), saturate<1>(b), (int)old, HI);
}

// Four products v_i * s -> four codes in one word (byte i = element i).
template <int FMT>
__device__ __forceinline__ uint32_t enc4(float a, float b, float c, float d)
{
    uint32_t r = cvt2<FMT, false>(a, b, 0u);
    return cvt2<FMT, true>(c, d, r);
}

// Quantise the 8 bf16 of a 16-byte word with scale s -> 8 codes (2 words).
template <int FMT>
__device__ __forceinline__ uint2 quant8(uint4 x, float s)
{
    uint2 r;
    r.x = enc4<FMT>(bf16_lo(x.x) * s, bf16_hi(x.x) * s, bf16_lo(x.y) * s, bf16_hi(x.y) * s);
    r.y = enc4<FMT>(bf16_lo(x.z) * s, bf16_hi(x.z) * s, bf16_lo(x.w) * s, bf16_hi(x.w) * s);
    return r;
}

// Byte transpose of a 4x4 block held as 4 words (word r = row r, byte c = col c):
// returns in c0..c3 the columns (word c, byte r = row r).
__device__ __forceinline__ void transpose4x4(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3,
                                             uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3)
{
    // v_perm_b32 D, S0, S1, sel: byte i of D is byte sel[i] of the 8-byte value S0:S1
    // (selectors 0-3 pick S1's bytes, 4-7 pick S0's).
    uint32_t t01l = __builtin_amdgcn_perm(r1, r0, 0x05010400u);   // r0b0 r1b0 r0b1 r1b1
    uint32_t t01h = __builtin_amdgcn_perm(r1, r0, 0x07030602u);   // r0b2 r1b2 r0b3 r1b3
    uint32_t t23l = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
    uint32_t t23h = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
    c0 = __builtin_amdgcn_perm(t23l, t01l, 0x05040100u);          // r0b0 r1b0 r2b0 r3b0
    c1 = __builtin_amdgcn_perm(t23l, t01l, 0x07060302u);
    c2 = __builtin_amdgcn_perm(t23h, t01h, 0x05040100u);
    c3 = __builtin_amdgcn_perm(t23h, t01h, 0x07060302u);
}

// Max over a wavefront (64 lanes) of an unsigned value.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
        v = v > o ? v : o;
    }
    return v;
}

// Block-wide max of `v` (blockDim.x a multiple of 64, at most 1024) folded into
// *out.  `out` holds the fp32 bits of a non-negative value (or NaN with the sign
// bit clear), for which unsigned order equals the magnitude order used by the
// absmax definition.  One atomicMax per block: device-scope atomics on one
// address serialise past the (per-XCD) L2, so launches keep to about one block
// per CU.  A block first reads the running maximum and skips its atomic if it
// cannot raise it (a stale read is smaller or equal, so the test is safe).
__device__ __forceinline__ void block_max_to_global(uint32_t v, uint32_t* out)
{
    __shared__ uint32_t part[16];
    v = wave_max_u32(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if (lane == 0) part[wave] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t m = part[0];
        for (int w = 1; w < nw; ++w) m = m > part[w] ? m : part[w];
        const uint32_t seen = __hip_atomic_load(out, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (m > seen) atomicMax(out, m);
    }
}

}  // namespace fp8k
