// swiglu.hip -- SwiGLU fused with its E4M3 requantisation, for gfx950.
//
// "LLMQ: Efficient Lower-Precision Pretraining for Consumer GPUs", section 3.1:
// the block input and the forward's absmax statistic are kept, so the
// recomputed SwiGLU output is requantised in the kernel that evaluates it,
// with no second pass to find its maximum.
//
// h = RN32(s_g * u), s_g = RN32(g / RN32(1 + RN32(e^-g))) with e^-g correctly
// rounded.  g is a bf16 value, so s_g is a function of 16 bits.  It is read
// from a table for the bf16 exponents where it is non-trivial and given by
// exact rules elsewhere:
//   |g| < 2^(E_LO-127): e^-g rounds into [1 - 2^-24, 1 + 2^-23], 1 + E rounds
//                       to exactly 2, so s_g = RN32(g / 2) = RN32(g * 0.5);
//   |g| >= 2^(E_HI-126), g > 0 (and +inf, NaN): e^-g < 2^-24, 1 + E = 1, s_g = g;
//   same range, g < 0: e^-g overflows to +inf, s_g = g / inf = -0; -inf and
//                       NaN give NaN.
// The table (2 signs x 34 exponents x 128 mantissas, 34 KB) is constant device
// data compiled into the library: gen_silu_tables.py evaluates each entry
// exactly (e^-g to 60 digits) and rounds every step once to binary32 in the
// order above, at build time; kernels copy it into LDS.
//
// The backward (the gradients of gate and up, for the gate/up backward GEMMs)
// uses the textbook derivative of g * sigma(g): with sig = RN32(1 / t),
//   ds = RN32(sig * RN32(1 + RN32(g * RN32(1 - sig))))          (silu'(g))
//   du = RN32(dh * s_g),  dg = RN32(RN32(dh * u) * ds)
// ds is a function of the 16 bits of g too: a second table over the same
// exponent range, generated with the same single roundings; outside it
//   |g| < 2^-27: sig = 1/2, 1 + g/2 rounds to 1, ds = 1/2;
//   |g| >= 128 finite: g > 0 gives sig = 1, ds = 1; g < 0 gives sig = 0, ds = -0;
//   infinities and NaN: ds = NaN.
#include <mutex>
#include "fp8_device.hpp"
#include "fp8_internal.hpp"

namespace fp8k {

constexpr int kELo = kSiluELo;                // bf16 biased exponent range of the table
constexpr int kEHi = kSiluEHi;                // |g| in [2^-27, 128)
constexpr int kNE = kEHi - kELo + 1;          // 34
constexpr int kHalf = kNE * 128;              // entries per sign
constexpr int kTable = 2 * kHalf;             // 8704 entries

// Bit patterns of s_g and ds, written by gen_silu_tables.py into the build directory.
#include "silu_tables.inc"
static_assert(FP8_SILU_ELO == kELo && FP8_SILU_EHI == kEHi && FP8_SILU_ENTRIES == kTable,
              "generated SwiGLU tables do not match the kernel's exponent range");

__device__ __attribute__((aligned(16))) uint32_t g_silu_table[kTable] = {FP8_SILU_SG_BITS};
__device__ __attribute__((aligned(16))) uint32_t g_dsilu_table[kTable] = {FP8_SILU_DS_BITS};

// Device address of the s_g table on the current device (for kernels in other
// translation units), looked up once per device.  No kernel runs and the host
// does not wait: the table is part of the loaded code object.
hipError_t silu_table(const float** table, hipStream_t stream)
{
    (void)stream;
    static std::mutex mu;
    static const float* addr[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_silu_table));
        if (e != hipSuccess) return e;
        addr[dev] = static_cast<const float*>(p);
    }
    *table = addr[dev];
    return hipSuccess;
}

__device__ __forceinline__ void load_table_to_lds(float* lds)
{
    const float4* src = reinterpret_cast<const float4*>(g_silu_table);
    float4* dst = reinterpret_cast<float4*>(lds);
    for (int i = threadIdx.x; i < kTable / 4; i += blockDim.x) dst[i] = src[i];
    __syncthreads();
}

// The forward statistic's LDS table: |s_g| (only magnitudes are needed), the
// positive half at entry 0 and the negative half at entry kAbsNeg, in a 64 KB
// array: every 16-bit byte offset lies inside it.
constexpr int kAbsNeg = 8192;
constexpr int kAbsLds = 16384;

__device__ __forceinline__ void load_abs_table_to_lds(float* lds)
{
    const float4* src = reinterpret_cast<const float4*>(g_silu_table);
    float4* dst = reinterpret_cast<float4*>(lds);
    for (int i = threadIdx.x; i < kTable / 4; i += blockDim.x) {
        const float4 v = src[i];
        const int d = i < kHalf / 4 ? i : i - kHalf / 4 + kAbsNeg / 4;
        dst[d] = make_float4(fabsf(v.x), fabsf(v.y), fabsf(v.z), fabsf(v.w));
    }
    __syncthreads();
}

// Both tables (s_g, then ds) into 2 * 34 KB of LDS.
__device__ __forceinline__ void load_tables_to_lds(float* lds)
{
    const float4* s0 = reinterpret_cast<const float4*>(g_silu_table);
    const float4* s1 = reinterpret_cast<const float4*>(g_dsilu_table);
    float4* dst = reinterpret_cast<float4*>(lds);
    for (int i = threadIdx.x; i < kTable / 4; i += blockDim.x) {
        dst[i] = s0[i];
        dst[kTable / 4 + i] = s1[i];
    }
    __syncthreads();
}

// s_g for one bf16 gate value (16-bit pattern b, fp32 value g).  NEG: the index
// of the first entry of the negative half in tbl.
template <int NEG = kHalf>
__device__ __forceinline__ float silu_of(const float* tbl, uint32_t b, float g)
{
    const uint32_t t = (b & 0x7FFFu) - (uint32_t)(kELo * 128);
    const uint32_t neg = b >> 15;
    const bool in_table = t < (uint32_t)kHalf;
    const float tv = tbl[in_table ? t + neg * NEG : 0u];
    if (in_table) return tv;
    if ((int32_t)t < 0) return g * 0.5f;                     // tiny |g|
    if (!neg) return g;                                      // large g, +inf, +NaN
    return ((b & 0x7F80u) == 0x7F80u) ? __builtin_nanf("") : -0.0f;
}

// silu'(g) for one bf16 gate value (16-bit pattern b).
__device__ __forceinline__ float dsilu_of(const float* tbl, uint32_t b)
{
    const uint32_t t = (b & 0x7FFFu) - (uint32_t)(kELo * 128);
    const uint32_t neg = b >> 15;
    const bool in_table = t < (uint32_t)kHalf;
    const float tv = tbl[in_table ? t + neg * kHalf : 0u];
    if (in_table) return tv;
    if ((int32_t)t < 0) return 0.5f;                                 // tiny |g|
    if ((b & 0x7F80u) == 0x7F80u) return __builtin_nanf("");         // infinities, NaN
    return neg ? -0.0f : 1.0f;                                       // large finite |g|
}

// h for the 8 (gate, up) pairs of two 16-byte words.
template <int NEG = kHalf>
__device__ __forceinline__ void swiglu8(const float* tbl, uint4 gw, uint4 uw, float h[8])
{
    const uint32_t g32[4] = {gw.x, gw.y, gw.z, gw.w};
    const uint32_t u32[4] = {uw.x, uw.y, uw.z, uw.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float g0 = bf16_lo(g32[k]), g1 = bf16_hi(g32[k]);
        h[2 * k] = silu_of<NEG>(tbl, g32[k] & 0xFFFFu, g0) * bf16_lo(u32[k]);
        h[2 * k + 1] = silu_of<NEG>(tbl, g32[k] >> 16, g1) * bf16_hi(u32[k]);
    }
}

__device__ __forceinline__ uint32_t mag_max8(uint32_t m, const float h[8])
{
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t a = __float_as_uint(h[k]) & 0x7FFFFFFFu;
        m = m > a ? m : a;
    }
    return m;
}

__device__ __forceinline__ uint2 quant8_h(const float h[8], float s)
{
    uint2 r;
    r.x = enc4<0>(h[0] * s, h[1] * s, h[2] * s, h[3] * s);
    r.y = enc4<0>(h[4] * s, h[5] * s, h[6] * s, h[7] * s);
    return r;
}

// Work decomposition of the row-streaming kernels: a wave item is one row and
// 1024 consecutive columns j; lane l handles columns 8l..8l+7 and
// 512+8l..512+8l+7 of the item (one 16-byte load per half row and operand).
struct RowItems {
    int64_t chunks;     // items per row
    int64_t total;      // items in the tensor
};

__device__ __forceinline__ RowItems row_items(int64_t M, int64_t F)
{
    RowItems r;
    r.chunks = (F + 1023) / 1024;
    r.total = M * r.chunks;
    return r;
}

// Forward pass 1: absmax of h over the whole [M, F] output (no output written).
//
// Only magnitudes matter here: |h| = RN(|s_g| |u|) (rounding is symmetric in
// sign), read from the magnitude table above.  The fast form handles eight gate
// values without branches: for each 32-bit word (two gate values) the table
// byte offsets are ((|b| - base) << 2) | sign << 15 in packed 16-bit integer
// arithmetic, so they always fall inside the 64 KB table; a value outside the
// table's exponent range (tiny or large |g|, infinities, NaN) reads an entry
// that is discarded: it sets chk to kHalf or more, and its lane recomputes the
// whole item with the exact rules of silu_of.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u16x2 as_u16x2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }
__device__ __forceinline__ uint32_t as_u32(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }

__device__ __forceinline__ void swiglu_abs8_fast(const float* tbl, uint4 gw, uint4 uw, uint32_t& m, u16x2& chk)
{
    const uint32_t g32[4] = {gw.x, gw.y, gw.z, gw.w};
    const uint32_t u32[4] = {uw.x, uw.y, uw.z, uw.w};
    const char* base = reinterpret_cast<const char*>(tbl);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const u16x2 t = as_u16x2(g32[k] & 0x7FFF7FFFu) - (u16x2)(unsigned short)(kELo * 128);
        chk = __builtin_elementwise_max(chk, t);
        const uint32_t o = as_u32(t << (unsigned short)2) | (g32[k] & 0x80008000u);
        const float s0 = *reinterpret_cast<const float*>(base + (o & 0xFFFFu));
        const float s1 = *reinterpret_cast<const float*>(base + (o >> 16));
        // s0, s1 >= +0: the products are >= +0 or NaN (a NaN's sign is cleared
        // by the caller once per item)
        const uint32_t b0 = __float_as_uint(s0 * fabsf(bf16_lo(u32[k])));
        const uint32_t b1 = __float_as_uint(s1 * fabsf(bf16_hi(u32[k])));
        m = m > b0 ? m : b0;
        m = m > b1 ? m : b1;
    }
}

// A lane's share of one wave item: the gate and up words of its two half rows.
// A half row past F re-reads the row's last eight columns (F >= 16): repeated
// elements leave a maximum unchanged.
struct GuWords {
    uint4 g[2], u[2];
};

// Item (row i, chunk c) of a wave's walk through the items.  Successive items of
// a wave are `stride` apart: (i, c) advances by (q, r) = divmod(stride, chunks)
// with a carry, so the walk needs no division per item.
struct ItemPos {
    int64_t i;
    int64_t c;
};

__device__ __forceinline__ ItemPos advance(ItemPos p, int64_t q, int64_t r, int64_t chunks)
{
    p.i += q;
    p.c += r;
    if (p.c >= chunks) {
        p.c -= chunks;
        p.i += 1;
    }
    return p;
}

__device__ __forceinline__ GuWords load_item(const uint16_t* __restrict__ gu, int64_t F, ItemPos p, int lane)
{
    GuWords r;
    const int64_t jb = p.c * 1024 + lane * 8;
    const uint16_t* grow = gu + p.i * 2 * F;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int64_t j0 = jb + half * 512;
        const int64_t j = j0 < F ? j0 : F - 8;
        r.g[half] = *reinterpret_cast<const uint4*>(grow + j);
        r.u[half] = *reinterpret_cast<const uint4*>(grow + F + j);
    }
    return r;
}

__device__ __forceinline__ uint32_t item_absmax(const float* tbl, const GuWords& x)
{
    uint32_t mi = 0;
    u16x2 chk = (u16x2)(unsigned short)0;
    swiglu_abs8_fast(tbl, x.g[0], x.u[0], mi, chk);
    swiglu_abs8_fast(tbl, x.g[1], x.u[1], mi, chk);
    if (chk.x >= (unsigned short)kHalf || chk.y >= (unsigned short)kHalf) {
        mi = 0;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            float h[8];
            swiglu8<kAbsNeg>(tbl, x.g[half], x.u[half], h);
            mi = mag_max8(mi, h);
        }
    }
    return mi & 0x7FFFFFFFu;
}

// Each wave takes two items per iteration (w and w + stride), all eight 16-byte
// loads of a lane issued before any of them is used.  The wave's item index is
// uniform (kept in scalar registers).
__global__ void __launch_bounds__(1024) swiglu_absmax_kernel(const uint16_t* __restrict__ gu, int64_t M,
                                                            int64_t F, uint32_t* __restrict__ out)
{
    __shared__ float tbl[kAbsLds];
    load_abs_table_to_lds(tbl);
    const RowItems it = row_items(M, F);
    const int lane = threadIdx.x & 63;
    const int64_t wpb = blockDim.x >> 6;
    const int64_t stride = (int64_t)gridDim.x * wpb;
    const int64_t w0 = (int64_t)blockIdx.x * wpb + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t q = stride / it.chunks, r = stride - q * it.chunks;
    ItemPos pa = {w0 / it.chunks, w0 - (w0 / it.chunks) * it.chunks};
    uint32_t m = 0;
    for (int64_t w = w0; w < it.total; w += 2 * stride) {
        // past the end, the second item repeats the first (harmless for a maximum)
        const ItemPos pn = advance(pa, q, r, it.chunks);
        const ItemPos pb = w + stride < it.total ? pn : pa;
        const GuWords a = load_item(gu, F, pa, lane);
        const GuWords b = load_item(gu, F, pb, lane);
        __builtin_amdgcn_sched_barrier(0);    // every load in flight before the first use
        const uint32_t ma = item_absmax(tbl, a), mb = item_absmax(tbl, b);
        m = m > ma ? m : ma;
        m = m > mb ? m : mb;
        pa = advance(pn, q, r, it.chunks);
    }
    block_max_to_global(m, out);
}

// Pass 2 (forward) or the only pass (recomputation): hq = e4m3(RN32(h * s_h)).
__global__ void __launch_bounds__(256) swiglu_quant_kernel(const uint16_t* __restrict__ gu, int64_t M,
                                                           int64_t F, const float* __restrict__ absmax_h,
                                                           uint8_t* __restrict__ hq,
                                                           float* __restrict__ inv_out)
{
    __shared__ float tbl[kTable];
    float s, inv;
    tensor_scale(*absmax_h, kMaxE4M3, s, inv);
    if (blockIdx.x == 0 && threadIdx.x == 0 && inv_out) *inv_out = inv;
    load_table_to_lds(tbl);
    const RowItems it = row_items(M, F);
    const int lane = threadIdx.x & 63;
    for (int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); w < it.total; w += (int64_t)gridDim.x * 4) {
        const int64_t i = w / it.chunks;
        const int64_t jb = (w - i * it.chunks) * 1024 + lane * 8;
        const uint16_t* grow = gu + i * 2 * F;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int64_t j = jb + half * 512;
            if (j < F) {
                const uint4 gw = *reinterpret_cast<const uint4*>(grow + j);
                const uint4 uw = *reinterpret_cast<const uint4*>(grow + F + j);
                float h[8];
                swiglu8(tbl, gw, uw, h);
                *reinterpret_cast<uint2*>(hq + i * F + j) = quant8_h(h, s);
            }
        }
    }
}

// Requantisation with the transposed copy hqt [F, M] (and optionally hq).  A
// block of 4 waves owns a 128 x 128 tile of h and walks the tiles persistently
// (the s_g table is copied into LDS once per block).  Lane l of wave w takes the
// 8 x 8 block at rows 32 w + 8 (l / 16) .. and columns 8 (l % 16) ..: its 16
// loads (gate and up) are all issued first, each instruction reading four
// 256-byte row segments; hq is written as 128-byte row segments; the lane's
// 8 x 8 code block is transposed in registers (v_perm_b32) into eight 8-byte
// pieces of hqt rows, parked in a 16 KB LDS tile laid out as hqt ([128
// columns][128 rows], 16-byte pieces XOR-swizzled by column), and written back
// after a barrier as full 128-byte hqt row segments.  (Writing hqt straight from
// registers, 64 bytes per row and instruction, ran at 3.1-3.5 TB/s with a cold
// cache.)  M and F are multiples of 16, so a lane's block is whole.
constexpr int kSqEdge = 128;
typedef unsigned int u32x4s __attribute__((ext_vector_type(4)));

// NTQ: hqt written with non-temporal stores (the forward form: hqt is read by the
// backward pass, not by the next call; a compile-time choice, so the hint stays).
template <bool NTQ>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
swiglu_quant_t_kernel(const uint16_t* __restrict__ gu, int64_t M, int64_t F, const float* __restrict__ absmax_h,
                      uint8_t* __restrict__ hq, uint8_t* __restrict__ hqt, float* __restrict__ inv_out)
{
    __shared__ float tbl[kTable];                                               // 34 KB
    __shared__ __attribute__((aligned(16))) uint8_t tile[kSqEdge * kSqEdge];    // 16 KB
    float s, inv;
    tensor_scale(*absmax_h, kMaxE4M3, s, inv);
    if (blockIdx.x == 0 && threadIdx.x == 0 && inv_out) *inv_out = inv;
    load_table_to_lds(tbl);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rt = wave * 32 + (lane >> 4) * 8;           // first row of the lane within the tile
    const int ct = (lane & 15) * 8;                       // first column of the lane within the tile
    const int64_t ntc = (F + kSqEdge - 1) / kSqEdge;
    const int64_t ntiles = ntc * ((M + kSqEdge - 1) / kSqEdge);
    for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const int64_t tr = (t / ntc) * kSqEdge, tc = (t % ntc) * kSqEdge;
        if (tr + rt < M && tc + ct < F) {
            const int64_t i0 = tr + rt, j = tc + ct;
            uint4 gw[8], uw[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const uint16_t* grow = gu + (i0 + r) * 2 * F + j;
                gw[r] = *reinterpret_cast<const uint4*>(grow);
                uw[r] = *reinterpret_cast<const uint4*>(grow + F);
            }
            uint32_t lo[8], hi[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                float h[8];
                swiglu8(tbl, gw[r], uw[r], h);
                const uint2 c = quant8_h(h, s);
                lo[r] = c.x;
                hi[r] = c.y;
            }
            if (hq) {
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    *reinterpret_cast<uint2*>(hq + (i0 + r) * F + j) = make_uint2(lo[r], hi[r]);
            }
            // column k of the block: rows 0..3 (word 0) and rows 4..7 (word 1)
            uint32_t c0[8], c1[8];
            transpose4x4(lo[0], lo[1], lo[2], lo[3], c0[0], c0[1], c0[2], c0[3]);
            transpose4x4(lo[4], lo[5], lo[6], lo[7], c1[0], c1[1], c1[2], c1[3]);
            transpose4x4(hi[0], hi[1], hi[2], hi[3], c0[4], c0[5], c0[6], c0[7]);
            transpose4x4(hi[4], hi[5], hi[6], hi[7], c1[4], c1[5], c1[6], c1[7]);
            const int piece = rt >> 4, half = (rt >> 3) & 1;   // 8-byte half of a 16-byte piece
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int col = ct + k;
                const int phys = piece ^ ((col >> 3) & 7);
                *reinterpret_cast<uint2*>(tile + col * kSqEdge + phys * 16 + half * 8) = make_uint2(c0[k], c1[k]);
            }
        }
        __syncthreads();
        // write-back: 1024 pieces of 16 bytes, 4 per thread; a wave instruction
        // covers 8 hqt rows x 128 bytes
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int id = u * 256 + threadIdx.x;
            const int col = id >> 3, p = id & 7;
            const int64_t qrow = tc + col, qcol = tr + p * 16;
            if (qrow < F && qcol < M) {
                const int phys = p ^ ((col >> 3) & 7);
                const u32x4s piece16 = *reinterpret_cast<const u32x4s*>(tile + col * kSqEdge + phys * 16);
                u32x4s* dst = reinterpret_cast<u32x4s*>(hqt + qrow * M + qcol);
                if (NTQ)
                    __builtin_nontemporal_store(piece16, dst);
                else
                    *dst = piece16;
            }
        }
        __syncthreads();                                  // the tile is read back before it is reused
    }
}

__global__ void __launch_bounds__(64) zero_u32_kernel_sw(uint32_t* p)
{
    if (threadIdx.x == 0) *p = 0u;
}

hipError_t launch_swiglu_requant(const void* gu, int64_t M, int64_t F, float* absmax_h, int compute_absmax,
                                 uint8_t* hq, uint8_t* hqt, float* inv_scale_h, hipStream_t stream)
{
    const uint16_t* g = reinterpret_cast<const uint16_t*>(gu);
    const int64_t items = M * ((F + 1023) / 1024);
    int64_t blocks = (items + 3) / 4;
    const int64_t cap = (int64_t)device_cu_count() * 4;   // 34 KB LDS per block: 4 blocks per CU
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    if (compute_absmax) {
        // 1: reset first; 2: accumulate into the caller's (cleared) statistic
        hipError_t e = hipSuccess;
        if (compute_absmax == 1)
            e = launch(zero_u32_kernel_sw, dim3(1), dim3(64), stream, reinterpret_cast<uint32_t*>(absmax_h));
        if (e != hipSuccess) return e;
        // one 1024-thread block per CU: one atomic per CU, the table copied once per CU
        int64_t ablocks = (items + 15) / 16;
        if (ablocks > device_cu_count()) ablocks = device_cu_count();
        e = launch(swiglu_absmax_kernel, dim3((unsigned)ablocks), dim3(1024), stream, g, M, F,
                   reinterpret_cast<uint32_t*>(absmax_h));
        if (e != hipSuccess) return e;
    }
    if (hqt) {
        // three resident blocks per CU (50 KB of LDS each), persistent over the tiles;
        // the forward form (the statistic computed here) writes hqt for the backward
        // pass, the recomputation form for the backward product that follows it
        const int64_t tiles = ((F + kSqEdge - 1) / kSqEdge) * ((M + kSqEdge - 1) / kSqEdge);
        int64_t tblocks = tiles;
        if (tblocks > 3 * (int64_t)device_cu_count()) tblocks = 3 * (int64_t)device_cu_count();
        if (compute_absmax)
            return launch(swiglu_quant_t_kernel<true>, dim3((unsigned)tblocks), dim3(256), stream, g, M, F, absmax_h,
                          hq, hqt, inv_scale_h);
        return launch(swiglu_quant_t_kernel<false>, dim3((unsigned)tblocks), dim3(256), stream, g, M, F, absmax_h, hq,
                      hqt, inv_scale_h);
    }
    return launch(swiglu_quant_kernel, dim3((unsigned)blocks), dim3(256), stream, g, M, F, absmax_h, hq,
                  inv_scale_h);
}

// ---------------------------------------------------------------------------
// Block (MX) requantisation of the SwiGLU output: h in blocks of 32 consecutive
// features of a row, each with its own scale 2^e (e = floor(log2 max |h|) - 8,
// clamped at -127; E4M3 codes of h * 2^-e; a block with a NaN or an infinite h
// gets the NaN scale 255 and the unscaled encodings), following the OCP MX
// specification v1.0 (section 6.3) -- the block-scaled alternative of the LLMQ
// summary's section 2.  The block maximum is local to the block, so one pass
// does it all: no statistic pass over [gate | up] comes first.  The walk of
// swiglu_quant_kernel: lane l takes columns 8 l .. and 512 + 8 l .. of a
// 1024-column item, so a block is 4 adjacent lanes (DPP quad maximum); scales
// stored step-major ([F / 128][M][4]) like fp8_mx_quantize's.
__device__ __forceinline__ uint32_t quad_max_sw(uint32_t v)
{
    uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // lanes 1 0 3 2
    v = v > o ? v : o;
    o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);            // lanes 2 3 0 1
    return v > o ? v : o;
}

__global__ void __launch_bounds__(256) mx_swiglu_kernel(const uint16_t* __restrict__ gu, int64_t M, int64_t F,
                                                        uint8_t* __restrict__ hq, uint8_t* __restrict__ scales)
{
    __shared__ float tbl[kTable];
    load_table_to_lds(tbl);
    const RowItems it = row_items(M, F);
    const int lane = threadIdx.x & 63;
    for (int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); w < it.total; w += (int64_t)gridDim.x * 4) {
        const int64_t i = w / it.chunks;
        const int64_t jb = (w - i * it.chunks) * 1024 + lane * 8;
        const uint16_t* grow = gu + i * 2 * F;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int64_t j = jb + half * 512;
            if (j < F) {                  // F % 32 == 0: the 4 lanes of a block agree
                const uint4 gw = *reinterpret_cast<const uint4*>(grow + j);
                const uint4 uw = *reinterpret_cast<const uint4*>(grow + F + j);
                float h[8];
                swiglu8(tbl, gw, uw, h);
                // the largest magnitude pattern reaches 0x7F800000 exactly when a NaN or
                // an infinity occurs, and is the largest finite |h| otherwise
                const uint32_t m = quad_max_sw(mag_max8(0u, h));
                const bool bad = m >= 0x7F800000u;
                float sc = 1.0f;
                uint32_t sbyte = 255;
                if (!bad) {
                    // floor(log2 m): the exponent field of a normal fp32, the leading bit's
                    // position - 149 for a subnormal one
                    const int fl = m >= 0x00800000u ? (int)(m >> 23) - 127 : 31 - __builtin_clz(m | 1u) - 149;
                    int e = m ? fl - 8 : -127;
                    e = e < -127 ? -127 : e;                       // at most 119: no upper clamp
                    sc = __uint_as_float((uint32_t)(127 - e) << 23); // 2^-e
                    sbyte = (uint32_t)(e + 127);
                }
                uint2 c = quant8_h(h, sc);
                if (bad) {
                    // a NaN h takes the NaN code (S.1111111)
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        if (__builtin_isnan(h[k])) {
                            const uint32_t code = ((__float_as_uint(h[k]) >> 24) & 0x80u) | 0x7Fu;
                            const uint32_t sh = (uint32_t)(k & 3) * 8;
                            if (k < 4)
                                c.x = (c.x & ~(0xFFu << sh)) | (code << sh);
                            else
                                c.y = (c.y & ~(0xFFu << sh)) | (code << sh);
                        }
                    }
                }
                *reinterpret_cast<uint2*>(hq + i * F + j) = c;
                if ((lane & 3) == 0) {
                    const int64_t b = j / 32;                   // block b of row i, stored step-major
                    scales[((b >> 2) * M + i) * 4 + (b & 3)] = (uint8_t)sbyte;
                }
            }
        }
    }
}

hipError_t launch_mx_swiglu(const void* gu, int64_t M, int64_t F, uint8_t* hq, uint8_t* scales, hipStream_t stream)
{
    const int64_t items = M * ((F + 1023) / 1024);
    int64_t blocks = (items + 3) / 4;
    const int64_t cap = (int64_t)device_cu_count() * 4;   // 34 KB LDS per block: 4 blocks per CU
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    return launch(mx_swiglu_kernel, dim3((unsigned)blocks), dim3(256), stream, reinterpret_cast<const uint16_t*>(gu),
                  M, F, hq, scales);
}

// ---------------------------------------------------------------------------
// SwiGLU backward fused with the quantisation of [dg | du].

// dg, du for the 8 (gate, up, dh) triples of three 16-byte words.  ts / tds: the
// s_g and ds tables in LDS.
__device__ __forceinline__ void swiglu_grad8(const float* ts, const float* tds, uint4 gw, uint4 uw, uint4 dw,
                                             float dg[8], float du[8])
{
    const uint32_t g32[4] = {gw.x, gw.y, gw.z, gw.w};
    const uint32_t u32[4] = {uw.x, uw.y, uw.z, uw.w};
    const uint32_t d32[4] = {dw.x, dw.y, dw.z, dw.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const uint32_t b = hf ? (g32[k] >> 16) : (g32[k] & 0xFFFFu);
            const float g = hf ? bf16_hi(g32[k]) : bf16_lo(g32[k]);
            const float u = hf ? bf16_hi(u32[k]) : bf16_lo(u32[k]);
            const float d = hf ? bf16_hi(d32[k]) : bf16_lo(d32[k]);
            du[2 * k + hf] = d * silu_of(ts, b, g);
            const float p = d * u;
            dg[2 * k + hf] = p * dsilu_of(tds, b);
        }
    }
}

template <int FMT>
__device__ __forceinline__ uint2 quant8_f(const float v[8], float s)
{
    uint2 r;
    r.x = enc4<FMT>(v[0] * s, v[1] * s, v[2] * s, v[3] * s);
    r.y = enc4<FMT>(v[4] * s, v[5] * s, v[6] * s, v[7] * s);
    return r;
}

// Pass 1: absmax of [dg | du] over the whole [M, 2F] gradient (nothing written).
__global__ void __launch_bounds__(1024) swiglu_bwd_absmax_kernel(const uint16_t* __restrict__ gu,
                                                                const uint16_t* __restrict__ dh, int64_t M,
                                                                int64_t F, uint32_t* __restrict__ out)
{
    __shared__ float tbl[2 * kTable];
    load_tables_to_lds(tbl);
    const RowItems it = row_items(M, F);
    const int lane = threadIdx.x & 63;
    uint32_t m = 0;
    const int wpb = blockDim.x >> 6;
    for (int64_t w = (int64_t)blockIdx.x * wpb + (threadIdx.x >> 6); w < it.total; w += (int64_t)gridDim.x * wpb) {
        const int64_t i = w / it.chunks;
        const int64_t jb = (w - i * it.chunks) * 1024 + lane * 8;
        const uint16_t* grow = gu + i * 2 * F;
        const uint16_t* drow = dh + i * F;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int64_t j = jb + half * 512;
            if (j < F) {
                const uint4 gw = *reinterpret_cast<const uint4*>(grow + j);
                const uint4 uw = *reinterpret_cast<const uint4*>(grow + F + j);
                const uint4 dw = *reinterpret_cast<const uint4*>(drow + j);
                float dg[8], du[8];
                swiglu_grad8(tbl, tbl + kTable, gw, uw, dw, dg, du);
                m = mag_max8(mag_max8(m, dg), du);
            }
        }
    }
    block_max_to_global(m, out);
}

// Pass 2 without the transposed copy: q [M, 2F] = [codes of dg | codes of du].
template <int FMT>
__global__ void __launch_bounds__(256) swiglu_bwd_quant_kernel(const uint16_t* __restrict__ gu,
                                                               const uint16_t* __restrict__ dh, int64_t M, int64_t F,
                                                               const float* __restrict__ absmax,
                                                               uint8_t* __restrict__ q, float* __restrict__ scale_out,
                                                               float* __restrict__ inv_out)
{
    __shared__ float tbl[2 * kTable];
    float s, inv;
    tensor_scale(*absmax, Fmt<FMT>::max, s, inv);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (scale_out) *scale_out = s;
        if (inv_out) *inv_out = inv;
    }
    load_tables_to_lds(tbl);
    const RowItems it = row_items(M, F);
    const int lane = threadIdx.x & 63;
    for (int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); w < it.total; w += (int64_t)gridDim.x * 4) {
        const int64_t i = w / it.chunks;
        const int64_t jb = (w - i * it.chunks) * 1024 + lane * 8;
        const uint16_t* grow = gu + i * 2 * F;
        const uint16_t* drow = dh + i * F;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int64_t j = jb + half * 512;
            if (j < F) {
                const uint4 gw = *reinterpret_cast<const uint4*>(grow + j);
                const uint4 uw = *reinterpret_cast<const uint4*>(grow + F + j);
                const uint4 dw = *reinterpret_cast<const uint4*>(drow + j);
                float dg[8], du[8];
                swiglu_grad8(tbl, tbl + kTable, gw, uw, dw, dg, du);
                *reinterpret_cast<uint2*>(q + i * 2 * F + j) = quant8_f<FMT>(dg, s);
                *reinterpret_cast<uint2*>(q + i * 2 * F + F + j) = quant8_f<FMT>(du, s);
            }
        }
    }
}

// Pass 2 with the transposed copy qt [2F, M] (and optionally q).  The layout
// of the forward's transposed requant: a 4-wave group owns a 128 x 128 tile of
// (g, u, dh) and a lane its 8 x 8 block (24 loads, all issued first); the dg
// and du code blocks are transposed in registers and parked in two 16 KB LDS
// tiles laid out as qt rows j and F + j, then written back as full 128-byte
// rows.  A block is two such groups (512 threads, one copy of the two tables:
// 132 KB of LDS, one block per CU) taking two tiles per iteration, so both
// groups meet every barrier.  M and F are multiples of 16: blocks are whole.
template <int FMT>
__global__ void __launch_bounds__(512) swiglu_bwd_quant_t_kernel(const uint16_t* __restrict__ gu,
                                                                 const uint16_t* __restrict__ dh, int64_t M,
                                                                 int64_t F, const float* __restrict__ absmax,
                                                                 uint8_t* __restrict__ q, uint8_t* __restrict__ qt,
                                                                 float* __restrict__ scale_out,
                                                                 float* __restrict__ inv_out)
{
    __shared__ float tbl[2 * kTable];                                                   // 68 KB
    __shared__ __attribute__((aligned(16))) uint8_t tiles[2][2][kSqEdge * kSqEdge];     // [group][dg | du], 64 KB
    float s, inv;
    tensor_scale(*absmax, Fmt<FMT>::max, s, inv);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (scale_out) *scale_out = s;
        if (inv_out) *inv_out = inv;
    }
    load_tables_to_lds(tbl);
    const int grp = threadIdx.x >> 8, gt = threadIdx.x & 255;
    const int lane = gt & 63, wave = gt >> 6;
    const int rt = wave * 32 + (lane >> 4) * 8;           // first row of the lane within the tile
    const int ct = (lane & 15) * 8;                       // first column of the lane within the tile
    uint8_t* tg = tiles[grp][0];
    uint8_t* tu = tiles[grp][1];
    const int64_t ntc = (F + kSqEdge - 1) / kSqEdge;
    const int64_t ntiles = ntc * ((M + kSqEdge - 1) / kSqEdge);
    for (int64_t t0 = 2 * (int64_t)blockIdx.x; t0 < ntiles; t0 += 2 * (int64_t)gridDim.x) {
        const int64_t t = t0 + grp;
        const bool has = t < ntiles;
        const int64_t tr = has ? (t / ntc) * kSqEdge : 0, tc = has ? (t % ntc) * kSqEdge : 0;
        if (has && tr + rt < M && tc + ct < F) {
            const int64_t i0 = tr + rt, j = tc + ct;
            uint4 gw[8], uw[8], dw[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const uint16_t* grow = gu + (i0 + r) * 2 * F + j;
                gw[r] = *reinterpret_cast<const uint4*>(grow);
                uw[r] = *reinterpret_cast<const uint4*>(grow + F);
                dw[r] = *reinterpret_cast<const uint4*>(dh + (i0 + r) * F + j);
            }
            uint32_t glo[8], ghi[8], ulo[8], uhi[8];      // codes of dg (g...) and du (u...), per row
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                float dg[8], du[8];
                swiglu_grad8(tbl, tbl + kTable, gw[r], uw[r], dw[r], dg, du);
                const uint2 cg = quant8_f<FMT>(dg, s);
                const uint2 cu = quant8_f<FMT>(du, s);
                glo[r] = cg.x;
                ghi[r] = cg.y;
                ulo[r] = cu.x;
                uhi[r] = cu.y;
            }
            if (q) {
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    *reinterpret_cast<uint2*>(q + (i0 + r) * 2 * F + j) = make_uint2(glo[r], ghi[r]);
                    *reinterpret_cast<uint2*>(q + (i0 + r) * 2 * F + F + j) = make_uint2(ulo[r], uhi[r]);
                }
            }
            const int piece = rt >> 4, half = (rt >> 3) & 1;
            uint32_t c0[8], c1[8];
            transpose4x4(glo[0], glo[1], glo[2], glo[3], c0[0], c0[1], c0[2], c0[3]);
            transpose4x4(glo[4], glo[5], glo[6], glo[7], c1[0], c1[1], c1[2], c1[3]);
            transpose4x4(ghi[0], ghi[1], ghi[2], ghi[3], c0[4], c0[5], c0[6], c0[7]);
            transpose4x4(ghi[4], ghi[5], ghi[6], ghi[7], c1[4], c1[5], c1[6], c1[7]);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int col = ct + k;
                const int phys = piece ^ ((col >> 3) & 7);
                *reinterpret_cast<uint2*>(tg + col * kSqEdge + phys * 16 + half * 8) = make_uint2(c0[k], c1[k]);
            }
            transpose4x4(ulo[0], ulo[1], ulo[2], ulo[3], c0[0], c0[1], c0[2], c0[3]);
            transpose4x4(ulo[4], ulo[5], ulo[6], ulo[7], c1[0], c1[1], c1[2], c1[3]);
            transpose4x4(uhi[0], uhi[1], uhi[2], uhi[3], c0[4], c0[5], c0[6], c0[7]);
            transpose4x4(uhi[4], uhi[5], uhi[6], uhi[7], c1[4], c1[5], c1[6], c1[7]);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int col = ct + k;
                const int phys = piece ^ ((col >> 3) & 7);
                *reinterpret_cast<uint2*>(tu + col * kSqEdge + phys * 16 + half * 8) = make_uint2(c0[k], c1[k]);
            }
        }
        __syncthreads();
        // write-back of the group's two tiles: 2 x 1024 pieces of 16 bytes, 8 per
        // thread; a wave instruction covers 8 qt rows x 128 bytes
        if (has) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int id = u * 256 + gt;
                const int col = id >> 3, p = id & 7;
                const int64_t qrow = tc + col, qcol = tr + p * 16;
                if (qrow < F && qcol < M) {
                    const int phys = p ^ ((col >> 3) & 7);
                    *reinterpret_cast<uint4*>(qt + qrow * M + qcol) =
                        *reinterpret_cast<const uint4*>(tg + col * kSqEdge + phys * 16);
                    *reinterpret_cast<uint4*>(qt + (F + qrow) * M + qcol) =
                        *reinterpret_cast<const uint4*>(tu + col * kSqEdge + phys * 16);
                }
            }
        }
        __syncthreads();                                  // the tiles are read back before they are reused
    }
}

template <int FMT>
static hipError_t launch_swiglu_bwd_quant(const uint16_t* g, const uint16_t* d, int64_t M, int64_t F, float* absmax,
                                    uint8_t* q, uint8_t* qt, float* scale, float* inv_scale, hipStream_t stream)
{
    // two resident blocks per CU (2 x 34 KB tables each), persistent
    const int64_t cap = 2 * (int64_t)device_cu_count();
    if (qt) {
        // one 512-thread block per CU (132 KB of LDS), two tiles per iteration
        const int64_t tiles = ((F + kSqEdge - 1) / kSqEdge) * ((M + kSqEdge - 1) / kSqEdge);
        int64_t blocks = (tiles + 1) / 2;
        if (blocks > (int64_t)device_cu_count()) blocks = device_cu_count();
        return launch(swiglu_bwd_quant_t_kernel<FMT>, dim3((unsigned)blocks), dim3(512), stream, g, d, M, F, absmax,
                      q, qt, scale, inv_scale);
    } else {
        const int64_t items = M * ((F + 1023) / 1024);
        int64_t blocks = (items + 3) / 4;
        if (blocks > cap) blocks = cap;
        if (blocks < 1) blocks = 1;
        return launch(swiglu_bwd_quant_kernel<FMT>, dim3((unsigned)blocks), dim3(256), stream, g, d, M, F, absmax,
                      q, scale, inv_scale);
    }
}

hipError_t launch_swiglu_backward(const void* gu, const void* dh, int64_t M, int64_t F, int fmt, float* absmax,
                                  uint8_t* q, uint8_t* qt, float* scale, float* inv_scale, hipStream_t stream)
{
    const uint16_t* g = reinterpret_cast<const uint16_t*>(gu);
    const uint16_t* d = reinterpret_cast<const uint16_t*>(dh);
    hipError_t e = launch(zero_u32_kernel_sw, dim3(1), dim3(64), stream, reinterpret_cast<uint32_t*>(absmax));
    if (e != hipSuccess) return e;
    const int64_t items = M * ((F + 1023) / 1024);
    int64_t ablocks = (items + 15) / 16;
    if (ablocks > device_cu_count()) ablocks = device_cu_count();
    e = launch(swiglu_bwd_absmax_kernel, dim3((unsigned)ablocks), dim3(1024), stream, g, d, M, F,
               reinterpret_cast<uint32_t*>(absmax));
    if (e != hipSuccess) return e;
    if (fmt == 0) return launch_swiglu_bwd_quant<0>(g, d, M, F, absmax, q, qt, scale, inv_scale, stream);
    return launch_swiglu_bwd_quant<1>(g, d, M, F, absmax, q, qt, scale, inv_scale, stream);
}

}  // namespace fp8k
