// quant.hip -- absmax reduction and per-tensor FP8 quantisation for gfx950, and
// the block-scaled (MX) quantisations.
//
// Dynamic tensor-level scaling ("LLMQ: Efficient Lower-Precision Pretraining
// for Consumer GPUs", section 1; FastML report, FP8 training without delayed
// scaling): the scale of every tensor is derived from its own current absmax.
// Block scaling (the same summary's section 2; the OCP MX format): one scale
// per 32 consecutive elements along the reduction, no statistic pass.
//
// All kernels here are HBM-bound streaming kernels:
//   absmax      reads 2 B per element
//   quantize    reads 2 B, writes 1 B per element (+1 B with the transposed copy)
//   MX          reads 2 B, writes 1 + 1/32 B per element (codes and scales)
// They move data in 16-byte vectors, each wave instruction covering a
// contiguous 1 KB (loads) or 512 B (stores); the transposed MX form reads
// 256-byte row segments.
#include "fp8_device.hpp"
#include "fp8_internal.hpp"

namespace fp8k {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ us2 as_us2(uint32_t w) { return __builtin_bit_cast(us2, w); }

// |bf16| max of the 8 elements of a 16-byte word, accumulated as two packed
// 16-bit lanes (v_pk_max_u16 on the magnitude bits).
__device__ __forceinline__ us2 absmax_acc(us2 m, uint4 v)
{
    m = __builtin_elementwise_max(m, as_us2(v.x & 0x7FFF7FFFu));
    m = __builtin_elementwise_max(m, as_us2(v.y & 0x7FFF7FFFu));
    m = __builtin_elementwise_max(m, as_us2(v.z & 0x7FFF7FFFu));
    m = __builtin_elementwise_max(m, as_us2(v.w & 0x7FFF7FFFu));
    return m;
}

__global__ void __launch_bounds__(64) zero_u32_kernel(uint32_t* p)
{
    if (threadIdx.x == 0) *p = 0u;
}

// n words set to zero (the +0 start of n running statistics), one per lane.
__global__ void __launch_bounds__(256) zero_words_kernel(uint32_t* __restrict__ p, int n)
{
    const int i = (int)blockIdx.x * 256 + (int)threadIdx.x;
    if (i < n) p[i] = 0u;
}

// One pass over x; each block folds its maximum into *out with one atomicMax on
// the fp32 bit pattern (for non-negative values the unsigned order of the bits
// is the numeric order, and NaN patterns sort above infinity).  One block of 16
// waves per CU; every lane keeps kAbsUnroll 16-byte loads in flight.  Tensors of at
// least kAbsStreamBytes are read with non-temporal loads: measured on MI355X
// (7B-layer shapes), that makes the pass ~30% faster on 90-180 MB tensors at a
// small cost to the quantise pass that follows; below that size the plain
// loads leave the tensor in the 256 MB Infinity Cache, where the quantise pass
// re-reads it about twice as fast as from HBM.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ us2 absmax_acc4(us2 m, u32x4 v)
{
    return absmax_acc(m, make_uint4(v.x, v.y, v.z, v.w));
}

constexpr int kAbsThreads = 1024;
// Loads in flight per lane: 2 x 16 B x 1024 lanes x 256 CUs = 8 MiB for the
// whole chip.  Measured with a cold Infinity Cache, plain streaming reads on
// MI355X peak at about 8 MiB in flight (7.0 TB/s over 1 GiB) and fall to
// 5.5-6.5 TB/s at 16-32 MiB; with 8 loads per lane the 90-180 MB statistics ran
// 6-10% slower.
constexpr int kAbsUnroll = 2;
constexpr int64_t kAbsStreamBytes = 64ll << 20;

template <bool NT>
__device__ __forceinline__ u32x4 ld16(const u32x4* p)
{
    if (NT) return __builtin_nontemporal_load(p);
    return *p;
}

// The pass of block `blk` of `nblk` over one tensor (nvec 16-byte vectors and
// ntail trailing elements, which block 0 takes).
template <bool NT>
__device__ __forceinline__ void absmax_body(const u32x4* __restrict__ x, int64_t nvec,
                                            const uint16_t* __restrict__ tail, int ntail, uint32_t* __restrict__ out,
                                            int blk, int nblk)
{
    us2 m = {0, 0};
    const int64_t stride = (int64_t)nblk * kAbsThreads;
    int64_t i = (int64_t)blk * kAbsThreads + threadIdx.x;
    for (; i + (kAbsUnroll - 1) * stride < nvec; i += kAbsUnroll * stride) {
        u32x4 v[kAbsUnroll];
#pragma unroll
        for (int u = 0; u < kAbsUnroll; ++u) v[u] = ld16<NT>(x + i + u * stride);
#pragma unroll
        for (int u = 0; u < kAbsUnroll; ++u) m = absmax_acc4(m, v[u]);
    }
    for (; i < nvec; i += stride) m = absmax_acc4(m, ld16<NT>(x + i));
    uint32_t r = m.x > m.y ? m.x : m.y;
    if (blk == 0 && (int)threadIdx.x < ntail) {
        uint32_t t = tail[threadIdx.x] & 0x7FFFu;
        r = r > t ? r : t;
    }
    block_max_to_global(r << 16, out);
}

template <bool NT>
__global__ void __launch_bounds__(kAbsThreads) absmax_bf16_kernel(const u32x4* __restrict__ x, int64_t nvec,
                                                                  const uint16_t* __restrict__ tail, int ntail,
                                                                  uint32_t* __restrict__ out)
{
    absmax_body<NT>(x, nvec, tail, ntail, out, blockIdx.x, gridDim.x);
}

// Several tensors in one launch: blocks first[i] .. first[i + 1] - 1 take tensor i.
struct AbsmaxGroup {
    const u32x4* x[kMaxAbsTensors];
    const uint16_t* tail[kMaxAbsTensors];
    uint32_t* out[kMaxAbsTensors];
    int64_t nvec[kMaxAbsTensors];
    int ntail[kMaxAbsTensors];
    int nt[kMaxAbsTensors];                   // non-temporal loads for this tensor
    int first[kMaxAbsTensors + 1];
    int count;
};

__global__ void __launch_bounds__(kAbsThreads) absmax_many_kernel(const AbsmaxGroup g)
{
    int i = 0;
    while (i + 1 < g.count && (int)blockIdx.x >= g.first[i + 1]) ++i;
    const int blk = blockIdx.x - g.first[i], nblk = g.first[i + 1] - g.first[i];
    if (g.nt[i])
        absmax_body<true>(g.x[i], g.nvec[i], g.tail[i], g.ntail[i], g.out[i], blk, nblk);
    else
        absmax_body<false>(g.x[i], g.nvec[i], g.tail[i], g.ntail[i], g.out[i], blk, nblk);
}

hipError_t launch_absmax_many(int count, const void* const* x, const int64_t* n, float* const* absmax,
                              hipStream_t stream)
{
    AbsmaxGroup g;
    g.count = count;
    // one load form for the whole launch, chosen by its largest tensor (non-temporal
    // when that one is 64 MiB or more): blocks of mixed forms ran slower together
    // than the two tensors did in launches of their own (measured)
    int64_t total = 0, largest = 0;
    for (int i = 0; i < count; ++i) {
        total += n[i];
        largest = n[i] > largest ? n[i] : largest;
    }
    const bool nt = 2 * largest >= kAbsStreamBytes;
    // blocks in proportion to the sizes (at least one per tensor), about one per CU
    // in all, each at most what its tensor fills (8 vectors per lane)
    const int64_t cus = device_cu_count();
    g.first[0] = 0;
    for (int i = 0; i < count; ++i) {
        const int64_t nvec = n[i] / 8;
        g.x[i] = reinterpret_cast<const u32x4*>(x[i]);
        g.nvec[i] = nvec;
        g.ntail[i] = (int)(n[i] - nvec * 8);
        g.tail[i] = reinterpret_cast<const uint16_t*>(x[i]) + nvec * 8;
        g.out[i] = reinterpret_cast<uint32_t*>(absmax[i]);
        g.nt[i] = nt;
        int64_t b = (cus * n[i] + total - 1) / total;
        const int64_t need = (nvec + 8 * kAbsThreads - 1) / (8 * kAbsThreads);
        if (b > need) b = need;
        if (b < 1) b = 1;
        g.first[i + 1] = g.first[i] + (int)b;
    }
    return launch(absmax_many_kernel, dim3((unsigned)g.first[count]), dim3(kAbsThreads), stream, g);
}

hipError_t launch_absmax_clear(float* absmax, int64_t count, hipStream_t stream)
{
    return launch(zero_words_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), stream,
                  reinterpret_cast<uint32_t*>(absmax), (int)count);
}

hipError_t launch_absmax_bf16(const void* x, int64_t n, float* absmax, bool accumulate, hipStream_t stream)
{
    const int64_t nvec = n / 8;
    const int ntail = (int)(n - nvec * 8);
    int64_t blocks = (nvec + 8 * kAbsThreads - 1) / (8 * kAbsThreads);   // up to 8 vectors per thread
    const int64_t cap = (int64_t)device_cu_count();  // one block per CU (one atomic per block)
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    const uint16_t* tail = reinterpret_cast<const uint16_t*>(x) + nvec * 8;
    uint32_t* out = reinterpret_cast<uint32_t*>(absmax);
    if (!accumulate) {
        const hipError_t e = launch(zero_u32_kernel, dim3(1), dim3(64), stream, out);
        if (e != hipSuccess) return e;
    }
    if (2 * n >= kAbsStreamBytes)
        return launch(absmax_bf16_kernel<true>, dim3((unsigned)blocks), dim3(kAbsThreads), stream, xv, nvec, tail,
                      ntail, out);
    return launch(absmax_bf16_kernel<false>, dim3((unsigned)blocks), dim3(kAbsThreads), stream, xv, nvec, tail,
                  ntail, out);
}

// ---------------------------------------------------------------------------
// Quantisation without a transposed copy.  A wave tile is 1024 consecutive
// elements (128 16-byte vectors): lane l converts vectors l and l + 64, so
// every load instruction reads 1 KB and every store writes 512 B contiguously.
template <int FMT>
__global__ void __launch_bounds__(256) quantize_flat_kernel(const uint4* __restrict__ x, int64_t nvec,
                                                            const float* __restrict__ absmax,
                                                            uint2* __restrict__ q,
                                                            float* __restrict__ scale_out,
                                                            float* __restrict__ inv_out)
{
    float s, inv;
    tensor_scale(*absmax, Fmt<FMT>::max, s, inv);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (scale_out) *scale_out = s;
        if (inv_out) *inv_out = inv;
    }
    const int lane = threadIdx.x & 63;
    const int64_t ntiles = (nvec + 127) / 128;
    const int64_t wstride = (int64_t)gridDim.x * 4;
    for (int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); t < ntiles; t += 2 * wstride) {
        const int64_t t2 = t + wstride;
        const int64_t v0 = t * 128 + lane, v1 = v0 + 64;
        const int64_t v2 = t2 * 128 + lane, v3 = v2 + 64;
        uint4 a = {0, 0, 0, 0}, b = a, c = a, d = a;
        if (v0 < nvec) a = x[v0];
        if (v1 < nvec) b = x[v1];
        if (t2 < ntiles) {
            if (v2 < nvec) c = x[v2];
            if (v3 < nvec) d = x[v3];
        }
        if (v0 < nvec) q[v0] = quant8<FMT>(a, s);
        if (v1 < nvec) q[v1] = quant8<FMT>(b, s);
        if (t2 < ntiles) {
            if (v2 < nvec) q[v2] = quant8<FMT>(c, s);
            if (v3 < nvec) q[v3] = quant8<FMT>(d, s);
        }
    }
}

// ---------------------------------------------------------------------------
// Quantisation with the transposed copy (and optionally the plain one).  A block
// of 4 waves owns a 128 x 128 tile.  Lane l of wave w converts the 16-byte
// vectors of 8 consecutive rows (w * 32 + (l / 16) * 8 ..) at columns
// 8 (l % 16) .. +7: every load instruction reads four 256-byte row segments,
// every q store writes four 128-byte segments.  The lane transposes its 8 x 8
// code block in registers (v_perm_b32) into 8 column pieces of 8 bytes and parks
// them in an LDS tile laid out as qt ([128 columns][128 rows], 16-byte pieces
// XOR-swizzled by column); after a barrier the block writes qt back as full
// 128-byte row segments.  Measured on MI355X against a 128 x 256 tile (16 rows
// per lane): 4096 x 4096 15.0 -> 14.0 us, 4096 x 11008 36.9 -> 35.1 us, the
// 7B-layer step's quantisations 318 -> 314 us -- twice the blocks, so a small
// tensor fills more of each CU and the blocks' load and store phases overlap.
constexpr int kQtEdge = 128;

// The 128 x 128 tile with origin (tr, tc) of one tensor: q (if given) and qt
// (if given; with qt == nullptr the LDS tile and its barrier are skipped, a
// uniform choice per tensor).  NT: non-temporal loads of x.  NTQ: qt written
// with non-temporal stores (a copy that is read later -- by the backward pass --
// and not by the next call; a compile-time choice, so the hint cannot be lost).
template <int FMT, bool NT, bool NTQ = false>
__device__ __forceinline__ void quantize_tile(const uint8_t* __restrict__ x, int64_t rows, int64_t cols, float s,
                                              uint8_t* __restrict__ q, uint8_t* __restrict__ qt, int64_t tr,
                                              int64_t tc, uint8_t* tile)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rt = wave * 32 + (lane >> 4) * 8;           // first row of the lane within the tile
    const int ct = (lane & 15) * 8;                       // first column of the lane within the tile
    // rows and cols are multiples of 16, rt and ct of 8: an active lane's 8 x 8 block is inside
    if (tr + rt < rows && tc + ct < cols) {
        const int64_t i0 = tr + rt, j = tc + ct;
        uint4 v[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const u32x4* src = reinterpret_cast<const u32x4*>(x + ((i0 + r) * cols + j) * 2);
            const u32x4 w = NT ? __builtin_nontemporal_load(src) : *src;
            v[r] = make_uint4(w.x, w.y, w.z, w.w);
        }
        uint32_t lo[8], hi[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const uint2 c = quant8<FMT>(v[r], s);
            lo[r] = c.x;
            hi[r] = c.y;
        }
        if (q) {
#pragma unroll
            for (int r = 0; r < 8; ++r)
                *reinterpret_cast<uint2*>(q + (i0 + r) * cols + j) = make_uint2(lo[r], hi[r]);
        }
        if (qt) {
            // column k of the block: rows 0..3 (word 0) and rows 4..7 (word 1)
            uint32_t c0[8], c1[8];
            transpose4x4(lo[0], lo[1], lo[2], lo[3], c0[0], c0[1], c0[2], c0[3]);
            transpose4x4(lo[4], lo[5], lo[6], lo[7], c1[0], c1[1], c1[2], c1[3]);
            transpose4x4(hi[0], hi[1], hi[2], hi[3], c0[4], c0[5], c0[6], c0[7]);
            transpose4x4(hi[4], hi[5], hi[6], hi[7], c1[4], c1[5], c1[6], c1[7]);
            const int piece = rt >> 4, half = (rt >> 3) & 1;   // 8-byte half of a 16-byte piece of the qt row
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int col = ct + k;
                const int phys = piece ^ ((col >> 3) & 7);
                *reinterpret_cast<uint2*>(tile + col * kQtEdge + phys * 16 + half * 8) = make_uint2(c0[k], c1[k]);
            }
        }
    }
    if (!qt) return;
    __syncthreads();
    // write-back: 1024 pieces of 16 bytes, 4 per thread; a wave instruction
    // covers 8 qt rows x 128 bytes
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int id = u * 256 + threadIdx.x;
        const int col = id >> 3, p = id & 7;
        const int64_t qrow = tc + col, qcol = tr + p * 16;
        if (qrow < cols && qcol < rows) {
            const int phys = p ^ ((col >> 3) & 7);
            const u32x4 piece16 = *reinterpret_cast<const u32x4*>(tile + col * kQtEdge + phys * 16);
            u32x4* dst = reinterpret_cast<u32x4*>(qt + qrow * rows + qcol);
            if (NTQ)
                __builtin_nontemporal_store(piece16, dst);
            else
                *dst = piece16;
        }
    }
}

template <int FMT, bool NT>
__global__ void __launch_bounds__(256) quantize_t_kernel(const uint8_t* __restrict__ x, int64_t rows,
                                                         int64_t cols, const float* __restrict__ absmax,
                                                         uint8_t* __restrict__ q, uint8_t* __restrict__ qt,
                                                         float* __restrict__ scale_out,
                                                         float* __restrict__ inv_out)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[kQtEdge * kQtEdge];    // 16 KB
    float s, inv;
    tensor_scale(*absmax, Fmt<FMT>::max, s, inv);
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
        if (scale_out) *scale_out = s;
        if (inv_out) *inv_out = inv;
    }
    quantize_tile<FMT, NT>(x, rows, cols, s, q, qt, (int64_t)blockIdx.y * kQtEdge, (int64_t)blockIdx.x * kQtEdge,
                           tile);
}

// Several tensors in one launch (each exactly as its own fp8_quantize call with
// the tile kernel): the blocks first[i] .. first[i + 1] - 1 are the 128 x 128
// tiles of tensor i, column tile fastest, as the grid of the single-tensor
// launch orders them.  The format and the load form are per tensor (uniform
// within a block).
struct QuantGroup {
    const uint8_t* x[kMaxQuantTensors];
    const float* absmax[kMaxQuantTensors];
    uint8_t* q[kMaxQuantTensors];
    uint8_t* qt[kMaxQuantTensors];
    float* scale[kMaxQuantTensors];
    float* inv[kMaxQuantTensors];
    int64_t rows[kMaxQuantTensors];
    int64_t cols[kMaxQuantTensors];
    int tiles_c[kMaxQuantTensors];
    int fmt[kMaxQuantTensors];
    int nt[kMaxQuantTensors];
    int first[kMaxQuantTensors + 1];
    int count;
};

template <int FMT, bool NTQ>
__device__ __forceinline__ void quantize_group_tile(const QuantGroup& g, int i, int64_t tr, int64_t tc, uint8_t* tile)
{
    float s, inv;
    tensor_scale(*g.absmax[i], Fmt<FMT>::max, s, inv);
    if (tr == 0 && tc == 0 && threadIdx.x == 0) {
        if (g.scale[i]) *g.scale[i] = s;
        if (g.inv[i]) *g.inv[i] = inv;
    }
    if (g.nt[i])
        quantize_tile<FMT, true, NTQ>(g.x[i], g.rows[i], g.cols[i], s, g.q[i], g.qt[i], tr, tc, tile);
    else
        quantize_tile<FMT, false, NTQ>(g.x[i], g.rows[i], g.cols[i], s, g.q[i], g.qt[i], tr, tc, tile);
}

// NTQ: every qt of the launch is read later (non-temporal stores); a launch
// quantises tensors of one kind only, so the hint is fixed at compile time.
template <bool NTQ>
__global__ void __launch_bounds__(256) quantize_many_kernel(const QuantGroup g)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[kQtEdge * kQtEdge];    // 16 KB
    int i = 0;
    while (i + 1 < g.count && (int)blockIdx.x >= g.first[i + 1]) ++i;
    const int t = blockIdx.x - g.first[i];
    const int64_t tr = (int64_t)(t / g.tiles_c[i]) * kQtEdge, tc = (int64_t)(t % g.tiles_c[i]) * kQtEdge;
    if (g.fmt[i] == 0)
        quantize_group_tile<0, NTQ>(g, i, tr, tc, tile);
    else
        quantize_group_tile<1, NTQ>(g, i, tr, tc, tile);
}

static hipError_t launch_quantize_group(int count, const int* idx, const void* const* x, const int64_t* rows,
                                        const int64_t* cols, const int* fmt, const float* const* absmax,
                                        uint8_t* const* q, uint8_t* const* qt, float* const* scale,
                                        float* const* inv_scale, bool ntq, hipStream_t stream)
{
    QuantGroup g;
    g.count = count;
    g.first[0] = 0;
    for (int k = 0; k < count; ++k) {
        const int i = idx[k];
        g.x[k] = reinterpret_cast<const uint8_t*>(x[i]);
        g.absmax[k] = absmax[i];
        g.q[k] = q[i];
        g.qt[k] = qt[i];
        g.scale[k] = scale[i];
        g.inv[k] = inv_scale[i];
        g.rows[k] = rows[i];
        g.cols[k] = cols[i];
        g.fmt[k] = fmt[i];
        // as the single-tensor launch: inputs of 64 MiB or more are read non-temporally
        g.nt[k] = 2 * rows[i] * cols[i] >= kAbsStreamBytes;
        g.tiles_c[k] = (int)((cols[i] + kQtEdge - 1) / kQtEdge);
        const int64_t tiles = (int64_t)g.tiles_c[k] * ((rows[i] + kQtEdge - 1) / kQtEdge);
        g.first[k + 1] = g.first[k] + (int)tiles;
    }
    if (ntq) return launch(quantize_many_kernel<true>, dim3((unsigned)g.first[count]), dim3(256), stream, g);
    return launch(quantize_many_kernel<false>, dim3((unsigned)g.first[count]), dim3(256), stream, g);
}

// Tensors whose qt is read later and those whose qt (or none) is read next go to
// separate launches (one launch when all are of one kind).
hipError_t launch_quantize_many(int count, const void* const* x, const int64_t* rows, const int64_t* cols,
                                const int* fmt, const float* const* absmax, uint8_t* const* q, uint8_t* const* qt,
                                float* const* scale, float* const* inv_scale, const int* qt_later,
                                hipStream_t stream)
{
    int later[kMaxQuantTensors], next[kMaxQuantTensors], nl = 0, nn = 0;
    for (int i = 0; i < count; ++i) {
        if (qt_later && qt_later[i] && qt[i])
            later[nl++] = i;
        else
            next[nn++] = i;
    }
    if (nl > 0) {
        const hipError_t e = launch_quantize_group(nl, later, x, rows, cols, fmt, absmax, q, qt, scale, inv_scale,
                                                   true, stream);
        if (e != hipSuccess || nn == 0) return e;
    }
    return launch_quantize_group(nn, next, x, rows, cols, fmt, absmax, q, qt, scale, inv_scale, false, stream);
}

// Plain quantisation only: the flat kernel above; with qt: the tile kernel.
template <int FMT>
static hipError_t launch_quantize_fmt(const void* x, int64_t rows, int64_t cols, const float* absmax,
                                uint8_t* q, uint8_t* qt, float* scale, float* inv_scale,
                                hipStream_t stream)
{
    if (qt) {
        dim3 grid((unsigned)((cols + kQtEdge - 1) / kQtEdge), (unsigned)((rows + kQtEdge - 1) / kQtEdge));
        // a large input is read non-temporally: nothing reads it again, and the
        // Infinity Cache is left to the codes the GEMMs read next
        if (2 * rows * cols >= kAbsStreamBytes)
            return launch(quantize_t_kernel<FMT, true>, grid, dim3(256), stream, reinterpret_cast<const uint8_t*>(x),
                          rows, cols, absmax, q, qt, scale, inv_scale);
        return launch(quantize_t_kernel<FMT, false>, grid, dim3(256), stream, reinterpret_cast<const uint8_t*>(x),
                      rows, cols, absmax, q, qt, scale, inv_scale);
    } else {
        const int64_t nvec = rows * cols / 8;
        const int64_t ntiles = (nvec + 127) / 128;
        int64_t blocks = (ntiles + 7) / 8;          // two wave tiles per wave per pass
        const int64_t cap = (int64_t)device_cu_count() * 8;
        if (blocks > cap) blocks = cap;
        if (blocks < 1) blocks = 1;
        return launch(quantize_flat_kernel<FMT>, dim3((unsigned)blocks), dim3(256), stream,
                      reinterpret_cast<const uint4*>(x), nvec, absmax, reinterpret_cast<uint2*>(q), scale, inv_scale);
    }
}

hipError_t launch_quantize(const void* x, int64_t rows, int64_t cols, int fmt, const float* absmax,
                           uint8_t* q, uint8_t* qt, float* scale, float* inv_scale, hipStream_t stream)
{
    if (fmt == 0) return launch_quantize_fmt<0>(x, rows, cols, absmax, q, qt, scale, inv_scale, stream);
    return launch_quantize_fmt<1>(x, rows, cols, absmax, q, qt, scale, inv_scale, stream);
}

// ---------------------------------------------------------------------------
// Block (MX) quantisation: the alternative to the per-tensor scale that the LLMQ
// summary (section 2) says needs native hardware support, as gfx950's
// block-scaled matrix instructions provide.  Following the OCP Microscaling
// (MX) formats specification v1.0 (section 6.3): every 32 consecutive elements
// of a row share the scale 2^e, e = floor(log2 max |x|) - emax (emax = 8 for
// E4M3, 15 for E5M2: the exponent of the format's largest normal), clamped to
// [-127, 127] (-127 for an all-zero block), stored as the E8M0 byte e + 127;
// the elements are x * 2^-e (exact) encoded like every other value (nearest
// even, saturating).  A block holding a NaN or an infinity gets the NaN scale
// (255) and the unscaled encodings.  One pass, no statistic launch before it:
// reads 2 B and writes 1 + 1/32 B per element.  The scales are stored
// step-major, [cols / 128][rows][4] (the four blocks of a 128-element
// reduction step of every row together), the layout the block-scaled GEMM
// loads contiguously.
//
// Lane l converts the 16-byte vectors v (8 elements each); the 4 lanes of a
// block are 4 consecutive lanes (v % 4 == l % 4: the grid stride is a multiple
// of 4, and the element count one of 32), so the block's maximum takes two
// shuffles, and the 4 lanes leave every loop together.  NT: non-temporal loads
// (large inputs).
// Saturate and encode four fp32 values (finite or infinite; a NaN reaches the
// converter as a bound and its code is replaced by the caller).
template <int FMT>
__device__ __forceinline__ uint32_t mx_enc4(float a, float b, float c, float d)
{
    constexpr float mx = Fmt<FMT>::max;
    a = __builtin_amdgcn_fmed3f(a, -mx, mx);
    b = __builtin_amdgcn_fmed3f(b, -mx, mx);
    c = __builtin_amdgcn_fmed3f(c, -mx, mx);
    d = __builtin_amdgcn_fmed3f(d, -mx, mx);
    if (FMT == 0) {
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
        return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
    }
    const int lo = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c, d, lo, true);
}

// Max over the 4 lanes of a block (lanes 4 j .. 4 j + 3) through DPP quad permutes.
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v)
{
    uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // lanes 1 0 3 2
    v = v > o ? v : o;
    o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);            // lanes 2 3 0 1
    return v > o ? v : o;
}

// One 16-byte vector of 8 elements: its share of the block maximum is combined
// over the block's 4 lanes, then the codes are written.  The maximum is taken
// over all magnitude bit patterns: it reaches 0x7F80 exactly when the block
// holds an infinity or a NaN, and is the largest finite magnitude otherwise.
template <int FMT>
__device__ __forceinline__ void mx_vector(const u32x4 w, int64_t v, uint2* __restrict__ q, uint8_t* __restrict__ scales,
                                          uint32_t rows, uint32_t nb)
{
    constexpr int emax = FMT == 0 ? 8 : 15;
    us2 m2 = {0, 0};
    m2 = absmax_acc(m2, make_uint4(w.x, w.y, w.z, w.w));
    const uint32_t m = quad_max_u32(m2.x > m2.y ? m2.x : m2.y);
    const bool bad = m >= 0x7F80u;
    float s = 1.0f;                       // a block with a NaN or an infinity: unscaled
    uint32_t sbyte = 255;
    if (!bad) {
        // floor(log2 m): the exponent field of a normal bf16; m * 2^-133 for a subnormal one
        const int fl = m >= 0x80u ? (int)(m >> 7) - 127 : 31 - __builtin_clz(m | 1u) - 133;
        int e = m ? fl - emax : -127;
        e = e < -127 ? -127 : e;          // at most 127 - emax: no upper clamp is reached
        s = __uint_as_float((uint32_t)(127 - e) << 23);           // 2^-e, a normal fp32
        sbyte = (uint32_t)(e + 127);
    }
    uint2 c;
    c.x = mx_enc4<FMT>(bf16_lo(w.x) * s, bf16_hi(w.x) * s, bf16_lo(w.y) * s, bf16_hi(w.y) * s);
    c.y = mx_enc4<FMT>(bf16_lo(w.z) * s, bf16_hi(w.z) * s, bf16_lo(w.w) * s, bf16_hi(w.w) * s);
    if (bad) {
        // a NaN element takes the NaN code with its sign (S.1111111)
        const uint32_t hw[8] = {w.x & 0xFFFFu, w.x >> 16, w.y & 0xFFFFu, w.y >> 16,
                                w.z & 0xFFFFu, w.z >> 16, w.w & 0xFFFFu, w.w >> 16};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if ((hw[i] & 0x7FFFu) > 0x7F80u) {
                const uint32_t code = ((hw[i] >> 8) & 0x80u) | 0x7Fu, sh = (uint32_t)(i & 3) * 8;
                if (i < 4)
                    c.x = (c.x & ~(0xFFu << sh)) | (code << sh);
                else
                    c.y = (c.y & ~(0xFFu << sh)) | (code << sh);
            }
        }
    }
    q[v] = c;
    if ((threadIdx.x & 3) == 0) {
        // block f = i nb + b of row i: stored step-major at ((b / 4) rows + i) 4 + b % 4
        const uint32_t f = (uint32_t)(v >> 2), i = f / nb, b = f - i * nb;
        scales[((size_t)(b >> 2) * rows + i) * 4 + (b & 3)] = (uint8_t)sbyte;
    }
}

// A plain grid-stride loop, one 16-byte load per lane and pass, eight 256-lane
// blocks per CU (32 waves): measured on MI355X (cold, 7B-layer tensors of
// 90-180 MB) 4.8-5.2 TB/s against 4.4-4.7 with 4 blocks per CU, 3.3-3.5 with 2,
// and no better with two or four loads per lane issued ahead.
template <int FMT, bool NT>
__global__ void __launch_bounds__(256) mx_quantize_kernel(const u32x4* __restrict__ x, int64_t nvec,
                                                          uint2* __restrict__ q, uint8_t* __restrict__ scales,
                                                          uint32_t rows, uint32_t nb)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < nvec; v += stride)
        mx_vector<FMT>(NT ? __builtin_nontemporal_load(x + v) : x[v], v, q, scales, rows, nb);
}

// The block scale 2^-e and its E8M0 byte for a block's largest magnitude bit
// pattern m (bf16 bits; >= 0x7F80: an infinity or a NaN -- unscaled, byte 255).
template <int FMT>
__device__ __forceinline__ float mx_scale_of(uint32_t m, uint32_t& sbyte)
{
    constexpr int emax = FMT == 0 ? 8 : 15;
    if (m >= 0x7F80u) {
        sbyte = 255;
        return 1.0f;
    }
    const int fl = m >= 0x80u ? (int)(m >> 7) - 127 : 31 - __builtin_clz(m | 1u) - 133;
    int e = m ? fl - emax : -127;
    e = e < -127 ? -127 : e;
    sbyte = (uint32_t)(e + 127);
    return __uint_as_float((uint32_t)(127 - e) << 23);
}

// Two codes (bytes 0, 1) of two bf16 values under one block scale; a NaN takes
// the NaN code with its sign.
template <int FMT>
__device__ __forceinline__ uint32_t mx_code2(uint32_t h0, uint32_t h1, float s)
{
    constexpr float mx = Fmt<FMT>::max;
    const float a = __builtin_amdgcn_fmed3f(__uint_as_float(h0 << 16) * s, -mx, mx);
    const float b = __builtin_amdgcn_fmed3f(__uint_as_float(h1 << 16) * s, -mx, mx);
    uint32_t c = FMT == 0 ? (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)
                          : (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    if ((h0 & 0x7FFFu) > 0x7F80u) c = (c & 0xFF00u) | ((h0 >> 8) & 0x80u) | 0x7Fu;
    if ((h1 & 0x7FFFu) > 0x7F80u) c = (c & 0x00FFu) | ((((h1 >> 8) & 0x80u) | 0x7Fu) << 8);
    return c & 0xFFFFu;
}

// The scaled conversion of gfx950 (v_cvt_scalef32_pk_{fp8,bf8}_bf16): two bf16
// values divided by the power of two whose fp32 exponent field is that of the
// scale operand, rounded to nearest-even into the format; an E8M0 byte b is
// passed as the fp32 bits b << 23 (b = 0 acts as 2^-127).  Checked against the
// encoder for every bf16 value under every byte 0..254: exact, subnormal results
// included, except that it does not saturate (a result past the largest finite
// value becomes NaN for E4M3, infinity for E5M2) -- so magnitudes are clamped
// first, below.  Four codes: w0's pair in bytes 0, 1 and w1's in bytes 2, 3.
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int FMT>
__device__ __forceinline__ uint32_t mx_cvt4(uint32_t w0, uint32_t w1, float s)
{
    const s16x2 z = {0, 0};
    const bf16x2 a = __builtin_bit_cast(bf16x2, w0), b = __builtin_bit_cast(bf16x2, w1);
    s16x2 r;
    if (FMT == 0) {
        r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(z, a, s, false);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, b, s, true);
    } else {
        r = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(z, a, s, false);
        r = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(r, b, s, true);
    }
    return __builtin_bit_cast(uint32_t, r);
}

// For a finite block with largest magnitude pattern m (< 0x7F80): the E8M0 byte
// e + 127 = max(exponent field of m - emax, 0) -- a subnormal or zero maximum
// gives e = -127 either way -- and the clamp limit: the largest bf16 magnitude
// that still rounds to the format's largest finite value under 2^-e (464 2^e for
// E4M3, whose tie at 464 goes to the even 448; just below 61440 2^e for E5M2,
// whose tie goes up).  Both packed into the two 16-bit halves.
template <int FMT>
__device__ __forceinline__ uint32_t mx_fast_scale(uint32_t m, uint32_t& limit2)
{
    constexpr int emax = FMT == 0 ? 8 : 15;
    constexpr uint32_t frac = FMT == 0 ? 0x68u : 0x6Fu;
    const int b = (int)(m >> 7) - emax;
    const uint32_t sbyte = (uint32_t)(b > 0 ? b : 0);
    const uint32_t lim = ((sbyte + emax) << 7) | frac;
    limit2 = lim | (lim << 16);
    return sbyte;
}

// Clamp both bf16 of w to magnitude limit (packed per half), keeping the signs.
__device__ __forceinline__ uint32_t mx_clamp2(uint32_t w, uint32_t a, uint32_t limit2)
{
    const uint32_t c = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(as_us2(a), as_us2(limit2)));
    return (c & 0x7FFF7FFFu) | (w & 0x80008000u);
}

// Both block quantisations of x in one read: q [rows, cols] with blocks along
// the rows (the forward operand) and qt [cols, rows] with blocks along the
// columns (the backward operand), each with its own step-major scales -- the
// bytes of fp8_mx_quantize and of fp8_mx_quantize_t.  A 256-thread block takes
// a 128 x 128 tile, each wave 32 rows of it, each lane an 8 x 8 piece: rows
// 8 (l & 3) .. + 7 of the wave's, columns 8 (l >> 2) .. + 7 (one 16-byte load
// per row).  A column block (32 rows) is then the 4 lanes of a quad and a row
// block (32 columns) the lanes l, l ^ 4, ... of one 16-lane DPP row, so both
// maxima take two DPP steps.  The row codes go straight to q (a wave store
// covers 4 rows x 128 bytes); the column codes are staged in LDS as qt rows and
// written out as 128-byte row segments, as are both tiles' 512 scale bytes.
// Tiles holding an infinity or a NaN take the generic per-element rule
// (per wave: blocks never cross waves).
template <int FMT, bool NT>
__global__ void __launch_bounds__(256) mx_quantize_both_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                               int64_t cols, uint8_t* __restrict__ q,
                                                               uint32_t* __restrict__ sq, uint8_t* __restrict__ qt,
                                                               uint32_t* __restrict__ sqt)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[kQtEdge * kQtEdge];    // qt rows of the tile
    __shared__ uint32_t srow[kQtEdge], scol[kQtEdge];                           // the tile's scale bytes
    uint8_t* const sr = reinterpret_cast<uint8_t*>(srow);
    uint8_t* const sc = reinterpret_cast<uint8_t*>(scol);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rq = lane & 3, g = lane >> 2;          // row group (8 rows), column group (8 columns)
    const int rt = wave * 32 + 8 * rq;               // the lane's first row within the tile
    // qt piece of this lane's 8 rows in LDS: qt row col holds 8 pieces of 16 bytes,
    // piece p at physical slot p ^ ((col >> 3) & 7); the lane's rows are half
    // (rt >> 3) & 1 of piece rt >> 4, and col >> 3 == g for all its columns
    uint8_t* const lds_qt = tile + 8 * g * kQtEdge + (((rt >> 4) ^ (g & 7)) * 16) + ((rt >> 3) & 1) * 8;
    const int ct = (int)(cols / kQtEdge), tiles = (int)(rows / kQtEdge) * ct;
    for (int t = blockIdx.x; t < tiles; t += gridDim.x) {
        const int tr = t / ct, tc = t - tr * ct;
        const int64_t R0 = (int64_t)tr * kQtEdge, C0 = (int64_t)tc * kQtEdge;
        const int64_t off = (R0 + rt) * cols + C0 + 8 * g;        // the lane's first element
        uint32_t v[8][4];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const u32x4* src = reinterpret_cast<const u32x4*>(x + off + j * cols);
            const u32x4 w = NT ? __builtin_nontemporal_load(src) : *src;
            v[j][0] = w.x; v[j][1] = w.y; v[j][2] = w.z; v[j][3] = w.w;
        }
        __syncthreads();               // the previous tile's write-out has read the LDS
        uint32_t a[8][4];
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int k = 0; k < 4; ++k) a[j][k] = v[j][k] & 0x7FFF7FFFu;
        // row maxima (the lane's 8 values, then the block's 4 lanes: rotations by 4 and 8)
        uint32_t rm[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const us2 m2 = __builtin_elementwise_max(__builtin_elementwise_max(as_us2(a[j][0]), as_us2(a[j][1])),
                                                     __builtin_elementwise_max(as_us2(a[j][2]), as_us2(a[j][3])));
            uint32_t m = m2.x > m2.y ? m2.x : m2.y;
            uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x124, 0xF, 0xF, false);
            m = m > o ? m : o;
            o = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x128, 0xF, 0xF, false);
            rm[j] = m > o ? m : o;
        }
        // column maxima, packed per pair of columns (the lane's 8 rows, then the quad)
        uint32_t cm[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            us2 m2 = as_us2(a[0][k]);
#pragma unroll
            for (int j = 1; j < 8; ++j) m2 = __builtin_elementwise_max(m2, as_us2(a[j][k]));
            uint32_t m = __builtin_bit_cast(uint32_t, m2);
            m2 = __builtin_elementwise_max(m2, as_us2((uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false)));
            m = __builtin_bit_cast(uint32_t, m2);
            m2 = __builtin_elementwise_max(m2, as_us2((uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false)));
            cm[k] = __builtin_bit_cast(uint32_t, m2);
        }
        uint32_t lane_max = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) lane_max = lane_max > rm[j] ? lane_max : rm[j];
        uint8_t* const qrow = q + off;
        if (__builtin_amdgcn_ballot_w64(lane_max >= 0x7F80u) == 0) {
            // every block of the wave finite: the scaled conversion on clamped values
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                uint32_t lim2;
                const uint32_t sb = mx_fast_scale<FMT>(rm[j], lim2);
                const float sf = __uint_as_float(sb << 23);
                const uint32_t c0 = mx_cvt4<FMT>(mx_clamp2(v[j][0], a[j][0], lim2), mx_clamp2(v[j][1], a[j][1], lim2), sf);
                const uint32_t c1 = mx_cvt4<FMT>(mx_clamp2(v[j][2], a[j][2], lim2), mx_clamp2(v[j][3], a[j][3], lim2), sf);
                *reinterpret_cast<uint2*>(qrow + j * cols) = make_uint2(c0, c1);
                if ((g & 3) == 0) sr[(rt + j) * 4 + (g >> 2)] = (uint8_t)sb;
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                uint32_t l0, l1;
                const uint32_t s0 = mx_fast_scale<FMT>(cm[k] & 0xFFFFu, l0), s1 = mx_fast_scale<FMT>(cm[k] >> 16, l1);
                const uint32_t lim2 = (l0 & 0xFFFFu) | (l1 & 0xFFFF0000u);
                const float f0 = __uint_as_float(s0 << 23), f1 = __uint_as_float(s1 << 23);
                uint32_t c[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) c[j] = mx_clamp2(v[j][k], a[j][k], lim2);
                // column 2k: the low halves of rows (0,1), (2,3), ...; column 2k + 1: the high halves
                uint2 e, o;
                e.x = mx_cvt4<FMT>(__builtin_amdgcn_perm(c[1], c[0], 0x05040100u), __builtin_amdgcn_perm(c[3], c[2], 0x05040100u), f0);
                e.y = mx_cvt4<FMT>(__builtin_amdgcn_perm(c[5], c[4], 0x05040100u), __builtin_amdgcn_perm(c[7], c[6], 0x05040100u), f0);
                o.x = mx_cvt4<FMT>(__builtin_amdgcn_perm(c[1], c[0], 0x07060302u), __builtin_amdgcn_perm(c[3], c[2], 0x07060302u), f1);
                o.y = mx_cvt4<FMT>(__builtin_amdgcn_perm(c[5], c[4], 0x07060302u), __builtin_amdgcn_perm(c[7], c[6], 0x07060302u), f1);
                *reinterpret_cast<uint2*>(lds_qt + (2 * k) * kQtEdge) = e;
                *reinterpret_cast<uint2*>(lds_qt + (2 * k + 1) * kQtEdge) = o;
                if (rq == 0) {
                    sc[(8 * g + 2 * k) * 4 + wave] = (uint8_t)s0;
                    sc[(8 * g + 2 * k + 1) * 4 + wave] = (uint8_t)s1;
                }
            }
        } else {
            // an infinity or a NaN in the wave's rows: the per-element rule, one row
            // or pair of columns at a time, re-reading x (rare: kept out of the
            // registers of the common path)
#pragma unroll 1
            for (int j = 0; j < 8; ++j) {
                const u32x4 w = *reinterpret_cast<const u32x4*>(x + off + j * cols);
                const uint32_t wr[4] = {w.x, w.y, w.z, w.w};
                uint32_t m = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t lo = wr[k] & 0x7FFFu, hi = (wr[k] >> 16) & 0x7FFFu;
                    m = m > lo ? m : lo;
                    m = m > hi ? m : hi;
                }
                uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x124, 0xF, 0xF, false);
                m = m > o ? m : o;
                o = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x128, 0xF, 0xF, false);
                m = m > o ? m : o;
                uint32_t sb;
                const float s = mx_scale_of<FMT>(m, sb);
                uint32_t c[2];
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    c[h] = mx_code2<FMT>(wr[2 * h] & 0xFFFFu, wr[2 * h] >> 16, s) |
                           (mx_code2<FMT>(wr[2 * h + 1] & 0xFFFFu, wr[2 * h + 1] >> 16, s) << 16);
                *reinterpret_cast<uint2*>(qrow + j * cols) = make_uint2(c[0], c[1]);
                if ((g & 3) == 0) sr[(rt + j) * 4 + (g >> 2)] = (uint8_t)sb;
            }
#pragma unroll 1
            for (int k = 0; k < 4; ++k) {
                uint32_t col[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) col[j] = reinterpret_cast<const uint32_t*>(x + off + j * cols)[k];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int sh = 16 * h;
                    uint32_t m = 0;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const uint32_t e = (col[j] >> sh) & 0x7FFFu;
                        m = m > e ? m : e;
                    }
                    uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false);
                    m = m > o ? m : o;
                    o = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false);
                    m = m > o ? m : o;
                    uint32_t sb;
                    const float s = mx_scale_of<FMT>(m, sb);
                    uint32_t c[2];
#pragma unroll
                    for (int r = 0; r < 2; ++r) {
                        const int j = 4 * r;
                        c[r] = mx_code2<FMT>((col[j] >> sh) & 0xFFFFu, (col[j + 1] >> sh) & 0xFFFFu, s) |
                               (mx_code2<FMT>((col[j + 2] >> sh) & 0xFFFFu, (col[j + 3] >> sh) & 0xFFFFu, s) << 16);
                    }
                    *reinterpret_cast<uint2*>(lds_qt + (2 * k + h) * kQtEdge) = make_uint2(c[0], c[1]);
                    if (rq == 0) sc[(8 * g + 2 * k + h) * 4 + wave] = (uint8_t)sb;
                }
            }
        }
        __syncthreads();
        // write-out: 1024 pieces of 16 bytes, 4 per thread (a wave instruction covers
        // 8 qt rows x 128 bytes), then the two 512-byte scale runs
        const int p = tid & 7;
        uint8_t* const qtp = qt + (C0 + (tid >> 3)) * rows + R0 + p * 16;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int col = u * 32 + (tid >> 3);
            const u32x4 piece16 = *reinterpret_cast<const u32x4*>(tile + col * kQtEdge + ((p ^ ((col >> 3) & 7)) * 16));
            *reinterpret_cast<u32x4*>(qtp + (int64_t)u * 32 * rows) = piece16;
        }
        // sq dword (tc rows + R0 + r): row r's four blocks of this column group;
        // sqt dword (tr cols + C0 + col): column col's four blocks of this row band
        if (tid < kQtEdge)
            sq[(int64_t)tc * rows + R0 + tid] = srow[tid];
        else
            sqt[(int64_t)tr * cols + C0 + (tid - kQtEdge)] = scol[tid - kQtEdge];
    }
}

hipError_t launch_mx_quantize_both(const void* x, int64_t rows, int64_t cols, int fmt, uint8_t* q, uint8_t* sq,
                                   uint8_t* qt, uint8_t* sqt, hipStream_t stream)
{
    const int64_t tiles = (rows / kQtEdge) * (cols / kQtEdge);
    int64_t blocks = tiles;
    const int64_t cap = (int64_t)device_cu_count() * 4;
    if (blocks > cap) blocks = cap;
    const uint16_t* xv = reinterpret_cast<const uint16_t*>(x);
    uint32_t* sqv = reinterpret_cast<uint32_t*>(sq);
    uint32_t* sqtv = reinterpret_cast<uint32_t*>(sqt);
    const bool nt = 2 * rows * cols >= kAbsStreamBytes;
    const dim3 grid((unsigned)blocks), block(256);
    if (fmt == 0)
        return nt ? launch(mx_quantize_both_kernel<0, true>, grid, block, stream, xv, rows, cols, q, sqv, qt, sqtv)
                  : launch(mx_quantize_both_kernel<0, false>, grid, block, stream, xv, rows, cols, q, sqv, qt, sqtv);
    return nt ? launch(mx_quantize_both_kernel<1, true>, grid, block, stream, xv, rows, cols, q, sqv, qt, sqtv)
              : launch(mx_quantize_both_kernel<1, false>, grid, block, stream, xv, rows, cols, q, sqv, qt, sqtv);
}


// Transposed block (MX) quantisation: qt = the codes of x^T [cols, rows] with
// blocks of 32 consecutive elements along qt's rows, i.e. 32 consecutive rows
// of one column of x -- the operand layout of a backward product whose
// reduction runs over x's rows (the blocks must lie along the reduction, so
// this is a second quantisation of x, not a transpose of the first).  A wave
// takes 64 rows x 128 columns: lane l reads columns 2 l, 2 l + 1 of each of the
// 64 rows (every load instruction reads a 256-byte row segment), so each of its
// two columns' two blocks lies in its own registers; it writes 64 contiguous
// codes per column (qt row c, columns r0 .. r0 + 63) and the column's two scale
// bytes.  Scales step-major for qt: block b of qt row c at ((b / 4) cols + c) 4
// + b % 4.  rows % 128 == 0 and cols % 128 == 0.
template <int FMT, bool NT>
__global__ void __launch_bounds__(256) mx_quantize_t_kernel(const uint32_t* __restrict__ x, int64_t rows,
                                                            int64_t cols, uint8_t* __restrict__ qt,
                                                            uint8_t* __restrict__ scales)
{
    constexpr int emax = FMT == 0 ? 8 : 15;
    const int lane = threadIdx.x & 63;
    const int64_t ct = cols / 128, tiles = (rows / 64) * ct;
    for (int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); t < tiles; t += (int64_t)gridDim.x * 4) {
        const int64_t r0 = (t / ct) * 64, c = (t % ct) * 128 + 2 * lane;    // the lane's columns c, c + 1
        uint32_t w[64];
#pragma unroll
        for (int r = 0; r < 64; ++r) {
            const uint32_t* src = x + ((r0 + r) * cols + c) / 2;
            w[r] = NT ? __builtin_nontemporal_load(src) : *src;
        }
#pragma unroll
        for (int col = 0; col < 2; ++col) {
            uint32_t codes[16];
            uint32_t sbytes = 0;
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                uint32_t m = 0;
#pragma unroll
                for (int r = 0; r < 32; ++r) {
                    const uint32_t a = (col ? (w[blk * 32 + r] >> 16) : w[blk * 32 + r]) & 0x7FFFu;
                    m = m > a ? m : a;
                }
                const bool bad = m >= 0x7F80u;     // an infinity or a NaN in the block
                float s = 1.0f;
                uint32_t sbyte = 255;
                if (!bad) {
                    const int fl = m >= 0x80u ? (int)(m >> 7) - 127 : 31 - __builtin_clz(m | 1u) - 133;
                    int e = m ? fl - emax : -127;
                    e = e < -127 ? -127 : e;
                    s = __uint_as_float((uint32_t)(127 - e) << 23);
                    sbyte = (uint32_t)(e + 127);
                }
                sbytes |= sbyte << (8 * blk);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    float v[4];
#pragma unroll
                    for (int e4 = 0; e4 < 4; ++e4) {
                        const uint32_t wv = w[blk * 32 + 4 * k + e4];
                        v[e4] = (col ? bf16_hi(wv) : bf16_lo(wv)) * s;
                    }
                    uint32_t cw = mx_enc4<FMT>(v[0], v[1], v[2], v[3]);
                    if (bad) {
#pragma unroll
                        for (int e4 = 0; e4 < 4; ++e4) {
                            const uint32_t hb = (col ? (w[blk * 32 + 4 * k + e4] >> 16) : w[blk * 32 + 4 * k + e4]) & 0xFFFFu;
                            if ((hb & 0x7FFFu) > 0x7F80u)
                                cw = (cw & ~(0xFFu << (8 * e4))) | ((((hb >> 8) & 0x80u) | 0x7Fu) << (8 * e4));
                        }
                    }
                    codes[blk * 8 + k] = cw;
                }
            }
            uint4* dst = reinterpret_cast<uint4*>(qt + (c + col) * rows + r0);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                dst[k] = make_uint4(codes[4 * k], codes[4 * k + 1], codes[4 * k + 2], codes[4 * k + 3]);
            // blocks r0 / 32 and r0 / 32 + 1 of qt row c + col (both in the same group of 4)
            const int64_t b0 = r0 / 32;
            *reinterpret_cast<uint16_t*>(scales + ((b0 >> 2) * cols + c + col) * 4 + (b0 & 3)) = (uint16_t)sbytes;
        }
    }
}

hipError_t launch_mx_quantize_t(const void* x, int64_t rows, int64_t cols, int fmt, uint8_t* qt, uint8_t* scales,
                                hipStream_t stream)
{
    const int64_t tiles = (rows / 64) * (cols / 128);
    int64_t blocks = (tiles + 3) / 4;
    const int64_t cap = (int64_t)device_cu_count() * 4;
    if (blocks > cap) blocks = cap;
    const uint32_t* xv = reinterpret_cast<const uint32_t*>(x);
    const bool nt = 2 * rows * cols >= kAbsStreamBytes;
    const dim3 grid((unsigned)blocks), block(256);
    if (fmt == 0)
        return nt ? launch(mx_quantize_t_kernel<0, true>, grid, block, stream, xv, rows, cols, qt, scales)
                  : launch(mx_quantize_t_kernel<0, false>, grid, block, stream, xv, rows, cols, qt, scales);
    return nt ? launch(mx_quantize_t_kernel<1, true>, grid, block, stream, xv, rows, cols, qt, scales)
              : launch(mx_quantize_t_kernel<1, false>, grid, block, stream, xv, rows, cols, qt, scales);
}

hipError_t launch_mx_quantize(const void* x, int64_t rows, int64_t cols, int fmt, uint8_t* q, uint8_t* scales,
                              hipStream_t stream)
{
    const int64_t n = rows * cols, nvec = n / 8;
    int64_t blocks = (nvec + 255) / 256;
    const int64_t cap = (int64_t)device_cu_count() * 8;
    if (blocks > cap) blocks = cap;
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    uint2* qv = reinterpret_cast<uint2*>(q);
    const uint32_t r = (uint32_t)rows, nb = (uint32_t)(cols / 32);
    const bool nt = 2 * n >= kAbsStreamBytes;
    const dim3 grid((unsigned)blocks), block(256);
    if (fmt == 0)
        return nt ? launch(mx_quantize_kernel<0, true>, grid, block, stream, xv, nvec, qv, scales, r, nb)
                  : launch(mx_quantize_kernel<0, false>, grid, block, stream, xv, nvec, qv, scales, r, nb);
    return nt ? launch(mx_quantize_kernel<1, true>, grid, block, stream, xv, nvec, qv, scales, r, nb)
              : launch(mx_quantize_kernel<1, false>, grid, block, stream, xv, nvec, qv, scales, r, nb);
}

}  // namespace fp8k
