// gemm.hip -- FP8 GEMM with fp32 accumulation and per-tensor descale, gfx950.
//
//   out[p, q] = bf16_RNE( RN32( sum_r dec(A[p, r]) * dec(B[q, r]) ) * RN32(inv_a * inv_b) )
//
// One TN kernel serves the forward, dgrad and wgrad products ("LLMQ: Efficient
// Lower-Precision Pretraining for Consumer GPUs", section 2: low-precision
// operands on the matrix units; section 4: larger models are dominated by
// these products).  Both operands are contiguous along the reduction index.
//
// Design (CDNA4):
//  - 256 x 256 output tile per workgroup, reduction step 128 bytes, 256 threads
//    = 4 waves in a 2 x 2 grid, each wave 128 x 128 outputs held as 8 x 8
//    blocks of v_mfma_f32_16x16x128_f8f6f4 accumulators (256 fp32 per lane);
//    on gfx950 this instruction issues faster than the 32x32x64 one.
//    The operand formats (E4M3 / E5M2) are selected per operand by the
//    instruction, so mixed E5M2 x E4M3 products run natively.
//  - Operand tiles go global -> LDS with 16-byte direct-to-LDS loads
//    (global_load_lds_dwordx4), two stages of 64 KB; tile k+2 is issued in the
//    middle of step k, so each load has about one and a half steps to land.
//  - Fragments are pipelined in registers: the LDS reads for the next half
//    step and the next step's B fragments (read into each B block's registers
//    as soon as that block is consumed) overlap the matrix instructions.
//  - LDS rows are 128 bytes; the 16-byte chunk c of row r is stored at chunk
//    c ^ f(r), f(r) = ((r >> 1) & 7) ^ ((r & 1) << 2).  A lane's 32 fragment
//    bytes are chunks g and g + 4 of its row (g = lane / 16); with this pairing
//    every 16-byte fragment read runs at the 4-cycle LDS minimum on gfx950
//    (no bank conflicts, measured).
//  - The instruction's operands are swapped (B fragment first), so each lane
//    ends with 4 consecutive output columns of one row; the epilogue stages
//    them through LDS and writes full 256-byte row segments.
//  - Persistent: one workgroup per CU walks tiles in a grouped raster order,
//    renumbered XCD-major so that the 32 CUs of an XCD (sharing one L2) work on
//    consecutive tiles; the next tile's first stages load during the epilogue.
//  - Deterministic: every output is reduced by one wave in a fixed order.
#include "fp8_device.hpp"
#include "fp8_internal.hpp"

namespace fp8k {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 128;
constexpr int kStageA = kBM * kBK;            // 32 KB
constexpr int kStageB = kBN * kBK;            // 32 KB
constexpr int kStage = kStageA + kStageB;     // 64 KB
constexpr int kLds = 2 * kStage;              // 128 KB
constexpr int kEpiRows = 32;                  // epilogue chunk: 32 rows x 128 columns of bf16 per wave
constexpr int kEpiWave = kEpiRows * 256;      // 8 KB per wave, 32 KB per workgroup (LDS total 160 KB)
constexpr int kGroupM = 8;                    // tile rows per raster group

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt[5:4] at [15:14]); expcnt and lgkmcnt are left at their maxima.
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitVm16 = 0x4F70;

__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

// 16-byte direct-to-LDS load in the scalar-base form: lane L reads 16 bytes at
// sbase + voff[L] and writes LDS bytes [lds + 16 L, lds + 16 L + 16).  Issued
// as inline assembly so that the compiler's LDS-DMA hazard tracking does not
// put a wait for every pending load in front of each LDS read: the kernel
// orders these loads itself with an explicit vmcnt wait and a barrier before
// the stage they fill is read.
__device__ __forceinline__ void dma16(uint32_t voff, const uint8_t* sbase, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}

// The 32 bytes of a fragment row are logical chunks c and c + 4 (16 bytes each),
// at physical chunks p and p ^ 4.
__device__ __forceinline__ v8i lds_frag(const uint8_t* tile, int row, int chunk)
{
    const int p = chunk ^ swz(row);
    const uint4 lo = *reinterpret_cast<const uint4*>(tile + row * kBK + p * 16);
    const uint4 hi = *reinterpret_cast<const uint4*>(tile + row * kBK + (p ^ 4) * 16);
    v8i r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
}

// Global -> LDS sources of one wave.  Load ii (0..7) of wave w fills LDS rows
// r = (w*8 + ii)*8 + L/8 of the A (B) stage, lane L at physical chunk L%8, i.e.
// it reads logical chunk (L%8) ^ f(r).  f(r) depends on ii only through ii & 1,
// so in the interior form a lane keeps two byte offsets per operand and the
// row step 8 * ii * R goes into the uniform base.  Matrices with fewer than
// 256 rows (EDGE) clamp each row to the last valid one instead.
struct Sources {
    const uint8_t* a;
    const uint8_t* b;
    uint32_t a_off[2];
    uint32_t b_off[2];
    uint32_t step;        // 8 rows
    int a_row, b_row;     // EDGE: the lane's first row and the last valid row
    int a_last, b_last;
    uint32_t chunk16[2];
};

// Load idx (0..15) of a stage: 0..7 fill A, 8..15 fill B.
template <bool EDGE>
__device__ __forceinline__ void issue_one(const Sources& src, uint32_t stage, int k0, int wave, int idx)
{
    const int ii = idx & 7;
    const bool is_b = idx >= 8;
    const uint32_t lds = __builtin_amdgcn_readfirstlane(stage + (is_b ? (uint32_t)kStageA : 0u) +
                                                        (uint32_t)(wave * 8 + ii) * 1024u);
    const uint8_t* base = is_b ? src.b : src.a;
    if (!EDGE) {
        const uint32_t off = is_b ? src.b_off[ii & 1] : src.a_off[ii & 1];
        dma16(off, base + ((size_t)ii * src.step + (size_t)k0), lds);
    } else {
        const uint32_t R = src.step / 8u;
        const int row = is_b ? min(src.b_row + ii * 8, src.b_last) : min(src.a_row + ii * 8, src.a_last);
        dma16((uint32_t)row * R + src.chunk16[ii & 1], base + k0, lds);
    }
}

template <bool EDGE>
__device__ __forceinline__ void issue_stage(const Sources& src, uint32_t stage, int k0, int wave)
{
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) issue_one<EDGE>(src, stage, k0, wave, idx);
}

// Fragments of the 16x16x128 instruction: block b of 16 rows, lane l holds row
// l % 16 and the k bytes 16 g .. 16 g + 15 and 64 + 16 g .. 64 + 16 g + 15 of the
// 128-byte step, g = l / 16 (the same k mapping for both operands, so the
// order of k within the instruction does not matter).  With the row swizzle
// above, each 16-byte LDS read of a block is free of bank conflicts on gfx950
// (measured with SQ_LDS_BANK_CONFLICT; the pairing of chunks 2g, 2g + 1 costs
// a 2-way conflict, 8 instead of 4 LDS cycles per read).  A wave owns
// 128 x 128 outputs = 8 x 8 blocks.
__device__ __forceinline__ v8i read_frag16(const uint8_t* tile, int row0, int lane)
{
    return lds_frag(tile, row0 + (lane & 15), lane >> 4);
}

typedef float v4f __attribute__((ext_vector_type(4)));

// acc[i][j] += A block i x B block j (the instruction's first source is the B
// block, so each lane ends with 4 consecutive output columns of one row).
template <int FA, int FB>
__device__ __forceinline__ void mma16(v4f (&acc)[8][8], const v8i& a, const v8i& b, int i, int j)
{
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, acc[i][j], FB, FA, 0, 0, 0, 0);
}

// A reduction step (128 bytes of k) runs in two halves split by A rows:
//   half 0: 32 instructions A[0..3] x B[0..7] (B block outer, A block inner),
//           interleaved with the LDS reads of A blocks 4..7 (ahi) of the step;
//   half 1: 32 instructions A[4..7] x B[0..7] in the same order, so B block j
//           is dead after its four instructions and the next step's B block j
//           is read into the same registers right then; the next step's A
//           blocks 0..3 (alo) and the 16 loads of tile k+2 are interleaved too.
// Between the halves a barrier (after this wave's loads of tile k+1 are waited
// for) guarantees that every wave has read all of the step's stage and that
// tile k+1 has landed.  The K loop body is [barrier, half 1 of step k, half 0
// of step k+1], so each LDS read and its first use lie in one straight-line
// body.
template <int FA, int FB>
__device__ __forceinline__ void half0(v4f (&acc)[8][8], const v8i (&bq)[8], const v8i (&alo)[4], v8i (&ahi)[4],
                                      const uint8_t* stage, int wm, int lane)
{
#pragma unroll
    for (int t = 0; t < 32; ++t) {
        const int j = t >> 2, i = t & 3;
        mma16<FA, FB>(acc, alo[i], bq[j], i, j);
        if ((t & 7) == 1) ahi[t >> 3] = read_frag16(stage, wm * 128 + (4 + (t >> 3)) * 16, lane);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int FA, int FB, bool EDGE, bool NEXT>
__device__ __forceinline__ void half1(v4f (&acc)[8][8], v8i (&bq)[8], v8i (&alo)[4], const v8i (&ahi)[4],
                                      const Sources& src, uint32_t cur_addr, const uint8_t* nxt, int k_issue,
                                      int wave, int wm, int wn, int lane)
{
#pragma unroll
    for (int t = 0; t < 32; ++t) {
        const int j = t >> 2, i = t & 3;
        mma16<FA, FB>(acc, ahi[i], bq[j], 4 + i, j);
        if (NEXT) {
            if (i == 3) bq[j] = read_frag16(nxt + kStageA, wn * 128 + j * 16, lane);
            if ((t & 7) == 1) alo[t >> 3] = read_frag16(nxt, wm * 128 + (t >> 3) * 16, lane);
            if ((t & 1) == 0) issue_one<EDGE>(src, cur_addr, k_issue, wave, t >> 1);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

__device__ __forceinline__ void mid_step_barrier()
{
    __builtin_amdgcn_s_waitcnt(kWaitVm0);     // the next tile has landed (this wave's loads)
    __syncthreads();                          // ... for all waves; the current stage fully read
    __builtin_amdgcn_sched_barrier(0);
}

// A launch covers a group of up to kMaxGroup independent problems of the same
// operand formats (e.g. the dgrad and wgrad products of one linear).  Their
// tiles form one virtual tile range, problem after problem; the host orders
// the problems by reduction length, longest first, so that the round-robin
// walk of the persistent workgroups starts with the longest tiles.
constexpr int kMaxGroup = 2;

struct GemmProblem {
    const uint8_t* A;
    const uint8_t* B;
    const float* inv_a;
    const float* inv_b;
    uint16_t* out;
    int P, Q, R;
    int tiles_m, tiles_n;
    int first_tile;
};

struct GemmGroup {
    GemmProblem p[kMaxGroup];
    int count;
    int total_tiles;
};

// Everything a workgroup needs about its current tile (all wave-uniform).
struct Work {
    const uint8_t* A;
    const uint8_t* B;
    uint16_t* out;
    const float* inv_a;
    const float* inv_b;
    int P, Q, R, KT;
    int ms, ns;     // logical origin (first row / column this tile stores)
    int m0, n0;     // origin actually computed (shifted back inside the matrix)
};

// Output tile of a virtual tile id: the problem it falls in, then a grouped
// raster order within it (kGroupM tile rows per group, column-major within a
// group), so consecutive ids share A and B panels.
template <bool EDGE>
__device__ __forceinline__ Work work_of(const GemmGroup& g, int v)
{
    const bool second = g.count > 1 && v >= g.p[1].first_tile;
    const GemmProblem& pr = second ? g.p[1] : g.p[0];
    Work w;
    w.A = pr.A;
    w.B = pr.B;
    w.out = pr.out;
    w.inv_a = pr.inv_a;
    w.inv_b = pr.inv_b;
    w.P = pr.P;
    w.Q = pr.Q;
    w.R = pr.R;
    w.KT = pr.R / kBK;
    const int lv = v - pr.first_tile;
    const int group_size = kGroupM * pr.tiles_n;
    const int group = lv / group_size;
    const int first_m = group * kGroupM;
    const int gm = min(pr.tiles_m - first_m, kGroupM);
    const int in_group = lv - group * group_size;
    w.ms = (first_m + in_group % gm) * kBM;
    w.ns = (in_group / gm) * kBN;
    // A last partial tile is shifted back to end at the matrix edge (P, Q >= 256),
    // recomputing rows / columns of its neighbour that it then does not store.
    w.m0 = EDGE ? w.ms : min(w.ms, w.P - kBM);
    w.n0 = EDGE ? w.ns : min(w.ns, w.Q - kBN);
    return w;
}

__device__ __forceinline__ void set_sources(Sources& src, const Work& w, int wave, int lane)
{
    src.a = w.A;
    src.b = w.B;
    src.a_last = w.P - 1;
    src.b_last = w.Q - 1;
    src.step = 8u * (uint32_t)w.R;
    src.a_row = w.m0 + wave * 64 + (lane >> 3);
    src.b_row = w.n0 + wave * 64 + (lane >> 3);
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int row = (wave * 8 + par) * 8 + (lane >> 3);     // row within the tile
        src.chunk16[par] = (uint32_t)(((lane & 7) ^ swz(row)) * 16);
        src.a_off[par] = (uint32_t)src.a_row * (uint32_t)w.R + src.chunk16[par];
        src.b_off[par] = (uint32_t)src.b_row * (uint32_t)w.R + src.chunk16[par];
    }
}

// Persistent kernel: one workgroup per CU walks the virtual tiles v = slot,
// slot + G, slot + 2G, ... where slot renumbers the workgroups XCD-major
// (workgroups are dealt round-robin to the 8 XCDs, each with its own L2), so in
// every round the 32 CUs of one XCD work on 32 consecutive tiles of the raster
// order.  While a tile's epilogue stores run, the first two stages of the next
// tile are already loading.
template <int FA, int FB, bool EDGE>
__global__ void __launch_bounds__(256, 1) gemm_tn_kernel(const GemmGroup g)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];
    __shared__ __attribute__((aligned(1024))) uint8_t epi[4 * kEpiWave];

    const int G = gridDim.x;
    int slot = blockIdx.x;
    if (G % 8 == 0) slot = (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;

    Sources src;
    v8i bq[8], alo[4], ahi[4];
    v4f acc[8][8];

    int v = slot;
    if (v >= g.total_tiles) return;
    Work w = work_of<EDGE>(g, v);
    set_sources(src, w, wave, lane);
    issue_stage<EDGE>(src, lds_addr, 0, wave);
    issue_stage<EDGE>(src, lds_addr + kStage, min(1, w.KT - 1) * kBK, wave);
    for (;;) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.0f;
        __builtin_amdgcn_s_waitcnt(kWaitVm16);    // stage 0 landed; stage 1's 16 loads may be in flight
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 8; ++j) bq[j] = read_frag16(lds + kStageA, wn * 128 + j * 16, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) alo[i] = read_frag16(lds, wm * 128 + i * 16, lane);
        half0<FA, FB>(acc, bq, alo, ahi, lds, wm, lane);
        const int KT = w.KT;
        for (int kt = 0; kt + 1 < KT; ++kt) {
            const int cur = kt & 1;
            mid_step_barrier();
            half1<FA, FB, EDGE, true>(acc, bq, alo, ahi, src, lds_addr + cur * kStage, lds + (cur ^ 1) * kStage,
                                      min(kt + 2, KT - 1) * kBK, wave, wm, wn, lane);
            half0<FA, FB>(acc, bq, alo, ahi, lds + (cur ^ 1) * kStage, wm, lane);
        }
        mid_step_barrier();
        half1<FA, FB, EDGE, false>(acc, bq, alo, ahi, src, 0, lds, 0, wave, wm, wn, lane);
        // every load of this tile has landed and every wave is done with LDS
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __syncthreads();

        const Work done = w;
        const int next = v + G;
        if (next < g.total_tiles) {
            v = next;
            w = work_of<EDGE>(g, v);
            set_sources(src, w, wave, lane);
            issue_stage<EDGE>(src, lds_addr, 0, wave);
            issue_stage<EDGE>(src, lds_addr + kStage, min(1, w.KT - 1) * kBK, wave);
        }

        // ---- epilogue of `done`: descale and round to bf16, stage 32-row chunks of
        // the wave's 128 x 128 tile in its private LDS region (16-byte chunks of a
        // 256-byte row XOR-swizzled by row), read back 16 bytes per lane and store
        // four full 256-byte row segments per instruction.
        const float d = done.inv_a[0] * done.inv_b[0];
        uint8_t* ew = epi + wave * kEpiWave;
        const int r16 = lane & 15, q4 = lane >> 4;
#pragma unroll
        for (int c2 = 0; c2 < 4; ++c2) {                 // chunk: A blocks 2*c2, 2*c2+1 (32 rows)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int i = 2 * c2 + h;
                const int row = h * 16 + r16;             // row within the chunk
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const f32x2 v01 = {acc[i][j][0] * d, acc[i][j][1] * d};
                    const f32x2 v23 = {acc[i][j][2] * d, acc[i][j][3] * d};
                    uint2 o;
                    o.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(v01, bf16x2));
                    o.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(v23, bf16x2));
                    // columns j*16 + 4*q4 .. +3 = bytes j*32 + 8*q4: 16-byte chunk 2j + q4/2
                    const int chunk = (2 * j + (q4 >> 1)) ^ (row & 15);
                    *reinterpret_cast<uint2*>(ew + row * 256 + chunk * 16 + (q4 & 1) * 8) = o;
                }
            }
#pragma unroll
            for (int it = 0; it < kEpiRows / 4; ++it) {
                const int rr = it * 4 + (lane >> 4);                   // row within the chunk
                const int c = lane & 15;                              // logical 16-byte chunk
                const uint4 o = *reinterpret_cast<const uint4*>(ew + rr * 256 + ((c ^ (rr & 15)) * 16));
                const int m = done.m0 + wm * 128 + c2 * 32 + rr;
                const int n = done.n0 + wn * 128 + c * 8;
                if (m >= done.ms && m < done.P && n >= done.ns && n < done.Q)
                    *reinterpret_cast<uint4*>(done.out + (size_t)m * done.Q + n) = o;
            }
        }
        // The loop-top wait (vmcnt <= 16) then proves the next tile's first stage
        // has landed: if one of its loads were pending, the 16 later loads of the
        // second stage would be too (loads complete in order), whatever the
        // interleaved stores do.
        if (next >= g.total_tiles) break;
    }
}

static GemmProblem make_problem(const uint8_t* A, const uint8_t* B, const float* inv_a, const float* inv_b,
                                void* out, int64_t P, int64_t Q, int64_t R)
{
    GemmProblem p;
    p.A = A;
    p.B = B;
    p.inv_a = inv_a;
    p.inv_b = inv_b;
    p.out = reinterpret_cast<uint16_t*>(out);
    p.P = (int)P;
    p.Q = (int)Q;
    p.R = (int)R;
    p.tiles_m = (int)((P + kBM - 1) / kBM);
    p.tiles_n = (int)((Q + kBN - 1) / kBN);
    p.first_tile = 0;
    return p;
}

template <int FA, int FB>
static hipError_t launch_group(GemmGroup g, hipStream_t stream)
{
    bool edge = false;
    int total = 0;
    for (int i = 0; i < g.count; ++i) {
        g.p[i].first_tile = total;
        total += g.p[i].tiles_m * g.p[i].tiles_n;
        edge = edge || g.p[i].P < kBM || g.p[i].Q < kBN;
    }
    g.total_tiles = total;
    const int grid = total < device_cu_count() ? total : device_cu_count();   // one workgroup per CU
    if (!edge)
        gemm_tn_kernel<FA, FB, false><<<grid, 256, 0, stream>>>(g);
    else
        gemm_tn_kernel<FA, FB, true><<<grid, 256, 0, stream>>>(g);
    return hipGetLastError();
}

static hipError_t dispatch(int fmt_a, int fmt_b, const GemmGroup& g, hipStream_t stream)
{
    if (fmt_a == 0 && fmt_b == 0) return launch_group<0, 0>(g, stream);
    if (fmt_a == 1 && fmt_b == 0) return launch_group<1, 0>(g, stream);
    if (fmt_a == 0 && fmt_b == 1) return launch_group<0, 1>(g, stream);
    return launch_group<1, 1>(g, stream);
}

hipError_t launch_gemm_tn(const uint8_t* A, int fmt_a, const uint8_t* B, int fmt_b, const float* inv_a,
                          const float* inv_b, void* out, int64_t P, int64_t Q, int64_t R, hipStream_t stream)
{
    GemmGroup g;
    g.p[0] = make_problem(A, B, inv_a, inv_b, out, P, Q, R);
    g.p[1] = g.p[0];
    g.count = 1;
    return dispatch(fmt_a, fmt_b, g, stream);
}

hipError_t launch_gemm_tn_pair(const uint8_t* A0, const uint8_t* B0, const float* ia0, const float* ib0, void* out0,
                               int64_t P0, int64_t Q0, int64_t R0, const uint8_t* A1, const uint8_t* B1,
                               const float* ia1, const float* ib1, void* out1, int64_t P1, int64_t Q1, int64_t R1,
                               int fmt_a, int fmt_b, hipStream_t stream)
{
    GemmGroup g;
    GemmProblem p0 = make_problem(A0, B0, ia0, ib0, out0, P0, Q0, R0);
    GemmProblem p1 = make_problem(A1, B1, ia1, ib1, out1, P1, Q1, R1);
    // longest reduction first: the first round then starts the longest tiles
    g.p[0] = R1 > R0 ? p1 : p0;
    g.p[1] = R1 > R0 ? p0 : p1;
    g.count = 2;
    return dispatch(fmt_a, fmt_b, g, stream);
}

}  // namespace fp8k
