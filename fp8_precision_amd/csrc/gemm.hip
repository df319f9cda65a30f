// gemm.hip -- FP8 GEMM with fp32 accumulation and per-tensor descale, gfx950.
//
//   out[p, q] = bf16_RNE( RN32( sum_r dec(A[p, r]) * dec(B[q, r]) ) * RN32(inv_a * inv_b) )
//
// One kernel serves the forward, dgrad and wgrad products ("LLMQ: Efficient
// Lower-Precision Pretraining for Consumer GPUs", section 2: low-precision
// operands on the matrix units; section 4: larger models are dominated by
// these products, and the backward pass needs transposed operands).  Each
// operand is read in one of two layouts:
//   K-major  (A[p, r] at A + p * R + r): contiguous along the reduction index;
//   MN-major (A[p, r] at A + r * P + p): contiguous along the output index --
//            the untransposed FP8 tensor, so the backward products need no
//            transposed copies (dgrad reads W [N, K] directly, wgrad reads dY
//            [M, N] and X [M, K] directly).
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
//  - K-major tiles: 256 rows of 128 bytes; the 16-byte chunk c of row r is
//    stored at chunk c ^ f(r), f(r) = ((r >> 1) & 7) ^ ((r & 1) << 2).  A lane's
//    32 fragment bytes are chunks g and g + 4 of its row (g = lane / 16), read
//    with two ds_read_b128.
//  - MN-major tiles: 128 rows (reduction index) of 256 bytes; chunk c of row r
//    is stored at c ^ h(r), h(r) = (r & 7) | (((r >> 4) & 1) << 3).  A fragment
//    is four ds_read_b64_tr_b8: in each 16-lane group, lanes 2t and 2t + 1 name
//    the two halves of a 16-byte piece of row t and lane i receives byte i of
//    all eight rows -- the same 32 reduction values per lane, in the same
//    order, as the K-major read, so both layouts give bit-identical results.
//    With these swizzles every fragment read runs at the LDS minimum on gfx950
//    (4 cycles per 1 KB ds_read_b128, 2 per 512-byte transpose read; measured
//    with SQ_LDS_BANK_CONFLICT = 0).
//  - The instruction's operands are swapped (B fragment first), so each lane
//    ends with 4 consecutive output columns of one row; the epilogue stages
//    them through LDS and writes full 256-byte row segments.
//  - Persistent: one workgroup per CU walks tiles in a grouped raster order
//    (8 tile rows per group; 4 for a backward problem wider than 32 column
//    tiles), renumbered XCD-major so that the 32 CUs of an XCD (sharing one L2)
//    work on consecutive tiles; the next tile's first stages load during the
//    epilogue.  When the last round would keep at most half of the CUs busy,
//    its tiles are split into 128 x 256 half tiles (the same B loads and
//    fragment reads, half the A rows, a 64 x 128 wave tile) in a launch of
//    their own; a half tile's 48 KB stage lets it run three stages, its loads
//    issued two steps ahead.
//  - Output stores: ordinary for the forward products (the statistic or
//    SwiGLU pass that follows reads them from the Infinity Cache); non-temporal
//    for the backward products (a template argument: with a run-time choice the
//    compiler merged the two store forms and dropped the hint).
//  - Deterministic: every output is reduced by one wave in a fixed order.
//  - Block-scaled (MX) products: gemm_mx_kernel, the same walk and tiles with
//    each row's E8M0 block scales loaded beside its codes and applied by
//    v_mfma_scale_f32_16x16x128_f8f6f4 (see the block-scaled section below).
#include "fp8_device.hpp"
#include "fp8_internal.hpp"

namespace fp8k {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 128;
constexpr int kStageA = kBM * kBK;            // 32 KB
constexpr int kStageB = kBN * kBK;            // 32 KB
constexpr int kStage = kStageA + kStageB;     // 64 KB
constexpr int kLds = 2 * kStage;              // 128 KB
constexpr int kEpiRows = 32;                  // epilogue chunk: 32 rows x 128 columns of bf16 per wave
constexpr int kEpiWave = kEpiRows * 256;      // 8 KB per wave, 32 KB per workgroup (LDS total 160 KB)
// Half tiles (128 rows of A) use 48 KB per stage (A at 0, B at 16 KB) and run
// three stages, with 16-row epilogue chunks (4 KB per wave) after them:
// 3 x 48 + 16 = 160 KB.
constexpr int kHalfA = kStageA / 2;           // 16 KB
constexpr int kHalfStage = kHalfA + kStageB;  // 48 KB
constexpr int kHalfEpi = 3 * kHalfStage;      // 144 KB: the half tiles' epilogue staging
// Block-scaled (MX) launches: per stage, the E8M0 scales of the step's four
// 32-byte reduction blocks for the 256 A rows and the 256 B rows (4 bytes per
// row, 2 KB); two stages take 4 KB, so the epilogue stages 16-row chunks
// (16 KB) and the LDS total is 148 KB.  The scale tensors are stored
// step-major ([R / 128][rows][4]), so a wave's scale load reads 256
// contiguous bytes; with row-major scales each load gathered 4 bytes from 64
// rows, and those loads cost the GEMM 20% (measured on MI355X, 7B-layer
// forward shapes: 2150-2380 against 2700-3020 TFLOP/s without them).
constexpr int kScStage = 2 * 256 * 4;
constexpr int kEpiRowsMx = 16;
constexpr int kGroupM = 8;                    // tile rows per raster group (the default)
constexpr int kBlockM = 8;                    // tile rows of a raster block (8 x 4 tiles: one XCD's round)
constexpr int kGroupMBigB = 24;               // tile rows per group when B exceeds the Infinity Cache
constexpr int64_t kInfinityCache = (int64_t)256 << 20;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt[5:4] at [15:14]); expcnt and lgkmcnt are left at their maxima.
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitVm16 = 0x4F70;
constexpr int kWaitVm18 = 0x4F72;
constexpr int kWaitVm12 = 0x0F7C;
constexpr int kWaitVm14 = 0x0F7E;
constexpr int kWaitVm24 = 0x4F78;

// Operand layouts.
constexpr int kKMajor = 0;
constexpr int kMNMajor = 1;

__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }
__device__ __forceinline__ int swz_mn(int r) { return (r & 7) | (((r >> 4) & 1) << 3); }

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

// 4-byte direct-to-LDS load (lane L writes LDS bytes [lds + 4 L, lds + 4 L + 4)):
// one row's four block scales of a reduction step.
__device__ __forceinline__ void dma4(uint32_t voff, const uint8_t* sbase, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}

// Global -> LDS sources of one operand for one wave.  A stage of an operand is
// filled by 8 loads per wave (1 KB each, load ii of wave w covering the LDS
// bytes (w * 8 + ii) * 1024 ..):
//   K-major: LDS rows (w * 8 + ii) * 8 + L / 8, lane L at physical chunk L % 8,
//            i.e. logical chunk (L % 8) ^ f(row); f depends on ii only through
//            ii & 1, so a lane keeps two offsets and the row step 8 ii R goes
//            into the uniform base.  Matrices with fewer than 256 rows (EDGE)
//            clamp each row to the last valid one instead.
//   MN-major: LDS rows (w * 8 + ii) * 4 + L / 16, lane L at physical chunk
//            L % 16, logical chunk (L % 16) ^ h(row); h depends on ii through
//            bits 0 and 2, so a lane keeps four offsets; the row step 4 ii LD
//            goes into the base.  Columns past the matrix (EDGE) are clamped
//            into those offsets.
struct OpSrc {
    const uint8_t* base;
    uint32_t off[4];
    uint32_t step;        // bytes between loads ii and ii + 1 (interior forms)
    uint32_t ld;          // leading dimension (K-major: R; MN-major: P or Q)
    int row, last;        // K-major EDGE: the lane's first row and the last valid row
};

struct Sources {
    OpSrc a, b;
    // block-scaled launches: scale tensors [R / 128][rows][4] (the four block scales
    // of a reduction step, for every row, contiguous) and the lane's row offsets
    // (wave w loads the scales of tile rows 64 w + lane of A and of B)
    const uint8_t* sa;
    const uint8_t* sb;
    uint32_t sa_off, sb_off;
    uint32_t sa_step, sb_step;  // bytes between the scales of consecutive reduction steps
};

// K-major: a wave fills `wave_rows` consecutive rows of the stage (64 for the
// 256-row operand tiles, 32 for the A operand of a 128-row half tile).
template <int L>
__device__ __forceinline__ void set_op(OpSrc& s, const uint8_t* base, int origin, int extent, int R, int wave,
                                       int lane, int wave_rows = 64)
{
    s.base = base;
    if (L == kKMajor) {
        s.ld = (uint32_t)R;
        s.step = 8u * (uint32_t)R;
        s.row = origin + wave * wave_rows + (lane >> 3);
        s.last = extent - 1;
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            const int row = wave * wave_rows + par * 8 + (lane >> 3);  // row within the tile
            const uint32_t c16 = (uint32_t)(((lane & 7) ^ swz(row)) * 16);
            s.off[par] = c16;                                         // EDGE form: chunk only
            s.off[par + 2] = (uint32_t)s.row * (uint32_t)R + c16;     // interior form
        }
    } else {
        s.ld = (uint32_t)extent;
        s.step = 4u * (uint32_t)extent;
        s.row = 0;
        s.last = 0;
#pragma unroll
        for (int idx = 0; idx < 4; ++idx) {
            // ii bit 0 -> row bit 2, ii bit 2 -> row bit 4 (see swz_mn)
            const int row = wave * 32 + (idx & 1) * 4 + (idx >> 1) * 16 + (lane >> 4);
            int col = origin + (((lane & 15) ^ swz_mn(row)) * 16);
            col = min(col, extent - 16);                            // only EDGE tiles reach past the end
            s.off[idx] = (uint32_t)(wave * 32 + (lane >> 4)) * (uint32_t)extent + (uint32_t)col;
        }
    }
}

// Load ii (0..7) of one operand for the k-step kt.
template <int L, bool EDGE>
__device__ __forceinline__ void issue_op(const OpSrc& s, uint32_t lds, int kt, int ii)
{
    if (L == kKMajor) {
        if (!EDGE) {
            dma16(s.off[2 + (ii & 1)], s.base + ((size_t)ii * s.step + (size_t)kt * kBK), lds);
        } else {
            const int row = min(s.row + ii * 8, s.last);
            dma16((uint32_t)row * s.ld + s.off[ii & 1], s.base + (size_t)kt * kBK, lds);
        }
    } else {
        const int idx = (ii & 1) | (((ii >> 2) & 1) << 1);
        dma16(s.off[idx], s.base + ((size_t)ii * s.step + (size_t)kt * kBK * s.ld), lds);
    }
}

// Load idx (0..15) of a stage: 0..7 fill A, 8..15 fill B.
template <bool EDGE, int LA, int LB>
__device__ __forceinline__ void issue_one(const Sources& src, uint32_t stage, int kt, int wave, int idx)
{
    const int ii = idx & 7;
    if (idx < 8) {
        const uint32_t lds = __builtin_amdgcn_readfirstlane(stage + (uint32_t)(wave * 8 + ii) * 1024u);
        issue_op<LA, EDGE>(src.a, lds, kt, ii);
    } else {
        const uint32_t lds = __builtin_amdgcn_readfirstlane(stage + (uint32_t)kStageA +
                                                            (uint32_t)(wave * 8 + ii) * 1024u);
        issue_op<LB, EDGE>(src.b, lds, kt, ii);
    }
}

template <bool EDGE, int LA, int LB>
__device__ __forceinline__ void issue_stage(const Sources& src, uint32_t stage, int kt, int wave)
{
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) issue_one<EDGE, LA, LB>(src, stage, kt, wave, idx);
}

// Block-scaled launches: the scale loads of a stage for one wave -- `which` 0: the
// scales of A rows 64 s .. 64 s + 63, 1: those of B rows (LDS: A rows at 4 r,
// B rows at 1024 + 4 r of the scale stage); s is the wave's slot (the wave
// itself, or wave % 2 for the 128 A rows of a half tile).
__device__ __forceinline__ void issue_scale(const Sources& src, uint32_t sc_stage, int kt, int s, int which)
{
    const uint32_t lds = __builtin_amdgcn_readfirstlane(sc_stage + (uint32_t)(which * 1024 + s * 256));
    if (which == 0)
        dma4(src.sa_off, src.sa + (size_t)kt * src.sa_step, lds);
    else
        dma4(src.sb_off, src.sb + (size_t)kt * src.sb_step, lds);
}

__device__ __forceinline__ void issue_stage_mx(const Sources& src, uint32_t stage, uint32_t sc_stage, int kt, int wave)
{
    issue_stage<false, kKMajor, kKMajor>(src, stage, kt, wave);
    issue_scale(src, sc_stage, kt, wave, 0);
    issue_scale(src, sc_stage, kt, wave, 1);
}

// Half tile (128 rows of A x 256 columns of B, K-major operands): a stage
// holds 16 KB of A (4 loads per wave) and the usual 32 KB of B (8 per wave).
// Load idx (0..11): 0..3 fill A, 4..11 fill B.
__device__ __forceinline__ void issue_half(const Sources& src, uint32_t stage, int kt, int wave, int idx)
{
    if (idx < 4) {
        const uint32_t lds = __builtin_amdgcn_readfirstlane(stage + (uint32_t)(wave * 4 + idx) * 1024u);
        issue_op<kKMajor, false>(src.a, lds, kt, idx);
    } else {
        const uint32_t lds = __builtin_amdgcn_readfirstlane(stage + (uint32_t)kStageA +
                                                            (uint32_t)(wave * 8 + idx - 4) * 1024u);
        issue_op<kKMajor, false>(src.b, lds, kt, idx - 4);
    }
}

__device__ __forceinline__ void issue_half_stage(const Sources& src, uint32_t stage, int kt, int wave)
{
#pragma unroll
    for (int idx = 0; idx < 12; ++idx) issue_half(src, stage, kt, wave, idx);
}

// A block-scaled half tile's stage: the 12 operand loads, then the scales of its
// 128 A rows (waves 0 and 1 load them; waves 2 and 3 load the same rows into the
// same LDS bytes again, so that every wave issues 14 loads per stage and one
// vmcnt count serves all of them) and of its 256 B rows.
__device__ __forceinline__ void issue_half_stage_mx(const Sources& src, uint32_t stage, uint32_t sc_stage, int kt,
                                                    int wave)
{
    issue_half_stage(src, stage, kt, wave);
    issue_scale(src, sc_stage, kt, wave & 1, 0);
    issue_scale(src, sc_stage, kt, wave, 1);
}

// Three-stage half tiles (48 KB stages, B at 16 KB): load idx (0..11), 0..3
// fill A, 4..11 fill B.
__device__ __forceinline__ void issue_half3(const Sources& src, uint32_t stage, int kt, int wave, int idx)
{
    if (idx < 4) {
        const uint32_t lds = __builtin_amdgcn_readfirstlane(stage + (uint32_t)(wave * 4 + idx) * 1024u);
        issue_op<kKMajor, false>(src.a, lds, kt, idx);
    } else {
        const uint32_t lds = __builtin_amdgcn_readfirstlane(stage + (uint32_t)kHalfA +
                                                            (uint32_t)(wave * 8 + idx - 4) * 1024u);
        issue_op<kKMajor, false>(src.b, lds, kt, idx - 4);
    }
}

__device__ __forceinline__ void issue_half3_stage(const Sources& src, uint32_t stage, int kt, int wave)
{
#pragma unroll
    for (int idx = 0; idx < 12; ++idx) issue_half3(src, stage, kt, wave, idx);
}

// Fragments of the 16x16x128 instruction: block b covers 16 rows of A (or of
// B), lane l holds row (l % 16) of the block and the reduction bytes
// 16 g .. 16 g + 15 and 64 + 16 g .. 64 + 16 g + 15 of the 128-byte step,
// g = l / 16 (the same mapping for both operands, so the order of the
// reduction within the instruction does not matter).  A wave owns 128 x 128
// outputs = 8 x 8 blocks; `blk` is the block's index within the tile (0..15).
__device__ __forceinline__ v8i frag_k(const uint8_t* tile, int blk, int lane)
{
    const int row = blk * 16 + (lane & 15);
    const int p = (lane >> 4) ^ swz(row);
    const uint4 lo = *reinterpret_cast<const uint4*>(tile + row * kBK + p * 16);
    const uint4 hi = *reinterpret_cast<const uint4*>(tile + row * kBK + (p ^ 4) * 16);
    v8i r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
}

// MN-major: the block is the 16-byte column chunk `blk` of the 256-byte rows.
// Lane l = 16 g + 2 t + e names row kb + t, bytes 8 e .. 8 e + 7 of that chunk,
// for kb = 16 g, 16 g + 8, 64 + 16 g, 64 + 16 g + 8; h(kb + t) = t | (g & 1) << 3.
__device__ __forceinline__ v8i frag_mn(const uint8_t* tile, int blk, int lane)
{
    const int g = lane >> 4, t = (lane & 15) >> 1, e = lane & 1;
    const int h = t | ((g & 1) << 3);
    // (blk ^ h) * 16 occupies address bits 4..7, which neither the 256-byte row
    // term, the 8-byte half nor the (1 KB-aligned) stage base touches: the
    // lane's address for block 0, XOR blk << 4, is the address for block blk.
    // The base is made opaque here, so the compiler computes that one XOR at each
    // read instead of holding the 16 addresses of every stage live across the
    // persistent loop (where it spilled them, and each reload waited for the
    // whole prefetch in flight)
    uint32_t base = (uint32_t)(uintptr_t)tile + (uint32_t)((16 * g + t) * 256 + h * 16 + 8 * e);
    asm volatile("" : "+v"(base));
    const uint32_t a = base ^ (uint32_t)(blk << 4);
    const lds_u8* q = (const lds_u8*)(uintptr_t)a;
    const v2i x0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(q));
    const v2i x1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(q + 8 * 256));
    const v2i x2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(q + 64 * 256));
    const v2i x3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(q + 72 * 256));
    v8i r;
    r[0] = x0[0]; r[1] = x0[1]; r[2] = x1[0]; r[3] = x1[1];
    r[4] = x2[0]; r[5] = x2[1]; r[6] = x3[0]; r[7] = x3[1];
    return r;
}

// The lane number from v_mbcnt in volatile assembly: a value the compiler cannot
// hoist out of a loop (see its uses).
__device__ __forceinline__ int opaque_lane()
{
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    return ln;
}

template <int L>
__device__ __forceinline__ v8i frag(const uint8_t* tile, int blk, int lane)
{
    if (L == kKMajor) return frag_k(tile, blk, lane);
    return frag_mn(tile, blk, lane);
}

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
template <int FA, int FB, int LA>
__device__ __forceinline__ void half0(v4f (&acc)[8][8], const v8i (&bq)[8], const v8i (&alo)[4], v8i (&ahi)[4],
                                      const uint8_t* stage, int wm, int lane)
{
#pragma unroll
    for (int t = 0; t < 32; ++t) {
        const int j = t >> 2, i = t & 3;
        mma16<FA, FB>(acc, alo[i], bq[j], i, j);
        if ((t & 7) == 1) ahi[t >> 3] = frag<LA>(stage, wm * 8 + 4 + (t >> 3), lane);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int FA, int FB, bool EDGE, int LA, int LB, bool NEXT>
__device__ __forceinline__ void half1(v4f (&acc)[8][8], v8i (&bq)[8], v8i (&alo)[4], const v8i (&ahi)[4],
                                      const Sources& src, uint32_t cur_addr, const uint8_t* nxt, int kt_issue,
                                      int wave, int wm, int wn, int lane)
{
#pragma unroll
    for (int t = 0; t < 32; ++t) {
        const int j = t >> 2, i = t & 3;
        mma16<FA, FB>(acc, ahi[i], bq[j], 4 + i, j);
        if (NEXT) {
            if (i == 3) bq[j] = frag<LB>(nxt + kStageA, wn * 8 + j, lane);
            if ((t & 7) == 1) alo[t >> 3] = frag<LA>(nxt, wm * 8 + (t >> 3), lane);
            if ((t & 1) == 0) issue_one<EDGE, LA, LB>(src, cur_addr, kt_issue, wave, t >> 1);
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

// The reduction of one tile whose first two stages have been issued: zero the
// accumulators, run the K loop, and return with every load of the tile landed
// and every wave done with the LDS stages.
template <int FA, int FB, bool EDGE, int LA, int LB>
__device__ __forceinline__ void tile_mainloop(v4f (&acc)[8][8], v8i (&bq)[8], v8i (&alo)[4], v8i (&ahi)[4],
                                              const Sources& src, uint8_t* lds, uint32_t lds_addr, int KT, int wave,
                                              int wm, int wn, int lane)
{
    // MN-major forms: the lane number taken afresh for every tile (volatile, so
    // neither it nor the fragment addresses derived from it are hoisted out of
    // the persistent loop, where the allocator spilled them and each reload
    // waited for the whole prefetch in flight)
    if (LA == kMNMajor || LB == kMNMajor) lane = opaque_lane();
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.0f;
    __builtin_amdgcn_s_waitcnt(kWaitVm16);    // stage 0 landed; stage 1's 16 loads may be in flight
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) bq[j] = frag<LB>(lds + kStageA, wn * 8 + j, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) alo[i] = frag<LA>(lds, wm * 8 + i, lane);
    half0<FA, FB, LA>(acc, bq, alo, ahi, lds, wm, lane);
    for (int kt = 0; kt + 1 < KT; ++kt) {
        const int cur = kt & 1;
        mid_step_barrier();
        half1<FA, FB, EDGE, LA, LB, true>(acc, bq, alo, ahi, src, lds_addr + cur * kStage, lds + (cur ^ 1) * kStage,
                                          min(kt + 2, KT - 1), wave, wm, wn, lane);
        half0<FA, FB, LA>(acc, bq, alo, ahi, lds + (cur ^ 1) * kStage, wm, lane);
    }
    mid_step_barrier();
    half1<FA, FB, EDGE, LA, LB, false>(acc, bq, alo, ahi, src, 0, lds, 0, wave, wm, wn, lane);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
}

// ---- block-scaled (MX) launches.  The matrix instruction takes, per lane, one
// E8M0 scale of its operand row (lane % 16 of the block) and reduction block
// (lane / 16: bytes 32 g .. 32 g + 31 of the step) for each operand, picked from
// a 32-bit register by a byte selector (op_sel) that is part of the instruction.
// A wave's scales of a step are packed four blocks per register: A blocks
// 4 h .. 4 h + 3 in sa[h] (byte i % 4), B blocks 4 h .. in sb[h].  (Measured on
// gfx950 with an in-bounds probe: byte 127 is 1.0, 255 gives NaN, and the scale
// of lane group g applies to the step's bytes 32 g .. 32 g + 31, which the
// fragment layout above -- chunks g and g + 4, i.e. bytes 16 g .. and
// 64 + 16 g .. -- feeds to the instruction in its own order.)
// The scale bytes a lane needs for one operand's 8 blocks of a step: rows
// 16 i + lane % 16 (i = 0..7, 64 bytes apart from the wave's first row), byte
// lane / 16 of each.  Loaded in one place and packed in a later one, so that
// the wait for these LDS reads (and for the fragment reads issued before them)
// comes a few matrix instructions after they are issued.
__device__ __forceinline__ void load_scale_bytes(const uint8_t* rows, int lane, uint32_t (&raw)[8])
{
    const uint8_t* p = rows + (lane & 15) * 4 + (lane >> 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) raw[i] = p[64 * i];
}

__device__ __forceinline__ void pack_scale_bytes(const uint32_t (&raw)[8], uint32_t (&s)[2])
{
#pragma unroll
    for (int h = 0; h < 2; ++h)
        s[h] = raw[4 * h] | (raw[4 * h + 1] << 8) | (raw[4 * h + 2] << 16) | (raw[4 * h + 3] << 24);
}

__device__ __forceinline__ void read_scales(const uint8_t* sc_stage, int wm, int wn, int lane, uint32_t (&sa)[2],
                                            uint32_t (&sb)[2])
{
    uint32_t raw[8];
    load_scale_bytes(sc_stage + wm * 512, lane, raw);
    pack_scale_bytes(raw, sa);
    load_scale_bytes(sc_stage + 1024 + wn * 512, lane, raw);
    pack_scale_bytes(raw, sb);
}

// Half tiles: a wave's 4 A blocks are rows 64 wm + 16 i + lane % 16 (i = 0..3),
// one scale register (sa[1] is a copy, never selected).
__device__ __forceinline__ void load_scale_bytes4(const uint8_t* rows, int lane, uint32_t (&raw)[4])
{
    const uint8_t* p = rows + (lane & 15) * 4 + (lane >> 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = p[64 * i];
}

__device__ __forceinline__ void pack_scale_bytes4(const uint32_t (&raw)[4], uint32_t (&s)[2])
{
    s[0] = raw[0] | (raw[1] << 8) | (raw[2] << 16) | (raw[3] << 24);
    s[1] = s[0];
}

__device__ __forceinline__ void read_scales_half(const uint8_t* sc_stage, int wm, int wn, int lane,
                                                 uint32_t (&sa)[2], uint32_t (&sb)[2])
{
    uint32_t r4[4], raw[8];
    load_scale_bytes4(sc_stage + wm * 256, lane, r4);
    pack_scale_bytes4(r4, sa);
    load_scale_bytes(sc_stage + 1024 + wn * 512, lane, raw);
    pack_scale_bytes(raw, sb);
}

template <int FA, int FB, int OA, int OB>
__device__ __forceinline__ v4f mfma_mx(const v8i& a, const v8i& b, const v4f& c, uint32_t sa, uint32_t sb)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, FB, FA, OB, (int)sb, OA, (int)sa);
}

// acc[i][j] += A block i x B block j with their scales (i, j are constants once
// the callers' loops are unrolled, so the switch folds to one instruction).
template <int FA, int FB>
__device__ __forceinline__ void mma16_mx(v4f (&acc)[8][8], const v8i& a, const v8i& b, int i, int j,
                                         const uint32_t (&sa)[2], const uint32_t (&sb)[2])
{
    const uint32_t xa = sa[i >> 2], xb = sb[j >> 2];
    v4f& c = acc[i][j];
    switch ((i & 3) * 4 + (j & 3)) {
#define FP8_MX_CASE(OA, OB) \
    case OA * 4 + OB: c = mfma_mx<FA, FB, OA, OB>(a, b, c, xa, xb); break;
        FP8_MX_CASE(0, 0) FP8_MX_CASE(0, 1) FP8_MX_CASE(0, 2) FP8_MX_CASE(0, 3)
        FP8_MX_CASE(1, 0) FP8_MX_CASE(1, 1) FP8_MX_CASE(1, 2) FP8_MX_CASE(1, 3)
        FP8_MX_CASE(2, 0) FP8_MX_CASE(2, 1) FP8_MX_CASE(2, 2) FP8_MX_CASE(2, 3)
        FP8_MX_CASE(3, 0) FP8_MX_CASE(3, 1) FP8_MX_CASE(3, 2) FP8_MX_CASE(3, 3)
#undef FP8_MX_CASE
    }
}

// The two halves of a step as half0 / half1 above, with the scales: sa / sb
// hold the step's, and half1 also reads the next step's into na / nb (from the
// next stage's scales, landed at the barrier before it) and issues the two
// scale loads of tile k + 2 beside its 16 operand loads (at t = 5 and 21:
// measured 1-3% faster than at t = 1 and 3, next to the first operand loads).
template <int FA, int FB>
__device__ __forceinline__ void half0_mx(v4f (&acc)[8][8], const v8i (&bq)[8], const v8i (&alo)[4], v8i (&ahi)[4],
                                         const uint8_t* stage, int wm, int lane, const uint32_t (&sa)[2],
                                         const uint32_t (&sb)[2])
{
#pragma unroll
    for (int t = 0; t < 32; ++t) {
        const int j = t >> 2, i = t & 3;
        mma16_mx<FA, FB>(acc, alo[i], bq[j], i, j, sa, sb);
        if ((t & 7) == 1) ahi[t >> 3] = frag_k(stage, wm * 8 + 4 + (t >> 3), lane);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int FA, int FB, bool NEXT>
__device__ __forceinline__ void half1_mx(v4f (&acc)[8][8], v8i (&bq)[8], v8i (&alo)[4], const v8i (&ahi)[4],
                                         const Sources& src, uint32_t cur_addr, uint32_t cur_sc, const uint8_t* nxt,
                                         const uint8_t* nxt_sc, int kt_issue, int wave, int wm, int wn, int lane,
                                         const uint32_t (&sa)[2], const uint32_t (&sb)[2], uint32_t (&na)[2],
                                         uint32_t (&nb)[2])
{
    uint32_t raw[8];
#pragma unroll
    for (int t = 0; t < 32; ++t) {
        const int j = t >> 2, i = t & 3;
        mma16_mx<FA, FB>(acc, ahi[i], bq[j], 4 + i, j, sa, sb);
        if (NEXT) {
            if (i == 3) bq[j] = frag_k(nxt + kStageA, wn * 8 + j, lane);
            if ((t & 7) == 1) alo[t >> 3] = frag_k(nxt, wm * 8 + (t >> 3), lane);
            if ((t & 1) == 0) issue_one<false, kKMajor, kKMajor>(src, cur_addr, kt_issue, wave, t >> 1);
            if (t == 5 || t == 21) issue_scale(src, cur_sc, kt_issue, wave, t == 5 ? 0 : 1);
            // the next step's scales: A bytes read at t = 2 and packed at t = 6,
            // B bytes read at t = 10 and packed at t = 14
            if (t == 2) load_scale_bytes(nxt_sc + wm * 512, lane, raw);
            if (t == 6) pack_scale_bytes(raw, na);
            if (t == 10) load_scale_bytes(nxt_sc + 1024 + wn * 512, lane, raw);
            if (t == 14) pack_scale_bytes(raw, nb);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The reduction of one block-scaled tile whose first two stages (operands and
// scales) have been issued; as tile_mainloop, with 18 loads per stage.
template <int FA, int FB>
__device__ __forceinline__ void tile_mainloop_mx(v4f (&acc)[8][8], v8i (&bq)[8], v8i (&alo)[4], v8i (&ahi)[4],
                                                 const Sources& src, uint8_t* lds, uint32_t lds_addr, uint8_t* sc,
                                                 uint32_t sc_addr, int KT, int wave, int wm, int wn, int lane)
{
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.0f;
    __builtin_amdgcn_s_waitcnt(kWaitVm18);    // stage 0 landed; stage 1's 18 loads may be in flight
    __syncthreads();
    uint32_t sa[2], sb[2], na[2], nb[2];
#pragma unroll
    for (int j = 0; j < 8; ++j) bq[j] = frag_k(lds + kStageA, wn * 8 + j, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) alo[i] = frag_k(lds, wm * 8 + i, lane);
    read_scales(sc, wm, wn, lane, sa, sb);
    half0_mx<FA, FB>(acc, bq, alo, ahi, lds, wm, lane, sa, sb);
    for (int kt = 0; kt + 1 < KT; ++kt) {
        const int cur = kt & 1;
        mid_step_barrier();
        half1_mx<FA, FB, true>(acc, bq, alo, ahi, src, lds_addr + cur * kStage, sc_addr + cur * kScStage,
                               lds + (cur ^ 1) * kStage, sc + (cur ^ 1) * kScStage, min(kt + 2, KT - 1), wave, wm,
                               wn, lane, sa, sb, na, nb);
        half0_mx<FA, FB>(acc, bq, alo, ahi, lds + (cur ^ 1) * kStage, wm, lane, na, nb);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            sa[h] = na[h];
            sb[h] = nb[h];
        }
    }
    mid_step_barrier();
    half1_mx<FA, FB, false>(acc, bq, alo, ahi, src, 0, 0, lds, sc, 0, wave, wm, wn, lane, sa, sb, na, nb);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
}

// Half tiles balance the last partial round of a launch (tiles that would
// leave most CUs idle are split into two 128-row halves, each a unit of work).
// A wave owns 64 x 128 outputs (A blocks 0..3 of its 64 rows, B blocks 0..7 of
// its 128 columns).  A step is 32 instructions (B block outer); interleaved
// with them: the next step's B block j is read into the registers of block j
// right after its last use, the next step's A blocks go to the other A buffer,
// and the 12 loads of tile k+2 are issued into the stage this step's fragments
// came from.  One barrier per step (after this wave's loads of tile k+1 are
// waited for) separates the reads of a stage from the loads that refill it.
template <int FA, int FB, bool NEXT>
__device__ __forceinline__ void half_step(v4f (&acc)[8][8], v8i (&bq)[8], const v8i (&ac)[4], v8i (&an)[4],
                                          const Sources& src, uint32_t cur_addr, const uint8_t* nxt, int kt_issue,
                                          int wave, int wm, int wn, int lane)
{
#pragma unroll
    for (int t = 0; t < 32; ++t) {
        const int j = t >> 2, i = t & 3;
        mma16<FA, FB>(acc, ac[i], bq[j], i, j);
        if (NEXT) {
            if (i == 3) bq[j] = frag_k(nxt + kStageA, wn * 8 + j, lane);
            if ((t & 7) == 1) an[t >> 3] = frag_k(nxt, wm * 4 + (t >> 3), lane);
            if ((t & 1) == 0 && t < 24) issue_half(src, cur_addr, kt_issue, wave, t >> 1);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int FA, int FB>
__device__ __forceinline__ void tile_mainloop_half(v4f (&acc)[8][8], v8i (&bq)[8], v8i (&a0)[4], v8i (&a1)[4],
                                                   const Sources& src, uint8_t* lds, uint32_t lds_addr, int KT,
                                                   int wave, int wm, int wn, int lane)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.0f;
    __builtin_amdgcn_s_waitcnt(kWaitVm12);    // stage 0 landed; stage 1's 12 loads may be in flight
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) bq[j] = frag_k(lds + kStageA, wn * 8 + j, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) a0[i] = frag_k(lds, wm * 4 + i, lane);
    int kt = 0;
    for (; kt + 2 < KT; kt += 2) {            // steps kt (even stage) and kt + 1 (odd stage)
        mid_step_barrier();
        half_step<FA, FB, true>(acc, bq, a0, a1, src, lds_addr, lds + kStage, kt + 2, wave, wm, wn, lane);
        mid_step_barrier();
        half_step<FA, FB, true>(acc, bq, a1, a0, src, lds_addr + kStage, lds, min(kt + 3, KT - 1), wave, wm, wn,
                                lane);
    }
    if (kt + 1 < KT) {                        // two steps left
        mid_step_barrier();
        half_step<FA, FB, true>(acc, bq, a0, a1, src, lds_addr, lds + kStage, KT - 1, wave, wm, wn, lane);
        mid_step_barrier();
        half_step<FA, FB, false>(acc, bq, a1, a0, src, 0, lds, 0, wave, wm, wn, lane);
    } else {                                  // one step left
        mid_step_barrier();
        half_step<FA, FB, false>(acc, bq, a0, a1, src, 0, lds, 0, wave, wm, wn, lane);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
}

// Half tiles with three 48 KB stages.  A step is the 32 instructions of
// half_step; interleaved with them the wave reads the next step's fragments
// (tile k+1) and issues the 12 loads of tile k+3 into the stage the current
// step's fragments came from, so each load has two steps to land (with two
// stages it had one, and the half tile's steps are half as long as a full
// tile's: its loads were late at every barrier).
template <int FA, int FB, bool NEXT>
__device__ __forceinline__ void half_step3(v4f (&acc)[8][8], v8i (&bq)[8], const v8i (&ac)[4], v8i (&an)[4],
                                           const Sources& src, uint32_t refill, const uint8_t* nxt, int kt_issue,
                                           int wave, int wm, int wn, int lane)
{
#pragma unroll
    for (int t = 0; t < 32; ++t) {
        const int j = t >> 2, i = t & 3;
        mma16<FA, FB>(acc, ac[i], bq[j], i, j);
        if (NEXT) {
            if (i == 3) bq[j] = frag_k(nxt + kHalfA, wn * 8 + j, lane);
            if ((t & 7) == 1) an[t >> 3] = frag_k(nxt, wm * 4 + (t >> 3), lane);
            if ((t & 1) == 0 && t < 24) issue_half3(src, refill, kt_issue, wave, t >> 1);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Before step k: tile k+1 has landed (this wave's loads: only the 12 of tile
// k+2 may be pending), and every wave has read the stage that step k refills.
__device__ __forceinline__ void half3_barrier()
{
    __builtin_amdgcn_s_waitcnt(kWaitVm12);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
}

// The reduction of one half tile whose first three stages (tiles 0, 1, 2,
// clamped to the last) have been issued into stages 0, 1, 2.  Tile k lives in
// stage k % 3; loads past the last tile re-load it into a stage that is not
// read again, so every step issues 12 loads and one vmcnt count serves all.
template <int FA, int FB>
__device__ __forceinline__ void tile_mainloop_half3(v4f (&acc)[8][8], v8i (&bq)[8], v8i (&a0)[4], v8i (&a1)[4],
                                                    const Sources& src, uint8_t* smem, uint32_t smem_addr, int KT,
                                                    int wave, int wm, int wn, int lane)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.0f;
    __builtin_amdgcn_s_waitcnt(kWaitVm24);    // tile 0 landed; the 24 loads of tiles 1 and 2 may be in flight
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) bq[j] = frag_k(smem + kHalfA, wn * 8 + j, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) a0[i] = frag_k(smem, wm * 4 + i, lane);
    int s0 = 0;                               // stage of tile kt
    int kt = 0;
    for (; kt + 2 < KT; kt += 2) {            // steps kt (A in a0) and kt + 1 (A in a1)
        const int s1 = s0 == 2 ? 0 : s0 + 1, s2 = s1 == 2 ? 0 : s1 + 1;
        half3_barrier();
        half_step3<FA, FB, true>(acc, bq, a0, a1, src, smem_addr + s0 * kHalfStage, smem + s1 * kHalfStage,
                                 min(kt + 3, KT - 1), wave, wm, wn, lane);
        half3_barrier();
        half_step3<FA, FB, true>(acc, bq, a1, a0, src, smem_addr + s1 * kHalfStage, smem + s2 * kHalfStage,
                                 min(kt + 4, KT - 1), wave, wm, wn, lane);
        s0 = s2;
    }
    if (kt + 1 < KT) {                        // two steps left
        const int s1 = s0 == 2 ? 0 : s0 + 1;
        half3_barrier();
        half_step3<FA, FB, true>(acc, bq, a0, a1, src, smem_addr + s0 * kHalfStage, smem + s1 * kHalfStage, KT - 1,
                                 wave, wm, wn, lane);
        half3_barrier();
        half_step3<FA, FB, false>(acc, bq, a1, a0, src, 0, smem, 0, wave, wm, wn, lane);
    } else {                                  // one step left
        half3_barrier();
        half_step3<FA, FB, false>(acc, bq, a0, a1, src, 0, smem, 0, wave, wm, wn, lane);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
}

// A block-scaled half tile: the steps of tile_mainloop_half with the scales of
// tile_mainloop_mx.  Each step also reads the next step's scales (from the stage
// that the step's barrier has seen land: A bytes at t = 2, packed at t = 6; B
// bytes at t = 10, packed at t = 14) and issues the two scale loads of the tile
// two steps ahead beside its 12 operand loads (at t = 5 and 21).
template <int FA, int FB, bool NEXT>
__device__ __forceinline__ void half_step_mx(v4f (&acc)[8][8], v8i (&bq)[8], const v8i (&ac)[4], v8i (&an)[4],
                                             const Sources& src, uint32_t cur_addr, uint32_t cur_sc,
                                             const uint8_t* nxt, const uint8_t* nxt_sc, int kt_issue, int wave,
                                             int wm, int wn, int lane, const uint32_t (&sa)[2],
                                             const uint32_t (&sb)[2], uint32_t (&na)[2], uint32_t (&nb)[2])
{
    uint32_t r4[4], raw[8];
#pragma unroll
    for (int t = 0; t < 32; ++t) {
        const int j = t >> 2, i = t & 3;
        mma16_mx<FA, FB>(acc, ac[i], bq[j], i, j, sa, sb);
        if (NEXT) {
            if (i == 3) bq[j] = frag_k(nxt + kStageA, wn * 8 + j, lane);
            if ((t & 7) == 1) an[t >> 3] = frag_k(nxt, wm * 4 + (t >> 3), lane);
            if ((t & 1) == 0 && t < 24) issue_half(src, cur_addr, kt_issue, wave, t >> 1);
            if (t == 5) issue_scale(src, cur_sc, kt_issue, wave & 1, 0);
            if (t == 21) issue_scale(src, cur_sc, kt_issue, wave, 1);
            if (t == 2) load_scale_bytes4(nxt_sc + wm * 256, lane, r4);
            if (t == 6) pack_scale_bytes4(r4, na);
            if (t == 10) load_scale_bytes(nxt_sc + 1024 + wn * 512, lane, raw);
            if (t == 14) pack_scale_bytes(raw, nb);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int FA, int FB>
__device__ __forceinline__ void tile_mainloop_half_mx(v4f (&acc)[8][8], v8i (&bq)[8], v8i (&a0)[4], v8i (&a1)[4],
                                                      const Sources& src, uint8_t* lds, uint32_t lds_addr,
                                                      uint8_t* sc, uint32_t sc_addr, int KT, int wave, int wm,
                                                      int wn, int lane)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.0f;
    __builtin_amdgcn_s_waitcnt(kWaitVm14);    // stage 0 landed; stage 1's 14 loads may be in flight
    __syncthreads();
    uint32_t sa[2], sb[2], na[2], nb[2];
#pragma unroll
    for (int j = 0; j < 8; ++j) bq[j] = frag_k(lds + kStageA, wn * 8 + j, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) a0[i] = frag_k(lds, wm * 4 + i, lane);
    read_scales_half(sc, wm, wn, lane, sa, sb);
    auto take = [&]() {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            sa[h] = na[h];
            sb[h] = nb[h];
        }
    };
    int kt = 0;
    for (; kt + 2 < KT; kt += 2) {            // steps kt (even stage) and kt + 1 (odd stage)
        mid_step_barrier();
        half_step_mx<FA, FB, true>(acc, bq, a0, a1, src, lds_addr, sc_addr, lds + kStage, sc + kScStage, kt + 2,
                                   wave, wm, wn, lane, sa, sb, na, nb);
        take();
        mid_step_barrier();
        half_step_mx<FA, FB, true>(acc, bq, a1, a0, src, lds_addr + kStage, sc_addr + kScStage, lds, sc,
                                   min(kt + 3, KT - 1), wave, wm, wn, lane, sa, sb, na, nb);
        take();
    }
    if (kt + 1 < KT) {                        // two steps left
        mid_step_barrier();
        half_step_mx<FA, FB, true>(acc, bq, a0, a1, src, lds_addr, sc_addr, lds + kStage, sc + kScStage, KT - 1,
                                   wave, wm, wn, lane, sa, sb, na, nb);
        take();
        mid_step_barrier();
        half_step_mx<FA, FB, false>(acc, bq, a1, a0, src, 0, 0, lds, sc, 0, wave, wm, wn, lane, sa, sb, na, nb);
    } else {                                  // one step left
        mid_step_barrier();
        half_step_mx<FA, FB, false>(acc, bq, a0, a1, src, 0, 0, lds, sc, 0, wave, wm, wn, lane, sa, sb, na, nb);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
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
    int la, lb;           // operand layouts
    int tiles_m, tiles_n;
    int group_m;          // tile rows per raster group
    int first_tile;
    const uint8_t* sa;    // block-scaled launches: E8M0 scales of A, [R / 128][P][4]
    const uint8_t* sb;    // and of B, [R / 128][Q][4]
};

struct GemmGroup {
    GemmProblem p[kMaxGroup];
    uint32_t* absmax_h;   // gate/up launches: the SwiGLU absmax accumulator (fp32 bits)
    const float* table;   // gate/up launches: the s_g table (bf16 exponents kGuELo - 3 .. 133)
    int count;
    int total_tiles;
    int full_units;       // units 0 .. full_units - 1 are the tiles of the same index; unit
                          // full_units + 2 k + h is half h of tile full_units + k
    int first_unit;       // this launch walks units first_unit .. units - 1
    int units;
};

// Everything a workgroup needs about its current tile (all wave-uniform).
struct Work {
    const uint8_t* A;
    const uint8_t* B;
    uint16_t* out;
    int prob;       // index of the tile's problem in the group
    int P, Q, R, KT;
    int la, lb;
    int ms, ns;     // logical origin (first row / column this tile stores)
    int m0, n0;     // origin actually computed (shifted back inside the matrix)
};

// Output tile of a virtual tile id: the problem it falls in, then a grouped
// raster order within it: groups of group_m tile rows, top to bottom; within a
// group, blocks of (up to) kBlockM rows x 4 columns, column blocks left to right
// and the blocks of a column block top to bottom; within a block, column-major.
// So the 32 consecutive ids an XCD takes in a round are one 8 x 4 block (12
// panels through its L2), and a group taller than a block spreads a round over
// several block rows (more rows, fewer columns: fewer passes over B).  For
// group_m <= kBlockM this is plain column-major order within the group.
template <bool EDGE, bool HALF, bool GU>
__device__ __forceinline__ Work work_of(const GemmGroup& g, int u)
{
    int v = u, hh = -1;
    if (HALF) {
        v = g.full_units + ((u - g.full_units) >> 1);
        hh = (u - g.full_units) & 1;
    }
    const bool second = g.count > 1 && v >= g.p[1].first_tile;
    const GemmProblem& pr = second ? g.p[1] : g.p[0];
    Work w;
    w.A = pr.A;
    w.B = pr.B;
    w.out = pr.out;
    w.prob = second;
    w.P = pr.P;
    w.Q = pr.Q;
    w.R = pr.R;
    w.KT = pr.R / kBK;
    w.la = pr.la;
    w.lb = pr.lb;
    const int lv = v - pr.first_tile;
    const int group_size = pr.group_m * pr.tiles_n;
    const int group = lv / group_size;
    const int first_m = group * pr.group_m;
    const int gm = min(pr.tiles_m - first_m, pr.group_m);
    const int in_group = lv - group * group_size;
    const int cb = in_group / (4 * gm);                   // column block
    const int r1 = in_group - cb * 4 * gm;
    const int wcb = min(4, pr.tiles_n - 4 * cb);           // its width (the last may be narrower)
    const int bh = min(kBlockM, gm);
    const int rb = r1 / (bh * wcb);                        // block within the column block
    const int r2 = r1 - rb * bh * wcb;
    const int hrb = min(bh, gm - rb * bh);                 // its height
    w.ms = (first_m + rb * bh + r2 % hrb) * kBM;
    w.ns = (4 * cb + r2 / hrb) * (GU ? kBN / 2 : kBN);   // gate/up: 128 gate columns per tile
    if (HALF) w.ms += hh * (kBM / 2);
    // A last partial tile is shifted back to end at the matrix edge (P, Q >= 256),
    // recomputing rows / columns of its neighbour that it then does not store
    // (a half tile that starts past the last row stores nothing).
    w.m0 = EDGE ? w.ms : min(w.ms, w.P - (HALF ? kBM / 2 : kBM));
    w.n0 = (EDGE || GU) ? w.ns : min(w.ns, w.Q - kBN);
    return w;
}

template <int LA, int LB>
__device__ __forceinline__ void set_sources(Sources& src, const Work& w, int wave, int lane)
{
    set_op<LA>(src.a, w.A, w.m0, w.P, w.R, wave, lane);
    set_op<LB>(src.b, w.B, w.n0, w.Q, w.R, wave, lane);
}

// Operand-layout sets a kernel is compiled for: every problem of a launch uses
// one of the set's (A, B) layout pairs.
constexpr int kSetKK = 0;       // (K, K)
constexpr int kSetMN = 1;       // (K, MN) and (MN, MN)

// Set up the sources of tile w and issue its first two stages.
template <bool EDGE, int SET, bool HALF, bool GU>
__device__ __forceinline__ void start_tile(Sources& src, const Work& w, uint32_t lds_addr, int wave, int lane)
{
    // Gate/up launches (B = [gate rows | up rows], F = Q / 2 each): wave w fills
    // B tile rows 64 w .. 64 w + 63 from the gate panel (w even) or the up panel
    // (w odd) at gate column n0 + 64 (w / 2), so the B blocks 0..3 of a wave are
    // gate columns and blocks 4..7 the up columns of the same outputs.
    const int b_origin = GU ? w.n0 + (wave >> 1) * 64 + (wave & 1) * (w.Q >> 1) - wave * 64 : w.n0;
    if (SET == kSetMN) lane = opaque_lane();  // as in tile_mainloop: no lane constants held across tiles
    if (HALF && !GU) {                        // three 48 KB stages
        set_op<kKMajor>(src.a, w.A, w.m0, w.P, w.R, wave, lane, 32);
        set_op<kKMajor>(src.b, w.B, b_origin, w.Q, w.R, wave, lane);
        issue_half3_stage(src, lds_addr, 0, wave);
        issue_half3_stage(src, lds_addr + kHalfStage, min(1, w.KT - 1), wave);
        issue_half3_stage(src, lds_addr + 2 * kHalfStage, min(2, w.KT - 1), wave);
    } else if (HALF) {
        set_op<kKMajor>(src.a, w.A, w.m0, w.P, w.R, wave, lane, 32);
        set_op<kKMajor>(src.b, w.B, b_origin, w.Q, w.R, wave, lane);
        issue_half_stage(src, lds_addr, 0, wave);
        issue_half_stage(src, lds_addr + kStage, min(1, w.KT - 1), wave);
    } else if (GU) {
        set_op<kKMajor>(src.a, w.A, w.m0, w.P, w.R, wave, lane);
        set_op<kKMajor>(src.b, w.B, b_origin, w.Q, w.R, wave, lane);
        issue_stage<false, kKMajor, kKMajor>(src, lds_addr, 0, wave);
        issue_stage<false, kKMajor, kKMajor>(src, lds_addr + kStage, min(1, w.KT - 1), wave);
    } else if (SET == kSetKK) {
        set_sources<kKMajor, kKMajor>(src, w, wave, lane);
        issue_stage<EDGE, kKMajor, kKMajor>(src, lds_addr, 0, wave);
        issue_stage<EDGE, kKMajor, kKMajor>(src, lds_addr + kStage, min(1, w.KT - 1), wave);
    } else if (w.la == kMNMajor) {
        set_sources<kMNMajor, kMNMajor>(src, w, wave, lane);
        issue_stage<EDGE, kMNMajor, kMNMajor>(src, lds_addr, 0, wave);
        issue_stage<EDGE, kMNMajor, kMNMajor>(src, lds_addr + kStage, min(1, w.KT - 1), wave);
    } else {
        set_sources<kKMajor, kMNMajor>(src, w, wave, lane);
        issue_stage<EDGE, kKMajor, kMNMajor>(src, lds_addr, 0, wave);
        issue_stage<EDGE, kKMajor, kMNMajor>(src, lds_addr + kStage, min(1, w.KT - 1), wave);
    }
}

// Block-scaled launches (K-major operands, tiles inside the matrices): set up
// the sources of unit w (a tile, or a 128-row half tile) and issue its first
// two stages with their scales.
template <bool HALF>
__device__ __forceinline__ void start_tile_mx(Sources& src, const GemmGroup& g, const Work& w, uint32_t lds_addr,
                                              uint32_t sc_addr, int wave, int lane)
{
    const GemmProblem& pr = w.prob ? g.p[1] : g.p[0];
    if (HALF)
        set_op<kKMajor>(src.a, w.A, w.m0, w.P, w.R, wave, lane, 32);
    else
        set_op<kKMajor>(src.a, w.A, w.m0, w.P, w.R, wave, lane);
    set_op<kKMajor>(src.b, w.B, w.n0, w.Q, w.R, wave, lane);
    src.sa = pr.sa;
    src.sb = pr.sb;
    // the lane number recomputed here (volatile, so it is not hoisted): held live
    // across the persistent loop, the allocator spilled it, and the reload's wait
    // here was a wait for the whole first stage just issued
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    // one row's 4 scales of a step; a half tile's 128 A rows are loaded by
    // waves 0 and 1 and again, identically, by waves 2 and 3
    src.sa_off = (uint32_t)(w.m0 + (HALF ? (wave & 1) : wave) * 64 + ln) * 4u;
    src.sb_off = (uint32_t)(w.n0 + wave * 64 + ln) * 4u;
    src.sa_step = (uint32_t)w.P * 4u;
    src.sb_step = (uint32_t)w.Q * 4u;
    if (HALF) {
        issue_half_stage_mx(src, lds_addr, sc_addr, 0, wave);
        issue_half_stage_mx(src, lds_addr + kStage, sc_addr + kScStage, min(1, w.KT - 1), wave);
    } else {
        issue_stage_mx(src, lds_addr, sc_addr, 0, wave);
        issue_stage_mx(src, lds_addr + kStage, sc_addr + kScStage, min(1, w.KT - 1), wave);
    }
}

// A 16-byte output store; NT: non-temporal, for the backward products' dX and dW:
// kept out of the caches, they do not displace the operand panels that the XCDs
// keep re-fetching (measured on the 7B-layer step: 1.1% shorter, the backward
// calls 2-3% faster).
template <bool NT>
__device__ __forceinline__ void store16(uint8_t* p, const uint4& v)
{
    if (NT)
        __builtin_nontemporal_store(u32x4v{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4v*>(p));
    else
        *reinterpret_cast<uint4*>(p) = v;
}

// Epilogue of a finished tile: descale and round to bf16, stage 32-row chunks of
// the wave's tile (8 A blocks x 128 columns, 4 for a half tile) in its private
// LDS region (16-byte chunks of a 256-byte row XOR-swizzled by row), read back
// 16 bytes per lane and store four full 256-byte row segments per instruction.
template <bool HALF, bool NT>
__device__ __forceinline__ void epilogue(const v4f (&acc)[8][8], const Work& done, float d, uint8_t* epi, int wave,
                                         int wm, int wn, int lane)
{
    uint8_t* ew = epi + wave * kEpiWave;
    // The LDS addresses below depend only on the lane; computing them here from
    // an opaque copy of it keeps the compiler from holding ~40 of them live
    // across the whole persistent loop (where they would spill).
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int r16 = ln & 15, q4 = ln >> 4;
    const int wrow = done.m0 + wm * (HALF ? 64 : 128);
    // a tile that is not shifted back and lies inside the matrix stores every output it computes
    const bool full = done.ms == done.m0 && done.ns == done.n0 && done.m0 + (HALF ? kBM / 2 : kBM) <= done.P &&
                      done.n0 + kBN <= done.Q;
#pragma unroll
    for (int c2 = 0; c2 < (HALF ? 2 : 4); ++c2) {        // chunk: A blocks 2*c2, 2*c2+1 (32 rows)
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
        if (full) {
            // every row and column is the tile's own: the chunk's 8 LDS reads go
            // out together, then 8 stores through a uniform base plus a per-lane
            // offset (no per-store bounds test, branch or 64-bit address math)
            static_assert(kEpiRows == 32, "8 row groups of 4 per chunk");
            auto rd = [&](int it) {
                const int rr = it * 4 + q4;
                return *reinterpret_cast<const uint4*>(ew + rr * 256 + ((r16 ^ (rr & 15)) * 16));
            };
            const uint4 o0 = rd(0), o1 = rd(1), o2 = rd(2), o3 = rd(3), o4 = rd(4), o5 = rd(5), o6 = rd(6),
                        o7 = rd(7);
            uint8_t* base = reinterpret_cast<uint8_t*>(done.out) +
                            ((size_t)(wrow + c2 * 32) * done.Q + done.n0 + wn * 128) * 2;
            const uint32_t loff = (uint32_t)(q4 * done.Q + r16 * 8) * 2u;
            const size_t rs = (size_t)8 * done.Q;                 // 4 rows, in bytes
            store16<NT>(base + loff, o0);
            store16<NT>(base + rs + loff, o1);
            store16<NT>(base + 2 * rs + loff, o2);
            store16<NT>(base + 3 * rs + loff, o3);
            store16<NT>(base + 4 * rs + loff, o4);
            store16<NT>(base + 5 * rs + loff, o5);
            store16<NT>(base + 6 * rs + loff, o6);
            store16<NT>(base + 7 * rs + loff, o7);
        } else {
#pragma unroll
            for (int it = 0; it < kEpiRows / 4; ++it) {
                const int rr = it * 4 + q4;                       // row within the chunk
                const int c = r16;                                // logical 16-byte chunk
                const uint4 o = *reinterpret_cast<const uint4*>(ew + rr * 256 + ((c ^ (rr & 15)) * 16));
                const int m = wrow + c2 * 32 + rr;
                const int n = done.n0 + wn * 128 + c * 8;
                if (m >= done.ms && m < done.P && n >= done.ns && n < done.Q)
                    store16<NT>(reinterpret_cast<uint8_t*>(done.out + (size_t)m * done.Q + n), o);
            }
        }
    }
}

// Epilogue staging 16-row chunks (one A block) in a 4 KB LDS region per wave:
// the block-scaled tiles (no descale: the block scales are inside the sums) and
// the three-stage half tiles (DESCALE: the per-tensor factor d, as epilogue()).
template <bool HALF, bool NT, bool DESCALE>
__device__ __forceinline__ void epilogue16(const v4f (&acc)[8][8], const Work& done, float d, uint8_t* epi, int wave,
                                           int wm, int wn, int lane)
{
    uint8_t* ew = epi + wave * (kEpiRowsMx * 256);
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int r16 = ln & 15, q4 = ln >> 4;
    const int wrow = done.m0 + wm * (HALF ? 64 : 128);
    const bool full = done.ms == done.m0 && done.ns == done.n0 && done.m0 + (HALF ? kBM / 2 : kBM) <= done.P &&
                      done.n0 + kBN <= done.Q;
#pragma unroll
    for (int i = 0; i < (HALF ? 4 : 8); ++i) {             // chunk: A block i (16 rows)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const f32x2 v01 = DESCALE ? f32x2{acc[i][j][0] * d, acc[i][j][1] * d} : f32x2{acc[i][j][0], acc[i][j][1]};
            const f32x2 v23 = DESCALE ? f32x2{acc[i][j][2] * d, acc[i][j][3] * d} : f32x2{acc[i][j][2], acc[i][j][3]};
            uint2 o;
            o.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(v01, bf16x2));
            o.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(v23, bf16x2));
            const int chunk = (2 * j + (q4 >> 1)) ^ r16;
            *reinterpret_cast<uint2*>(ew + r16 * 256 + chunk * 16 + (q4 & 1) * 8) = o;
        }
        if (full) {
            auto rd = [&](int it) {
                const int rr = it * 4 + q4;
                return *reinterpret_cast<const uint4*>(ew + rr * 256 + ((r16 ^ rr) * 16));
            };
            const uint4 o0 = rd(0), o1 = rd(1), o2 = rd(2), o3 = rd(3);
            uint8_t* base = reinterpret_cast<uint8_t*>(done.out) +
                            ((size_t)(wrow + i * 16) * done.Q + done.n0 + wn * 128) * 2;
            const uint32_t loff = (uint32_t)(q4 * done.Q + r16 * 8) * 2u;
            const size_t rs = (size_t)8 * done.Q;                 // 4 rows, in bytes
            store16<NT>(base + loff, o0);
            store16<NT>(base + rs + loff, o1);
            store16<NT>(base + 2 * rs + loff, o2);
            store16<NT>(base + 3 * rs + loff, o3);
        } else {
#pragma unroll
            for (int it = 0; it < kEpiRowsMx / 4; ++it) {
                const int rr = it * 4 + q4;
                const uint4 o = *reinterpret_cast<const uint4*>(ew + rr * 256 + ((r16 ^ rr) * 16));
                const int m = wrow + i * 16 + rr;
                const int n = done.n0 + wn * 128 + r16 * 8;
                if (m >= done.ms && m < done.P && n >= done.ns && n < done.Q)
                    store16<NT>(reinterpret_cast<uint8_t*>(done.out + (size_t)m * done.Q + n), o);
            }
        }
    }
}

// ---- gate/up launches: the SwiGLU statistic in the epilogue ("LLMQ", section
// 3.1: the forward computes absmax_h, which recomputation later reuses; here it
// comes out of the GEMM that produces [gate | up], saving the separate read
// pass over that output).  h = RN32(s_g * u) on the bf16 values as stored, with
// s_g = RN32(g / RN32(1 + RN32(e^-g))) read from the SwiGLU kernels' table for
// the bf16 exponents kGuELo .. kSiluEHi (31 KB, held in the LDS that other
// launches use to stage output rows) and exact rules elsewhere:
//   exponent < kGuELo: s_g = g / 2 (1 + e^-g rounds to exactly 2 there; the
//                      table's entries for exponents kSiluELo .. kGuELo - 1
//                      are g / 2 as well);
//   |g| >= 128 (and inf, NaN): s_g = g for g > 0, -0 for finite g < 0, NaN for
//                      -inf and negative NaN.
constexpr int kGuELo = 103;
constexpr int kGuHalf = (kSiluEHi - kGuELo + 1) * 128;           // entries per sign
constexpr int kSiluHalf = (kSiluEHi - kSiluELo + 1) * 128;       // source table, entries per sign
static_assert(2 * kGuHalf * 4 + 4 <= 4 * kEpiWave, "table and the maximum slot must fit the epilogue LDS");

__device__ __forceinline__ void load_gu_table(float* dst, const float* src, int tid)
{
    constexpr int kV = kGuHalf / 4;                                // float4 per sign
    for (int k = tid; k < 2 * kV; k += 256) {
        const int sgn = k >= kV;
        const int r = k - sgn * kV;
        reinterpret_cast<float4*>(dst)[k] =
            reinterpret_cast<const float4*>(src)[(sgn * kSiluHalf + (kGuELo - kSiluELo) * 128) / 4 + r];
    }
}

// Early returns, not selects: almost every gate value of real data is in the
// table's range, so the rule branches are skipped by whole waves (a branch-free
// form that evaluates every rule for every value measured slower).
__device__ __forceinline__ float s_g_of(const float* tbl, uint32_t b)
{
    const float g = __uint_as_float(b << 16);
    const uint32_t t = (b & 0x7FFFu) - (uint32_t)(kGuELo * 128);
    const uint32_t neg = b >> 15;
    const bool in_table = t < (uint32_t)kGuHalf;
    const float tv = tbl[in_table ? t + neg * kGuHalf : 0u];
    if (in_table) return tv;
    if ((int32_t)t < 0) return g * 0.5f;
    if (!neg) return g;
    return ((b & 0x7F80u) == 0x7F80u) ? __builtin_nanf("") : -0.0f;
}

// Epilogue of a gate/up tile: B blocks 0..3 of the wave are gate columns
// n0 + 64 wn + 16 j .., blocks 4..7 the up columns F + (the same); each lane
// holds 4 consecutive columns of one row.  Stores go straight from registers
// (8 bytes per lane; swapping halves between lanes for 16-byte stores measured
// no faster); every computed row enters the maximum of |h| bit patterns
// (rows that a shifted-back tile recomputes but does not store are its
// neighbour's values).  The wave's maximum goes into the workgroup's LDS slot
// `wg_max`; global memory sees one atomic per workgroup, after the last tile
// (an atomic per tile would sit in the vector-memory counter in front of the
// next tile's loads and stall its first wait, and a register held across the
// K loop would be spilled).
template <bool HALF>
__device__ __forceinline__ void epilogue_gu(const v4f (&acc)[8][8], const Work& done, float d, const float* tbl,
                                            uint32_t* wg_max, int wm, int wn, int lane)
{
    uint32_t mx = 0;
    const int F = done.Q >> 1;
    // the lane number recomputed here (volatile, so it is not hoisted), so that
    // no per-lane term is held live across the persistent loop (where it would
    // be spilled)
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    const int r16 = ln & 15, q4 = ln >> 4;
#pragma unroll
    for (int i = 0; i < (HALF ? 4 : 8); ++i) {
        const int m = done.m0 + wm * (HALF ? 64 : 128) + i * 16 + r16;
        uint16_t* row = done.out + (size_t)m * done.Q;
        const bool st = m >= done.ms;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x2 g01 = {acc[i][j][0] * d, acc[i][j][1] * d};
            const f32x2 g23 = {acc[i][j][2] * d, acc[i][j][3] * d};
            const f32x2 u01 = {acc[i][j + 4][0] * d, acc[i][j + 4][1] * d};
            const f32x2 u23 = {acc[i][j + 4][2] * d, acc[i][j + 4][3] * d};
            uint2 go, uo;
            go.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(g01, bf16x2));
            go.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(g23, bf16x2));
            uo.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(u01, bf16x2));
            uo.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(u23, bf16x2));
            const int c = done.n0 + wn * 64 + j * 16 + 4 * q4;
            if (st) {
                *reinterpret_cast<uint2*>(row + c) = go;
                *reinterpret_cast<uint2*>(row + F + c) = uo;
            }
            const uint32_t gb[4] = {go.x & 0xFFFFu, go.x >> 16, go.y & 0xFFFFu, go.y >> 16};
            const uint32_t ub[4] = {uo.x << 16, uo.x & 0xFFFF0000u, uo.y << 16, uo.y & 0xFFFF0000u};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float h = s_g_of(tbl, gb[e]) * __uint_as_float(ub[e]);
                const uint32_t a = __float_as_uint(h) & 0x7FFFFFFFu;
                mx = mx > a ? mx : a;
            }
        }
        __builtin_amdgcn_sched_barrier(0);    // one row block at a time: bounded register use
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)mx, off, 64);
        mx = mx > o ? mx : o;
    }
    if (ln == 0) atomicMax(wg_max, mx);
}

// Persistent kernel: one workgroup per CU walks the units v = slot, slot + G,
// slot + 2G, ... (a unit is a tile, or a half tile in a balanced last round)
// where slot renumbers the workgroups XCD-major (workgroups are dealt
// round-robin to the 8 XCDs, each with its own L2), so in every round the 32
// CUs of one XCD work on 32 consecutive units of the raster order.  While a
// tile's epilogue stores run, the first two stages of the next tile are
// already loading.
template <int FA, int FB, bool EDGE, int SET, bool HALF, bool GU, bool NT>
__global__ void __launch_bounds__(256, 1) gemm_tn_kernel(const GemmGroup g)
{
    // full tiles: two 64 KB stages, then 32 KB of epilogue staging; half tiles
    // (not gate/up): three 48 KB stages, then 16 KB of epilogue staging
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kLds + 4 * kEpiWave];
    uint8_t* const lds = smem;
    uint8_t* const epi = smem + kLds;
    constexpr bool kHalf3 = HALF && !GU;

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

    int v = g.first_unit + slot;
    if (v >= g.units) return;
    // The descale factors are loaded once, here, ahead of every direct-to-LDS
    // load, and first used after a K loop (whose final wait has drained all
    // loads).  The compiler does not see the inline-assembly loads: a wait of
    // its own for a plain load issued after them (e.g. in the epilogue) would
    // be a full vmcnt(0), i.e. a wait for the next tile's whole prefetch.
    const float d0 = g.p[0].inv_a[0] * g.p[0].inv_b[0];
    const float d1 = g.count > 1 ? g.p[1].inv_a[0] * g.p[1].inv_b[0] : d0;
    Work w = work_of<EDGE, HALF, GU>(g, v);
    start_tile<EDGE, SET, HALF, GU>(src, w, lds_addr, wave, lane);
    // gate/up: the s_g table and, after it, the workgroup's running max of |h|
    // (both read only after the first K loop's barriers)
    uint32_t* wg_max = reinterpret_cast<uint32_t*>(epi + 2 * kGuHalf * 4);
    if (GU) {
        load_gu_table(reinterpret_cast<float*>(epi), g.table, tid);
        if (tid == 0) *wg_max = 0;
    }
    for (;;) {
        if (kHalf3)
            tile_mainloop_half3<FA, FB>(acc, bq, alo, ahi, src, lds, lds_addr, w.KT, wave, wm, wn, lane);
        else if (HALF)
            tile_mainloop_half<FA, FB>(acc, bq, alo, ahi, src, lds, lds_addr, w.KT, wave, wm, wn, lane);
        else if (SET == kSetKK)
            tile_mainloop<FA, FB, EDGE, kKMajor, kKMajor>(acc, bq, alo, ahi, src, lds, lds_addr, w.KT, wave, wm, wn,
                                                          lane);
        else if (w.la == kMNMajor)
            tile_mainloop<FA, FB, EDGE, kMNMajor, kMNMajor>(acc, bq, alo, ahi, src, lds, lds_addr, w.KT, wave, wm,
                                                            wn, lane);
        else
            tile_mainloop<FA, FB, EDGE, kKMajor, kMNMajor>(acc, bq, alo, ahi, src, lds, lds_addr, w.KT, wave, wm, wn,
                                                           lane);

        float d = w.prob ? d1 : d0;
        asm volatile("" : "+v"(d));           // materialised here, before the next prefetch
        const Work done = w;
        const int next = v + G;
        if (next < g.units) {
            v = next;
            w = work_of<EDGE, HALF, GU>(g, v);
            start_tile<EDGE, SET, HALF, GU>(src, w, lds_addr, wave, lane);
        }

        if (GU)
            epilogue_gu<HALF>(acc, done, d, reinterpret_cast<const float*>(epi), wg_max, wm, wn, lane);
        else if (kHalf3)
            epilogue16<true, NT, true>(acc, done, d, smem + kHalfEpi, wave, wm, wn, lane);
        else
            epilogue<HALF, NT>(acc, done, d, epi, wave, wm, wn, SET == kSetMN ? opaque_lane() : lane);
        // The loop-top wait (vmcnt <= 16, or 12 / 24 for a half tile) then proves
        // the next tile's first stage has landed: if one of its loads were
        // pending, the 16 (12, 24) later loads of the following stages would be
        // too (loads complete in order), whatever the interleaved stores do.
        if (next >= g.units) break;
    }
    if (GU) {
        __syncthreads();
        if (tid == 0) atomicMax(g.absmax_h, *wg_max);
    }
}

// Block-scaled (MX) products: the persistent walk of gemm_tn_kernel (XCD-major
// slots, grouped raster, problem groups, next tile's first stages issued before
// the epilogue, a balanced last round of half tiles in a launch of its own:
// HALF) over tiles of K-major operands, with each operand row's E8M0 block
// scales loaded beside its codes and applied by the matrix instruction; the
// output is the bf16 of the fp32 sums (no per-tensor factor).
template <int FA, int FB, bool HALF, bool NT>
__global__ void __launch_bounds__(256, 1) gemm_mx_kernel(const GemmGroup g)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];
    __shared__ __attribute__((aligned(1024))) uint8_t epi[4 * kEpiRowsMx * 256];
    __shared__ __attribute__((aligned(1024))) uint8_t sc[2 * kScStage];

    const int G = gridDim.x;
    int slot = blockIdx.x;
    if (G % 8 == 0) slot = (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;
    const uint32_t sc_addr = (uint32_t)(uintptr_t)sc;

    Sources src;
    v8i bq[8], alo[4], ahi[4];
    v4f acc[8][8];

    int v = g.first_unit + slot;
    if (v >= g.units) return;
    Work w = work_of<false, HALF, false>(g, v);
    start_tile_mx<HALF>(src, g, w, lds_addr, sc_addr, wave, lane);
    for (;;) {
        if (HALF)
            tile_mainloop_half_mx<FA, FB>(acc, bq, alo, ahi, src, lds, lds_addr, sc, sc_addr, w.KT, wave, wm, wn,
                                          lane);
        else
            tile_mainloop_mx<FA, FB>(acc, bq, alo, ahi, src, lds, lds_addr, sc, sc_addr, w.KT, wave, wm, wn, lane);
        const Work done = w;
        const int next = v + G;
        if (next < g.units) {
            v = next;
            w = work_of<false, HALF, false>(g, v);
            start_tile_mx<HALF>(src, g, w, lds_addr, sc_addr, wave, lane);
        }
        epilogue16<HALF, NT, false>(acc, done, 1.0f, epi, wave, wm, wn, lane);
        // the loop-top wait (vmcnt <= 18, or 14 for a half tile) then proves the
        // next unit's first stage has landed, as in gemm_tn_kernel
        if (next >= g.units) break;
    }
}

static GemmProblem make_problem(const uint8_t* A, int la, const uint8_t* B, int lb, const float* inv_a,
                                const float* inv_b, void* out, int64_t P, int64_t Q, int64_t R)
{
    GemmProblem p{};
    p.A = A;
    p.B = B;
    p.inv_a = inv_a;
    p.inv_b = inv_b;
    p.out = reinterpret_cast<uint16_t*>(out);
    p.P = (int)P;
    p.Q = (int)Q;
    p.R = (int)R;
    p.la = la;
    p.lb = lb;
    p.tiles_m = (int)((P + kBM - 1) / kBM);
    p.tiles_n = (int)((Q + kBN - 1) / kBN);
    // A B operand larger than the Infinity Cache is re-read from HBM by every
    // group: taller groups read it fewer times.  Measured on MI355X, the 32B-class
    // gate/up forward (16384 x 55296 x 5120, B 283 MB) took 3582 / 3493 / 3385 /
    // 3334 / 3432 us with groups of 8 / 16 / 20 / 24 / 32 tile rows; no other
    // product of the 7B-, 14B- and 32B-class layers has such a B.
    p.group_m = Q * R > kInfinityCache ? kGroupMBigB : kGroupM;
    p.first_tile = 0;
    return p;
}

template <int FA, int FB, int SET, bool GU, bool NT>
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
    const int cus = device_cu_count();
    if constexpr (!GU) {
        if (edge) {
            g.full_units = g.units = total;
            g.first_unit = 0;
            return launch(gemm_tn_kernel<FA, FB, true, SET, false, false, NT>, dim3(total < cus ? total : cus), dim3(256),
                          stream, g);
        }
    }
    // Balance the last round: when the tiles past the last full round of the
    // persistent grid fill at most half of it, each becomes two half tiles (a
    // second launch of their own), so that round takes about half as long.
    // K-major operands only.
    const int tail = total % cus;
    const bool split = SET == kSetKK && tail > 0 && 2 * tail <= cus;
    g.full_units = split ? total - tail : total;
    g.units = g.full_units;
    g.first_unit = 0;
    if (g.full_units > 0) {
        const hipError_t e = launch(gemm_tn_kernel<FA, FB, false, SET, false, GU, NT>,
                                    dim3(g.full_units < cus ? g.full_units : cus), dim3(256), stream, g);
        if (e != hipSuccess) return e;
    }
    if constexpr (SET == kSetKK) {
        if (split) {
            g.first_unit = g.full_units;
            g.units = total + tail;
            return launch(gemm_tn_kernel<FA, FB, false, SET, true, GU, NT>, dim3(2 * tail), dim3(256), stream, g);
        }
    }
    return hipSuccess;
}

// B is always E4M3 (weights or activations); A is E4M3 or E5M2.  Layout sets:
// every problem (K, K), or every problem (K, MN) / (MN, MN).  nt: the outputs are
// the backward products' (stored non-temporally); A in E5M2 (a gradient) and
// the MN-major set only occur there.
static hipError_t dispatch(int fmt_a, int fmt_b, const GemmGroup& g, bool nt, hipStream_t stream)
{
    for (int i = 0; i < g.count; ++i) {
        const GemmProblem& p = g.p[i];
        const bool kk = p.la == kKMajor && p.lb == kKMajor;
        const bool mn = p.lb == kMNMajor;
        if (!(kk || mn) || (g.p[0].lb != p.lb)) return hipErrorInvalidValue;
    }
    if (fmt_b != 0) return hipErrorInvalidValue;
    if (!nt && (fmt_a != 0 || g.p[0].lb != kKMajor)) return hipErrorInvalidValue;
    if (g.p[0].lb == kKMajor) {
        if (fmt_a == 0) {
            if (nt) return launch_group<0, 0, kSetKK, false, true>(g, stream);
            return launch_group<0, 0, kSetKK, false, false>(g, stream);
        }
        return launch_group<1, 0, kSetKK, false, true>(g, stream);
    }
    if (fmt_a == 0) return launch_group<0, 0, kSetMN, false, true>(g, stream);
    return launch_group<1, 0, kSetMN, false, true>(g, stream);
}

hipError_t launch_gemm_gate_up(const uint8_t* A, const uint8_t* B, const float* inv_a, const float* inv_b, void* out,
                               float* absmax_h, int64_t M, int64_t F, int64_t K, hipStream_t stream)
{
    GemmGroup g{};
    hipError_t e = silu_table(&g.table, stream);
    if (e != hipSuccess) return e;
    g.absmax_h = reinterpret_cast<uint32_t*>(absmax_h);
    g.p[0] = make_problem(A, kKMajor, B, kKMajor, inv_a, inv_b, out, M, 2 * F, K);
    g.p[0].tiles_n = (int)(F / (kBN / 2));        // a tile: 128 gate and the matching 128 up columns
    g.p[1] = g.p[0];
    g.count = 1;
    return launch_group<0, 0, kSetKK, true, false>(g, stream);
}

// Block-scaled launches: full tiles, then (when the tiles past the last full
// round fill at most half of the grid) those tiles as half tiles in a second
// launch, as launch_group does.
template <int FA, bool NT>
static hipError_t launch_mx_group(GemmGroup g, hipStream_t stream)
{
    int total = 0;
    for (int i = 0; i < g.count; ++i) {
        if (g.p[i].P < kBM || g.p[i].Q < kBN) return hipErrorInvalidValue;
        g.p[i].first_tile = total;
        total += g.p[i].tiles_m * g.p[i].tiles_n;
    }
    g.total_tiles = total;
    const int cus = device_cu_count();
    const int tail = total % cus;
    const bool split = tail > 0 && 2 * tail <= cus;
    g.full_units = split ? total - tail : total;
    g.units = g.full_units;
    g.first_unit = 0;
    if (g.full_units > 0) {
        const hipError_t e = launch(gemm_mx_kernel<FA, 0, false, NT>, dim3(g.full_units < cus ? g.full_units : cus),
                                    dim3(256), stream, g);
        if (e != hipSuccess) return e;
    }
    if (split) {
        g.first_unit = g.full_units;
        g.units = total + tail;
        return launch(gemm_mx_kernel<FA, 0, true, NT>, dim3(2 * tail), dim3(256), stream, g);
    }
    return hipSuccess;
}

static GemmProblem make_problem_mx(const uint8_t* A, const uint8_t* sa, const uint8_t* B, const uint8_t* sb,
                                   void* out, int64_t P, int64_t Q, int64_t R)
{
    GemmProblem p = make_problem(A, kKMajor, B, kKMajor, nullptr, nullptr, out, P, Q, R);
    p.sa = sa;
    p.sb = sb;
    return p;
}

hipError_t launch_gemm_mx(const uint8_t* A, const uint8_t* sa, int fmt_a, const uint8_t* B, const uint8_t* sb,
                          int fmt_b, void* out, int64_t P, int64_t Q, int64_t R, hipStream_t stream)
{
    if (fmt_b != 0) return hipErrorInvalidValue;
    GemmGroup g{};
    g.p[0] = make_problem_mx(A, sa, B, sb, out, P, Q, R);
    g.p[1] = g.p[0];
    g.count = 1;
    if (fmt_a == 0) return launch_mx_group<0, false>(g, stream);
    return launch_mx_group<1, false>(g, stream);
}

hipError_t launch_gemm_mx_pair(const uint8_t* A0, const uint8_t* sa0, const uint8_t* B0, const uint8_t* sb0,
                               void* out0, int64_t P0, int64_t Q0, int64_t R0, const uint8_t* A1,
                               const uint8_t* sa1, const uint8_t* B1, const uint8_t* sb1, void* out1, int64_t P1,
                               int64_t Q1, int64_t R1, int fmt_a, hipStream_t stream)
{
    GemmGroup g{};
    GemmProblem p0 = make_problem_mx(A0, sa0, B0, sb0, out0, P0, Q0, R0);
    GemmProblem p1 = make_problem_mx(A1, sa1, B1, sb1, out1, P1, Q1, R1);
    // as launch_gemm_tn_pair: longest reduction first, groups of 4 tile rows for
    // outputs wider than 32 column tiles
    g.p[0] = R1 > R0 ? p1 : p0;
    g.p[1] = R1 > R0 ? p0 : p1;
    for (int i = 0; i < 2; ++i)
        if (g.p[i].group_m == kGroupM && g.p[i].tiles_n > 32) g.p[i].group_m = 4;
    g.count = 2;
    if (fmt_a == 0) return launch_mx_group<0, true>(g, stream);   // dX and dW: stored non-temporally
    return launch_mx_group<1, true>(g, stream);
}

hipError_t launch_gemm_tn(const uint8_t* A, int fmt_a, int la, const uint8_t* B, int fmt_b, int lb,
                          const float* inv_a, const float* inv_b, void* out, int64_t P, int64_t Q, int64_t R,
                          bool nt_out, hipStream_t stream)
{
    GemmGroup g{};
    g.p[0] = make_problem(A, la, B, lb, inv_a, inv_b, out, P, Q, R);
    g.p[1] = g.p[0];
    g.count = 1;
    return dispatch(fmt_a, fmt_b, g, nt_out, stream);
}

hipError_t launch_gemm_tn_pair(const uint8_t* A0, int la0, const uint8_t* B0, int lb0, const float* ia0,
                               const float* ib0, void* out0, int64_t P0, int64_t Q0, int64_t R0, const uint8_t* A1,
                               int la1, const uint8_t* B1, int lb1, const float* ia1, const float* ib1, void* out1,
                               int64_t P1, int64_t Q1, int64_t R1, int fmt_a, int fmt_b, hipStream_t stream)
{
    GemmGroup g{};
    GemmProblem p0 = make_problem(A0, la0, B0, lb0, ia0, ib0, out0, P0, Q0, R0);
    GemmProblem p1 = make_problem(A1, la1, B1, lb1, ia1, ib1, out1, P1, Q1, R1);
    // longest reduction first: the first round then starts the longest tiles
    g.p[0] = R1 > R0 ? p1 : p0;
    g.p[1] = R1 > R0 ? p0 : p1;
    // outputs wider than 32 column tiles walk groups of 4 tile rows: measured on
    // MI355X, the down-projection pairs of 7B-, 14B- and 32B-class layers (43, 54
    // and 108 column tiles) ran 4.6%, 2.4% and 0.7% faster than with 8, and no
    // other pair of those layers (16-28 column tiles) changed; forward launches
    // keep 8 (the 86-column gate/up forward ran 3% slower with 4)
    for (int i = 0; i < 2; ++i)
        if (g.p[i].group_m == kGroupM && g.p[i].tiles_n > 32) g.p[i].group_m = 4;
    g.count = 2;
    return dispatch(fmt_a, fmt_b, g, true, stream);      // dX and dW: stored non-temporally
}

}  // namespace fp8k
