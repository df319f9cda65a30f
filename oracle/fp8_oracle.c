/*
 * fp8_oracle.c -- the CPU oracle for the FP8 training hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark use it, to check and to time the GPU library.  It shares
 * no code, header, table or constant generator with the GPU library.
 *
 * What it computes (plain definitions, written for a reader to check by eye):
 *
 *   Sources.  "LLMQ: Efficient Lower-Precision Pretraining for Consumer GPUs"
 *   (paperlayer.ai summary of arXiv 2512.15306): section 1 (FP8 training with
 *   dynamic tensor-level scaling), section 3.1 (the forward's absmax statistic
 *   is kept, so the recomputed SwiGLU output is requantised in the same pass
 *   that evaluates it and is not reduced again), section 4 (dynamic quantisation and
 *   backward-pass transposes are overhead; extra transpose and quantisation
 *   buffers), section 5 / Figure 2 (E4M3 forward and backward versus E5M2
 *   activation gradients).  "FastML periodic report" (EU CORDIS), the item on
 *   FP8 training without delayed scaling: the scale comes just in time from the
 *   tensor's current absmax, so no value is clipped.
 *
 *   The pages give no bit layouts, formula, rounding mode or accumulation
 *   precision.  This file takes the readings below (each is listed with its
 *   reason in the design notes):
 *     - formats: OCP 8-bit floating point (OFP8) E4M3 ("fn": bias 7, no
 *       infinity, NaN = S.1111.111, max 448) and E5M2 (bias 15, IEEE-like,
 *       infinity S.11111.00, max 57344);
 *     - absmax = max |x| over the whole tensor (an exact maximum);
 *     - scale s = fp8_max / absmax as one IEEE fp32 division, s = 1 when
 *       absmax = 0, s clamped to FLT_MAX when the division overflows;
 *       inverse scale = 1 / s in fp32;
 *     - q = encode(RN32(x * s)): the product rounded to fp32 first, then
 *       rounded to the 8-bit format, nearest-even, saturating at +-max;
 *     - SwiGLU: h = silu(g) * u with silu(g) = g / (1 + e^-g), gate and up
 *       concatenated as [gate | up] along the feature axis, every step one
 *       fp32 operation in the order E = RN32(e^-g), t = 1 + E, s_g = g / t,
 *       h = s_g * u, and e^-g correctly rounded to fp32;
 *     - SwiGLU backward (the gradients of gate and up, quantised for the
 *       gate/up backward GEMMs): with sigma = 1 / (1 + e^-g) and
 *       silu'(g) = sigma * (1 + g * (1 - sigma)) (the textbook derivative of
 *       g * sigma), du = dh * silu(g) and dg = (dh * u) * silu'(g), every step
 *       one fp32 operation in the order written below, then the per-tensor
 *       absmax / scale / encode of [dg | du] like any other tensor;
 *     - GEMM: fp32 sum over ascending k of the decoded products (every
 *       FP8 x FP8 product is exact in fp32), then one multiply by
 *       RN32(da * db), then round-to-nearest-even to bf16.
 *     - Block (MX) scaling, the alternative to per-tensor scaling that the
 *       LLMQ summary (section 2) says needs native hardware support: the pages
 *       define no format, so this file follows the OCP Microscaling (MX)
 *       formats specification v1.0 (section 6.3, the scale and conversion of a
 *       block): blocks of 32 consecutive elements of a row; one shared scale
 *       2^e per block stored as an E8M0 byte e + 127 (255 = NaN), with
 *       e = floor(log2(max |x|)) - emax, emax = 8 for E4M3 and 15 for E5M2
 *       (the exponent of the format's largest normal), clamped to
 *       [-127, 127] (e = -127 for an all-zero block); the elements are
 *       x / 2^e (exact) encoded like every other value (nearest-even,
 *       saturating).  A block holding a NaN or an infinity gets the NaN
 *       scale and the unscaled encodings.  The MX GEMM is the GEMM above with
 *       each product dec(a) dec(b) multiplied by 2^(ea + eb) (its two blocks'
 *       scales) before the fp32 sum, and no per-tensor factor.
 *
 * Built with gcc -O2 -ffp-contract=off (no fast-math), so every float
 * operation below is exactly one IEEE binary32 operation (x86-64 SSE).
 */
#include <float.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <string.h>

#define FMT_E4M3 0
#define FMT_E5M2 1

static float f32_from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

/* bf16 -> fp32: the bf16 bits are the top half of the fp32 bits (exact). */
float oracle_bf16_to_f32(uint16_t b) { return f32_from_bits((uint32_t)b << 16); }

/* fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t b = bits_from_f32(f);
    if (isnan(f)) return (uint16_t)((b >> 16) | 0x0040u);
    uint32_t lower = b & 0xFFFFu;
    uint32_t upper = b >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
    return (uint16_t)upper;
}

/* Parameters of the two OFP8 formats. */
struct fmt_desc { int mbits; int bias; float maxv; uint8_t maxcode; };
static struct fmt_desc fmt_of(int fmt)
{
    struct fmt_desc d;
    if (fmt == FMT_E4M3) { d.mbits = 3; d.bias = 7;  d.maxv = 448.0f;   d.maxcode = 0x7E; }
    else                 { d.mbits = 2; d.bias = 15; d.maxv = 57344.0f; d.maxcode = 0x7B; }
    return d;
}

/*
 * Encode one fp32 value to an OFP8 byte: round to nearest, ties to even,
 * saturating.  NaN -> S.1111111 (0x7F | sign).  |v| > max (infinity included)
 * -> +-max.  Underflow keeps the sign (-tiny -> 0x80).
 */
uint8_t oracle_encode(float v, int fmt)
{
    struct fmt_desc d = fmt_of(fmt);
    uint8_t sign = (uint8_t)((bits_from_f32(v) >> 24) & 0x80u);
    if (isnan(v)) return (uint8_t)(sign | 0x7F);
    float a = fabsf(v);
    if (a > d.maxv) return (uint8_t)(sign | d.maxcode);

    int emin = 1 - d.bias;                      /* exponent of the smallest normal */
    float min_normal = ldexpf(1.0f, emin);
    if (a < min_normal) {
        /* Subnormal range: a multiple of the quantum 2^(emin - mbits). */
        float steps = ldexpf(a, d.mbits - emin);   /* exact: a power-of-two scaling up */
        float m = nearbyintf(steps);               /* default rounding mode: ties to even */
        /* m == 2^mbits lands exactly on the smallest normal code (exponent field 1). */
        return (uint8_t)(sign | (uint8_t)m);
    }
    int e;
    float r = frexpf(a, &e);                    /* a = r * 2^e, r in [0.5, 1) */
    r *= 2.0f; e -= 1;                          /* a = r * 2^e, r in [1, 2) (exact) */
    float m = nearbyintf(ldexpf(r - 1.0f, d.mbits));   /* r - 1 and the scaling are exact */
    if (m == ldexpf(1.0f, d.mbits)) { m = 0.0f; e += 1; }
    return (uint8_t)(sign | (uint8_t)((e + d.bias) << d.mbits) | (uint8_t)m);
}

/* Decode one OFP8 byte to fp32 (exact: every OFP8 value is an fp32 value). */
float oracle_decode(uint8_t c, int fmt)
{
    struct fmt_desc d = fmt_of(fmt);
    int sign = c & 0x80;
    int ebits = 7 - d.mbits;
    int efield = (c >> d.mbits) & ((1 << ebits) - 1);
    int mfield = c & ((1 << d.mbits) - 1);
    float mag;
    if (fmt == FMT_E4M3 && (c & 0x7F) == 0x7F) return sign ? -NAN : NAN;
    if (fmt == FMT_E5M2 && efield == 31) {
        if (mfield != 0) return sign ? -NAN : NAN;
        return sign ? -INFINITY : INFINITY;
    }
    if (efield == 0) mag = ldexpf((float)mfield, 1 - d.bias - d.mbits);
    else mag = ldexpf(1.0f + ldexpf((float)mfield, -d.mbits), efield - d.bias);
    return sign ? -mag : mag;
}

/*
 * absmax of a bf16 tensor: the largest magnitude bit pattern.  For finite data
 * this is max |x_i|; a NaN or infinity anywhere sorts above every finite value,
 * so it surfaces in the result.
 */
float oracle_absmax_bf16(const uint16_t* x, int64_t n)
{
    uint32_t best = 0;
    #pragma omp parallel for reduction(max:best) schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint32_t m = x[i] & 0x7FFFu;
        if (m > best) best = m;
    }
    return f32_from_bits(best << 16);
}

/* absmax of an fp32 tensor, same rule on the 31 magnitude bits. */
float oracle_absmax_f32(const float* x, int64_t n)
{
    uint32_t best = 0;
    #pragma omp parallel for reduction(max:best) schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint32_t m = bits_from_f32(x[i]) & 0x7FFFFFFFu;
        if (m > best) best = m;
    }
    return f32_from_bits(best);
}

/* scale = fp8_max / absmax (fp32), inverse = 1 / scale (fp32). */
void oracle_scale(float absmax, int fmt, float* scale, float* inv_scale)
{
    float s;
    if (absmax == 0.0f) s = 1.0f;
    else {
        s = fmt_of(fmt).maxv / absmax;
        if (isinf(s) && s > 0.0f) s = FLT_MAX;
    }
    *scale = s;
    *inv_scale = 1.0f / s;
}

/*
 * Quantise a row-major bf16 [rows, cols] tensor with scale s.
 * q[i*cols + j] = encode(RN32(x[i,j] * s)); qt[j*rows + i] is the same byte
 * (the transposed copy the backward GEMMs read).  Either output may be NULL.
 */
void oracle_quantize(const uint16_t* x, int64_t rows, int64_t cols, int fmt, float s,
                     uint8_t* q, uint8_t* qt)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        for (int64_t j = 0; j < cols; ++j) {
            float p = oracle_bf16_to_f32(x[i * cols + j]) * s;
            uint8_t c = oracle_encode(p, fmt);
            if (q) q[i * cols + j] = c;
            if (qt) qt[j * rows + i] = c;
        }
    }
}

/* RN32(e^-g): the exact exponential rounded once to fp32 (through libm's double exp). */
float oracle_exp_neg(float g)
{
    return (float)exp(-(double)g);
}

/* h = silu(g) * u, one fp32 operation at a time. */
float oracle_swiglu_one(float g, float u)
{
    float E = oracle_exp_neg(g);
    float t = 1.0f + E;
    float sg = g / t;
    return sg * u;
}

/* The SwiGLU output h[M, F] (fp32) of gu = [gate | up], a bf16 [M, 2F] tensor. */
void oracle_swiglu_h(const uint16_t* gu, int64_t M, int64_t F, float* h)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < F; ++j) {
            float g = oracle_bf16_to_f32(gu[i * 2 * F + j]);
            float u = oracle_bf16_to_f32(gu[i * 2 * F + F + j]);
            h[i * F + j] = oracle_swiglu_one(g, u);
        }
}

/*
 * SwiGLU requantisation.  compute_absmax = 1 (forward): absmax_h is the
 * absmax of every h and is written out.  compute_absmax = 0 (recomputation):
 * *absmax_h is the retained statistic and is only read, no reduction runs.
 * Then hq = encode_e4m3(RN32(h * s_h)); hqt (may be NULL) is its transpose.
 * h_buf is caller scratch of M*F floats.
 */
void oracle_swiglu_requant(const uint16_t* gu, int64_t M, int64_t F, int compute_absmax,
                           float* absmax_h, float* inv_scale_h, float* h_buf,
                           uint8_t* hq, uint8_t* hqt)
{
    float s, inv;
    oracle_swiglu_h(gu, M, F, h_buf);
    if (compute_absmax) *absmax_h = oracle_absmax_f32(h_buf, M * F);
    oracle_scale(*absmax_h, FMT_E4M3, &s, &inv);
    if (inv_scale_h) *inv_scale_h = inv;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < F; ++j) {
            uint8_t c = oracle_encode(h_buf[i * F + j] * s, FMT_E4M3);
            if (hq) hq[i * F + j] = c;
            if (hqt) hqt[j * M + i] = c;
        }
}

/*
 * SwiGLU backward, one element pair.  g, u: the gate and up values; d: the
 * gradient of h = silu(g) * u.  Every step is one fp32 operation:
 *   E = RN32(e^-g), t = 1 + E, sig = 1 / t, s = g / t            (s = silu(g))
 *   c = 1 - sig, p = g * c, q = 1 + p, ds = sig * q               (ds = silu'(g))
 *   du = d * s
 *   dg = (d * u) * ds
 */
void oracle_swiglu_grad_one(float g, float u, float d, float* dg, float* du)
{
    float E = oracle_exp_neg(g);
    float t = 1.0f + E;
    float sig = 1.0f / t;
    float s = g / t;
    float c = 1.0f - sig;
    float p = g * c;
    float q = 1.0f + p;
    float ds = sig * q;
    *du = d * s;
    float du_ = d * u;
    *dg = du_ * ds;
}

/*
 * The gradient of gu = [gate | up] (fp32, [M, 2F]) from gu (bf16 [M, 2F]) and
 * dh (bf16 [M, F]): dgu[i, j] = dg, dgu[i, F + j] = du.
 */
void oracle_swiglu_grad(const uint16_t* gu, const uint16_t* dh, int64_t M, int64_t F, float* dgu)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < F; ++j) {
            float g = oracle_bf16_to_f32(gu[i * 2 * F + j]);
            float u = oracle_bf16_to_f32(gu[i * 2 * F + F + j]);
            float d = oracle_bf16_to_f32(dh[i * F + j]);
            oracle_swiglu_grad_one(g, u, d, &dgu[i * 2 * F + j], &dgu[i * 2 * F + F + j]);
        }
}

/*
 * SwiGLU backward fused with the quantisation of its output: dgu as above
 * (caller scratch of M*2F floats), absmax = max |dgu| (fresh: gradients have no
 * retained statistic), scale for fmt, q = encode(RN32(dgu * s)) [M, 2F] and its
 * transpose qt [2F, M] (either may be NULL).
 */
void oracle_swiglu_backward(const uint16_t* gu, const uint16_t* dh, int64_t M, int64_t F, int fmt,
                            float* absmax, float* scale, float* inv_scale, float* dgu,
                            uint8_t* q, uint8_t* qt)
{
    float s, inv;
    oracle_swiglu_grad(gu, dh, M, F, dgu);
    *absmax = oracle_absmax_f32(dgu, M * 2 * F);
    oracle_scale(*absmax, fmt, &s, &inv);
    if (scale) *scale = s;
    if (inv_scale) *inv_scale = inv;
    const int64_t C = 2 * F;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < C; ++j) {
            uint8_t c = oracle_encode(dgu[i * C + j] * s, fmt);
            if (q) q[i * C + j] = c;
            if (qt) qt[j * M + i] = c;
        }
}

/*
 * FP8 GEMM with both operands K-contiguous:
 *   C[m, n] = sum over k = 0..K-1 (ascending) of dec(A[m, k]) * dec(B[n, k])   (fp32)
 *   Y[m, n] = bf16_RNE(RN32(C[m, n] * RN32(da * db)))
 * A is [M, K] in format fmt_a, B is [N, K] in format fmt_b.  When rows is not
 * NULL only the nrows listed rows m = rows[r] are computed, into Y[r, :].
 * a_dec / b_dec are caller scratch of nrows*K and N*K floats.
 */
void oracle_gemm(const uint8_t* A, int fmt_a, const uint8_t* B, int fmt_b,
                 int64_t M, int64_t N, int64_t K, float da, float db,
                 const int64_t* rows, int64_t nrows, float* a_dec, float* b_dec,
                 uint16_t* Y)
{
    float descale = da * db;
    if (!rows) nrows = M;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) b_dec[n * K + k] = oracle_decode(B[n * K + k], fmt_b);
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t m = rows ? rows[r] : r;
        for (int64_t k = 0; k < K; ++k) a_dec[r * K + k] = oracle_decode(A[m * K + k], fmt_a);
    }
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const float* a = a_dec + r * K;
        for (int64_t n = 0; n < N; ++n) {
            const float* b = b_dec + n * K;
            float acc = 0.0f;
            for (int64_t k = 0; k < K; ++k) acc += a[k] * b[k];
            Y[r * N + n] = oracle_f32_to_bf16(acc * descale);
        }
    }
}

/* ---- block (MX) scaling: see the header for the reading of the OCP MX specification. */
#define MX_BLOCK 32

/*
 * One block of MX_BLOCK fp32 values: its scale byte and codes (the reading in
 * the header).  The maximum is taken over the finite magnitudes; a NaN or an
 * infinity makes the block's scale NaN (255) and its codes the unscaled encodings.
 */
static void mx_block(const float* v, int fmt, uint8_t* q, uint8_t* scale)
{
    const int emax = fmt == FMT_E4M3 ? 8 : 15;
    float m = 0.0f;
    int nonfinite = 0;
    for (int k = 0; k < MX_BLOCK; ++k) {
        if (!isfinite(v[k])) nonfinite = 1;
        else if (fabsf(v[k]) > m) m = fabsf(v[k]);
    }
    if (nonfinite) {
        *scale = 255;
        for (int k = 0; k < MX_BLOCK; ++k) q[k] = oracle_encode(v[k], fmt);
        return;
    }
    int e = -127;
    if (m > 0.0f) {
        int k2;
        frexpf(m, &k2);                         /* m = r * 2^k2, r in [0.5, 1): floor(log2 m) = k2 - 1 */
        e = (k2 - 1) - emax;
        if (e < -127) e = -127;
        if (e > 127) e = 127;
    }
    *scale = (uint8_t)(e + 127);
    for (int k = 0; k < MX_BLOCK; ++k) q[k] = oracle_encode(ldexpf(v[k], -e), fmt);
}

/*
 * MX quantisation of a row-major bf16 [rows, cols] tensor (cols a multiple of
 * 32): q[i, j] = encode(x[i, j] / 2^e), scales[i, j / 32] = e + 127 for the
 * block's e (255 for a block with a NaN or an infinity, whose codes are the
 * unscaled encodings).
 */
void oracle_mx_quantize(const uint16_t* x, int64_t rows, int64_t cols, int fmt, uint8_t* q, uint8_t* scales)
{
    const int64_t nb = cols / MX_BLOCK;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        float v[MX_BLOCK];
        for (int64_t b = 0; b < nb; ++b) {
            for (int k = 0; k < MX_BLOCK; ++k) v[k] = oracle_bf16_to_f32(x[i * cols + b * MX_BLOCK + k]);
            mx_block(v, fmt, q + i * cols + b * MX_BLOCK, scales + i * nb + b);
        }
    }
}

/*
 * MX quantisation of an fp32 [rows, cols] tensor (the same blocks and rule).
 */
void oracle_mx_quantize_f32(const float* x, int64_t rows, int64_t cols, int fmt, uint8_t* q, uint8_t* scales)
{
    const int64_t nb = cols / MX_BLOCK;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t b = 0; b < nb; ++b)
            mx_block(x + i * cols + b * MX_BLOCK, fmt, q + i * cols + b * MX_BLOCK, scales + i * nb + b);
}

/*
 * The SwiGLU output h [M, F] of gu = [gate | up] (oracle_swiglu_one, one fp32
 * value per element, never rounded to bf16), quantised in MX blocks along F
 * (E4M3: h is an activation).  F a multiple of 32.
 */
void oracle_mx_swiglu(const uint16_t* gu, int64_t M, int64_t F, uint8_t* hq, uint8_t* scales)
{
    const int64_t nb = F / MX_BLOCK;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        float v[MX_BLOCK];
        for (int64_t b = 0; b < nb; ++b) {
            for (int k = 0; k < MX_BLOCK; ++k) {
                const int64_t j = b * MX_BLOCK + k;
                v[k] = oracle_swiglu_one(oracle_bf16_to_f32(gu[i * 2 * F + j]), oracle_bf16_to_f32(gu[i * 2 * F + F + j]));
            }
            mx_block(v, FMT_E4M3, hq + i * F + b * MX_BLOCK, scales + i * nb + b);
        }
    }
}

/*
 * MX GEMM: Y[m, n] = bf16(RN32(sum over ascending k of
 * ldexp(dec(A[m, k]) dec(B[n, k]), ea + eb))) with ea, eb the scales of the
 * blocks holding A[m, k] and B[n, k] (a NaN scale makes the product NaN).
 * A [M, K], B [N, K], scales [M, K / 32] and [N, K / 32]; rows as in oracle_gemm.
 */
void oracle_mx_gemm(const uint8_t* A, const uint8_t* SA, int fmt_a, const uint8_t* B, const uint8_t* SB,
                    int fmt_b, int64_t M, int64_t N, int64_t K, const int64_t* rows, int64_t nrows, uint16_t* Y)
{
    const int64_t nb = K / MX_BLOCK;
    if (!rows) nrows = M;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t m = rows ? rows[r] : r;
        for (int64_t n = 0; n < N; ++n) {
            float acc = 0.0f;
            for (int64_t k = 0; k < K; ++k) {
                uint8_t sa = SA[m * nb + k / MX_BLOCK], sb = SB[n * nb + k / MX_BLOCK];
                float p = oracle_decode(A[m * K + k], fmt_a) * oracle_decode(B[n * K + k], fmt_b);
                if (sa == 255 || sb == 255) p = NAN;
                else p = ldexpf(p, (int)sa + (int)sb - 254);
                acc += p;
            }
            Y[r * N + n] = oracle_f32_to_bf16(acc);
        }
    }
}

/* Element-wise helpers for vectors, so the Python side needs no loops. */
void oracle_encode_vec(const float* v, int64_t n, int fmt, uint8_t* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_encode(v[i], fmt);
}

void oracle_decode_vec(const uint8_t* c, int64_t n, int fmt, float* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_decode(c[i], fmt);
}

void oracle_exp_neg_vec(const float* g, int64_t n, float* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_exp_neg(g[i]);
}

int oracle_num_threads(void)
{
    int t = 1;
    #pragma omp parallel
    {
        #pragma omp single
        {
#ifdef _OPENMP
            t = omp_get_num_threads();
#endif
        }
    }
    return t;
}
