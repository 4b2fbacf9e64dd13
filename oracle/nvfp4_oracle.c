/*
 * nvfp4_oracle.c -- plain CPU oracle for the NVFP4 training quantizer.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the benchmark's CPU-baseline leg load this
 * library; the product (the HIP library under nvfp4_quantization_amd/) never includes, links or calls it, and
 * the two share no source, header, table or constant generator.
 *
 * Pages cited (title, then the section used):
 *   [P1] "在 RTX 5090 (SM120) 上补全 NVFP4 量化相关 kernel" (blog post on polyfilling NVFP4 quantization
 *        kernels for the RTX 5090, harrychen.xyz, 2026-04-14).
 *   [P2] "nvfp4-sm120" repository README.
 *   [P3] pytorch/ao pull request #4852, "Add a CuTe DSL fast-path kernel for four-over-six quantize".
 *   Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11.
 *
 * Arithmetic rules: every floating-point value in the method is IEEE-754 binary32 and every operation below is
 * one correctly rounded binary32 operation (round to nearest even).  Build with -O2 -ffp-contract=off and never
 * with -ffast-math; subnormals are kept.  Where a helper uses binary64 it is only to compare distances that are
 * exact in binary64 (stated at each use).
 *
 * The code is deliberately slow and literal: brute-force nearest-value searches instead of bit tricks, one
 * block at a time, in the order the method states.  Readings of the pages where they leave a step open are
 * marked READING.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>
#include <float.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------------------------------------------
 * Status codes (same numeric meaning as the product library's, so the tests can compare them).
 * ---------------------------------------------------------------------------------------------------------- */
#define NVO_OK 0
#define NVO_ERR_NULL 1
#define NVO_ERR_SHAPE 2
#define NVO_ERR_UNSUPPORTED 4

#define NVO_ROWWISE 1
#define NVO_COLWISE 2

#define NVO_G_PER_TENSOR 0
#define NVO_G_PER_ROW 1

#define NVO_MODE_RN 0
#define NVO_MODE_SR 1
#define NVO_MODE_RHT_SR 2

static float f32_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int nvo_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void nvo_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* bf16 -> fp32: a bf16 value is the upper half of a binary32 pattern, so the widening is exact. */
float nvo_bf16_to_f32(uint16_t h) { return f32_of((uint32_t)h << 16); }

/* ------------------------------------------------------------------------------------------------------------
 * E2M1 element format.  [P1, section on FP4 quantization techniques]: the representable magnitudes are
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6.  READING: the 4-bit code is sign<<3 | m where m indexes that list in increasing
 * order (the standard 1-sign / 2-exponent / 1-mantissa layout is the only one that orders the list this way).
 * ---------------------------------------------------------------------------------------------------------- */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

float nvo_e2m1_decode(uint8_t code) {
    double m = E2M1_MAG[code & 7];
    return (float)((code & 8) ? -m : m);
}

/* Round to nearest, ties to the even code.  [P1, section on stochastic rounding]: hardware conversion uses
 * IEEE round-to-nearest.  The "satfinite" conversions the page names clamp anything beyond the largest finite
 * magnitude (including infinity) to +-6.  READING (NaN): a NaN input gives code 0x7.
 * Distances |t - G[k]| are exact in binary64 because t < 6 here and both are binary32 values. */
uint8_t nvo_e2m1_rn(float q) {
    if (isnan(q)) return 0x7;
    uint8_t sign = signbit(q) ? 8 : 0;
    double t = fabs((double)q);
    if (t >= 6.0) return (uint8_t)(sign | 7);           /* satfinite, includes +-inf */
    int best = 0;
    double best_d = t;                                   /* distance to G[0] = 0 */
    for (int k = 1; k < 8; ++k) {
        double d = fabs(t - E2M1_MAG[k]);
        /* candidates are scanned in increasing order, so a tie is always between k-1 and k; keep the even one */
        if (d < best_d || (d == best_d && (k % 2) == 0)) { best = k; best_d = d; }
    }
    return (uint8_t)(sign | best);
}

/* Stochastic rounding.  [P1, section on stochastic rounding]: a value between neighbours a < b of the grid goes
 * to b with probability (x - a) / (b - a).  READING: the random source is one uniform byte rho per element
 * ([P1]: the hardware instruction takes one 32-bit random word per four values, i.e. 8 bits per value), and
 * the element rounds up iff rho < floor(256 * (x - a) / (b - a)).  Magnitudes at or above 6 (and inf) saturate
 * to 6.  NaN gives 0x7.  All the arithmetic here is exact in binary64 (t < 6, a and b-a are dyadic). */
uint8_t nvo_e2m1_sr(float q, uint8_t rho) {
    if (isnan(q)) return 0x7;
    uint8_t sign = signbit(q) ? 8 : 0;
    double t = fabs((double)q);
    if (t >= 6.0) return (uint8_t)(sign | 7);
    int lo = 0;
    for (int k = 0; k < 8; ++k)
        if (E2M1_MAG[k] <= t) lo = k;                    /* largest grid magnitude not above t */
    double a = E2M1_MAG[lo], b = E2M1_MAG[lo + 1];
    double frac = (t - a) / (b - a);                     /* in [0, 1) */
    unsigned f8 = (unsigned)floor(256.0 * frac);         /* in [0, 255] */
    int m = lo + ((unsigned)rho < f8 ? 1 : 0);
    return (uint8_t)(sign | m);
}

/* Array forms of the two E2M1 conversions (element-wise loops over the scalar definitions above). */
void nvo_e2m1_rn_array(const float* q, int64_t n, uint8_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = nvo_e2m1_rn(q[i]);
}

void nvo_e2m1_sr_array(const float* q, const uint8_t* rho, int64_t n, uint8_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = nvo_e2m1_sr(q[i], rho[i]);
}

/* ------------------------------------------------------------------------------------------------------------
 * E4M3 block-scale format ("fn" variant: 4 exponent bits with bias 7, 3 mantissa bits, no infinity, the single
 * NaN pattern S.1111.111, largest finite 448).  The scale is stored as an unsigned E4M3 code; the sign bit is
 * always 0.  [P2, section describing the layout]: two-level quantization with an E4M3 block scale;
 * [P3]: the E4M3 cast and its exact decode are pinned rounding steps.
 * ---------------------------------------------------------------------------------------------------------- */
float nvo_e4m3_decode(uint8_t b) {
    int s = (b >> 7) & 1, e = (b >> 3) & 0xF, m = b & 7;
    if (e == 0xF && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9)           /* subnormal: m * 2^-9 */
                        : ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
    return (float)(s ? -v : v);
}

/* Nearest of the 127 finite non-negative E4M3 values (codes 0x00..0x7E), ties to the even code; above 448
 * (including +inf) saturates to 0x7E ("satfinite", the convention of the conversions named in [P1]); NaN gives
 * 0x7F; a negative input's nearest non-negative value is 0.  |s - v| is exact in binary64 whenever it can
 * decide the result (s >= 2^-39, or else code 0 is the clear winner). */
uint8_t nvo_e4m3_encode(float s) {
    if (isnan(s)) return 0x7F;
    if (s > 448.0f) return 0x7E;
    if (!(s > 0.0f)) return 0x00;                        /* zero, and every negative value down to -inf */
    int best = 0;
    double best_d = fabs((double)s);
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs((double)s - (double)nvo_e4m3_decode((uint8_t)c));
        if (d < best_d || (d == best_d && (c % 2) == 0)) { best = c; best_d = d; }
    }
    return (uint8_t)best;
}

void nvo_e4m3_encode_array(const float* s, int64_t n, uint8_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = nvo_e4m3_encode(s[i]);
}

/* ------------------------------------------------------------------------------------------------------------
 * Philox4x32-10 (Salmon et al., SC'11): 10 rounds of the 4x32 Philox S-box with multipliers 0xD2511F53 and
 * 0xCD9E8D57 and the Weyl key increments 0x9E3779B9 / 0xBB67AE85 (the golden ratio and sqrt(3)-1 in 32-bit
 * fixed point).  Round: with the counter (c0, c1, c2, c3) and key (k0, k1),
 *   (c0, c1, c2, c3) <- (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)),
 * then the key is bumped; the key bump happens between rounds, not after the last.
 * [P1, sections on the vibe-coding process and the timeline]: the random bits come from Philox and the counter
 * layout is part of the semantics.
 * ---------------------------------------------------------------------------------------------------------- */
void nvo_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* READING (counter layout): the 16 random bytes of one call serve one 1x16 block.  Key = (seed low word,
 * seed high word); counter = (block index low, block index high, offset low, offset high), where the block index
 * is the block's position in the row-major order of the quantized view; element j of the block takes byte
 * (j % 4) of word (j / 4), least significant byte first. */
void nvo_block_random_bytes(uint64_t seed, uint64_t offset, uint64_t block_index, uint8_t rho[16]) {
    uint32_t ctr[4] = {(uint32_t)block_index, (uint32_t)(block_index >> 32), (uint32_t)offset,
                       (uint32_t)(offset >> 32)};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    nvo_philox4x32_10(ctr, key, w);
    for (int j = 0; j < 16; ++j) rho[j] = (uint8_t)((w[j >> 2] >> (8 * (j & 3))) & 0xFF);
}

/* ------------------------------------------------------------------------------------------------------------
 * 16-point Random Hadamard Transform.  [P1, section on the random Hadamard transform]: each 16-element block
 * along the last dimension is multiplied by a 16x16 Hadamard matrix (entries +-1, orthogonal) randomised every
 * iteration.  READINGS: the randomisation is a diagonal of random signs applied first (y = (1/4) H16 diag(s) v),
 * bit i of the 16-bit mask negating element i; H16 is the Sylvester matrix H[i][j] = (-1)^popcount(i & j); the
 * 1/4 = 1/sqrt(16) factor makes it orthonormal; the product is evaluated as the fast Walsh-Hadamard butterfly
 * with stages of stride 1, 2, 4, 8 in that order, (a, b) -> (a + b, a - b) in binary32, then one multiply by
 * 0.25.  The result stays binary32.
 * ---------------------------------------------------------------------------------------------------------- */
void nvo_rht16(const float v[16], uint16_t sign_mask, float y[16]) {
    float w[16];
    for (int i = 0; i < 16; ++i) w[i] = ((sign_mask >> i) & 1) ? -v[i] : v[i];
    for (int h = 1; h < 16; h *= 2) {
        for (int i = 0; i < 16; ++i) {
            if ((i & h) == 0) {
                float a = w[i], b = w[i + h];
                w[i] = a + b;
                w[i + h] = a - b;
            }
        }
    }
    for (int i = 0; i < 16; ++i) y[i] = 0.25f * w[i];
}

/* Inverse of nvo_rht16.  The forward map is M = (1/4) H16 diag(s) with H16 symmetric and H16 H16 = 16 I, so
 * M^-1 = diag(s) (1/4) H16.  READING (the pages only say the transform is orthogonal; its inverse is its
 * transpose): the product is evaluated in the forward's own way on the decoded block d -- the butterfly with
 * stages of stride 1, 2, 4, 8, (a, b) -> (a + b, a - b) in binary32, then one multiply by 0.25 -- and the random
 * signs are applied last, negating element i where bit i of the mask is set (exact). */
void nvo_rht16_inverse(const float y[16], uint16_t sign_mask, float v[16]) {
    float w[16];
    for (int i = 0; i < 16; ++i) w[i] = y[i];
    for (int h = 1; h < 16; h *= 2) {
        for (int i = 0; i < 16; ++i) {
            if ((i & h) == 0) {
                float a = w[i], b = w[i + h];
                w[i] = a + b;
                w[i + h] = a - b;
            }
        }
    }
    for (int i = 0; i < 16; ++i) {
        float t = 0.25f * w[i];
        v[i] = ((sign_mask >> i) & 1) ? -t : t;
    }
}

/* Absolute maximum as an integer maximum of the magnitude bit patterns.  [P1, sections on the RHT GEMM
 * rewrite and the vibe-coding process]: NaN must propagate (min/max helpers that drop NaN were a bug).  On the
 * magnitude bits, every NaN pattern is above +inf, which is above every finite value, so one NaN makes the
 * result NaN. */
static uint32_t absbits(float f) { return bits_of(f) & 0x7FFFFFFFu; }

/* ------------------------------------------------------------------------------------------------------------
 * Views.  Row-wise quantization works on V = X; column-wise on V = X^T ([P2, results section on amortising
 * weight quantization]: one GEMM contracts quant(w), the other quant(w.t())).  X is row-major [rows, cols] bf16.
 * Blocks are 16 consecutive elements of a row of V.
 * ---------------------------------------------------------------------------------------------------------- */
static int64_t view_rows(int64_t rows, int64_t cols, int orient) { return orient == NVO_ROWWISE ? rows : cols; }
static int64_t view_cols(int64_t rows, int64_t cols, int orient) { return orient == NVO_ROWWISE ? cols : rows; }

static float view_at(const uint16_t* x, int64_t cols, int orient, int64_t vr, int64_t vc) {
    return orient == NVO_ROWWISE ? nvo_bf16_to_f32(x[vr * cols + vc]) : nvo_bf16_to_f32(x[vc * cols + vr]);
}

/* The 16 values of block (vr, block b) of V, transformed by the RHT when use_rht is set. */
static void view_block(const uint16_t* x, int64_t cols, int orient, int64_t vr, int64_t b, int use_rht,
                       uint16_t sign_mask, float y[16]) {
    float v[16];
    for (int i = 0; i < 16; ++i) v[i] = view_at(x, cols, orient, vr, 16 * b + i);
    if (use_rht) nvo_rht16(v, sign_mask, y);
    else memcpy(y, v, sizeof v);
}

static int check_common(const void* x, int64_t rows, int64_t cols, int orient) {
    if (!x) return NVO_ERR_NULL;
    if (rows < 0 || cols < 0) return NVO_ERR_SHAPE;
    if (orient != NVO_ROWWISE && orient != NVO_COLWISE) return NVO_ERR_UNSUPPORTED;
    if (view_cols(rows, cols, orient) % 16 != 0) return NVO_ERR_SHAPE;
    return NVO_OK;
}

/* ------------------------------------------------------------------------------------------------------------
 * Per-tensor (or per-row-of-V) amax.  [P2, results section on quantizer speed]: the per-tensor amax feeds the
 * global scale and is computed on the device.  [P3]: row-scaled global scales are the per-row variant.
 * READING: with the RHT the amax is taken over the transformed values (the ones that get quantized).
 * Output: amax[0] (per tensor) or amax[Rv] (per row of V).
 * ---------------------------------------------------------------------------------------------------------- */
int nvo_amax(const uint16_t* x, int64_t rows, int64_t cols, int orient, int gmode, int use_rht,
             uint16_t sign_mask, float* amax) {
    int st = check_common(x, rows, cols, orient);
    if (st) return st;
    if (!amax) return NVO_ERR_NULL;
    int64_t rv = view_rows(rows, cols, orient), cv = view_cols(rows, cols, orient);
    int64_t nb = cv / 16;
    uint32_t total = 0;
    #pragma omp parallel for schedule(static) reduction(max : total)
    for (int64_t vr = 0; vr < rv; ++vr) {
        uint32_t row_max = 0;
        for (int64_t b = 0; b < nb; ++b) {
            float y[16];
            view_block(x, cols, orient, vr, b, use_rht, sign_mask, y);
            for (int i = 0; i < 16; ++i)
                if (absbits(y[i]) > row_max) row_max = absbits(y[i]);
        }
        if (gmode == NVO_G_PER_ROW) amax[vr] = f32_of(row_max);
        if (row_max > total) total = row_max;
    }
    if (gmode != NVO_G_PER_ROW) amax[0] = f32_of(total);
    return NVO_OK;
}

/* Global scale.  READING: g = amax / (6 * 448) as one binary32 division (2688 is exact); the two factors are
 * the largest E2M1 and E4M3 magnitudes, so the largest block maps its largest element onto 6 with the largest
 * block scale. */
float nvo_global_scale(float amax) { return amax / 2688.0f; }

/* Block scale and encode multiplier for one block.
 * [P2, layout section]: two-level scale, E4M3 per block on top of the FP32 global scale.
 * READINGS: d = fl(T * g) with T = 6 (or 4 for the four-over-six candidate); s = 0 when the block's amax is 0,
 * else fl(bamax / d) (correctly rounded division, as [P3] pins); sb = E4M3(s); the value multiplier is
 * S = fl(decode(sb) * g) and elements are scaled by r = fl(1 / S) (one correctly rounded reciprocal per block,
 * then one multiply per element), with r = 0 when S is 0, r = NaN when S is NaN, and r clamped to FLT_MAX if the
 * reciprocal overflows. */
void nvo_block_scale(float bamax, float g, float T, uint8_t* sb_out, float* r_out) {
    float d = T * g;
    float s = (bamax == 0.0f) ? 0.0f : bamax / d;
    uint8_t sb = nvo_e4m3_encode(s);
    float S = nvo_e4m3_decode(sb) * g;
    float r;
    if (isnan(S)) r = NAN;
    else if (S == 0.0f) r = 0.0f;
    else {
        r = 1.0f / S;
        if (isinf(r)) r = FLT_MAX;
    }
    *sb_out = sb;
    *r_out = r;
}

static float max_of_block(const float* y, int n) {
    uint32_t m = 0;
    for (int i = 0; i < n; ++i)
        if (absbits(y[i]) > m) m = absbits(y[i]);
    return f32_of(m);
}

/* ------------------------------------------------------------------------------------------------------------
 * 1x16 quantization (RN, SR, RHT+SR) of V rows [vr_begin, vr_end).
 * [P1, sections on stochastic rounding and the RHT]; [P2, layout and results sections]: two-level scale and
 * per-GEMM recipes (round-to-nearest for forward activations and weights, SR for gradients, RHT+SR for the
 * weight-gradient operands).
 * Outputs (full-size arrays; only the requested rows are written):
 *   codes  [Rv, Cv/2]  byte k of a row = code[2k] | code[2k+1] << 4   (READING: even element in the low nibble)
 *   scales [Rv, Cv/16] E4M3 codes
 *   g      [1] (per tensor) or [Rv] (per row of V): fl(amax / 2688)
 * amax is [1] or [Rv] as produced by nvo_amax (with the same RHT mask when mode is RHT+SR).
 * ---------------------------------------------------------------------------------------------------------- */
int nvo_quantize_1x16(const uint16_t* x, int64_t rows, int64_t cols, int orient, int gmode, int mode,
                      const float* amax, uint16_t sign_mask, uint64_t seed, uint64_t offset, int64_t vr_begin,
                      int64_t vr_end, uint8_t* codes, uint8_t* scales, float* g) {
    int st = check_common(x, rows, cols, orient);
    if (st) return st;
    if (!amax || !codes || !scales || !g) return NVO_ERR_NULL;
    if (mode != NVO_MODE_RN && mode != NVO_MODE_SR && mode != NVO_MODE_RHT_SR) return NVO_ERR_UNSUPPORTED;
    if (gmode != NVO_G_PER_TENSOR && gmode != NVO_G_PER_ROW) return NVO_ERR_UNSUPPORTED;
    int64_t rv = view_rows(rows, cols, orient), cv = view_cols(rows, cols, orient);
    if (vr_begin < 0 || vr_end > rv || vr_begin > vr_end) return NVO_ERR_SHAPE;
    int64_t nb = cv / 16;
    int use_rht = (mode == NVO_MODE_RHT_SR);
    if (gmode == NVO_G_PER_TENSOR) g[0] = nvo_global_scale(amax[0]);
    #pragma omp parallel for schedule(static)
    for (int64_t vr = vr_begin; vr < vr_end; ++vr) {
        float gr = nvo_global_scale(gmode == NVO_G_PER_ROW ? amax[vr] : amax[0]);
        if (gmode == NVO_G_PER_ROW) g[vr] = gr;
        for (int64_t b = 0; b < nb; ++b) {
            float y[16];
            view_block(x, cols, orient, vr, b, use_rht, sign_mask, y);
            uint8_t sb;
            float r;
            nvo_block_scale(max_of_block(y, 16), gr, 6.0f, &sb, &r);
            uint8_t rho[16];
            if (mode != NVO_MODE_RN) nvo_block_random_bytes(seed, offset, (uint64_t)(vr * nb + b), rho);
            uint8_t code[16];
            for (int i = 0; i < 16; ++i) {
                float q = y[i] * r;
                code[i] = (mode == NVO_MODE_RN) ? nvo_e2m1_rn(q) : nvo_e2m1_sr(q, rho[i]);
            }
            for (int k = 0; k < 8; ++k)
                codes[vr * (cv / 2) + 8 * b + k] = (uint8_t)(code[2 * k] | (code[2 * k + 1] << 4));
            scales[vr * nb + b] = sb;
        }
    }
    return NVO_OK;
}

/* ------------------------------------------------------------------------------------------------------------
 * 16x16 ("2D") weight quantization, RN, per-tensor global scale, both orientations from one pass over the
 * tiles of X in tile rows [tr_begin, tr_end).  [P2, intro]: 2D weight scaling is part of the recipe; [P3]: 1x16
 * and 16x16 blocks; [P2, results section on weight-quant amortisation]: weights are needed as quant(w) and
 * quant(w.t()), both round-to-nearest.
 * READINGS: one E4M3 scale per 16x16 tile from the tile's 256-element amax; every element is scaled and
 * rounded once, so the W^T codes are the W codes transposed; each orientation's scales are stored expanded to
 * the 1x16 layout of that orientation so that both outputs are ordinary NVFP4 tensors:
 *   W   : codes_w  [R, C/2],  scales_w  [R, C/16]  (scales_w[r][j]  = tile (r/16, j))
 *   W^T : codes_wt [C, R/2],  scales_wt [C, R/16]  (scales_wt[c][i] = tile (i, c/16))
 *   g_w[0] = g_wt[0] = fl(amax / 2688).  Any of the output pointers of one orientation may all be NULL to skip it.
 * ---------------------------------------------------------------------------------------------------------- */
int nvo_quantize_16x16(const uint16_t* x, int64_t rows, int64_t cols, const float* amax, int64_t tr_begin,
                       int64_t tr_end, uint8_t* codes_w, uint8_t* scales_w, float* g_w, uint8_t* codes_wt,
                       uint8_t* scales_wt, float* g_wt) {
    if (!x || !amax) return NVO_ERR_NULL;
    if (rows < 0 || cols < 0 || rows % 16 || cols % 16) return NVO_ERR_SHAPE;
    int want_w = codes_w != NULL, want_wt = codes_wt != NULL;
    if ((want_w && (!scales_w || !g_w)) || (want_wt && (!scales_wt || !g_wt)) || (!want_w && !want_wt))
        return NVO_ERR_NULL;
    int64_t ntr = rows / 16, ntc = cols / 16;
    if (tr_begin < 0 || tr_end > ntr || tr_begin > tr_end) return NVO_ERR_SHAPE;
    float g = nvo_global_scale(amax[0]);
    if (want_w) g_w[0] = g;
    if (want_wt) g_wt[0] = g;
    #pragma omp parallel for schedule(static)
    for (int64_t ti = tr_begin; ti < tr_end; ++ti) {
        for (int64_t tj = 0; tj < ntc; ++tj) {
            float v[256];
            for (int i = 0; i < 16; ++i)
                for (int j = 0; j < 16; ++j) v[16 * i + j] = nvo_bf16_to_f32(x[(16 * ti + i) * cols + 16 * tj + j]);
            uint8_t sb;
            float r;
            nvo_block_scale(max_of_block(v, 256), g, 6.0f, &sb, &r);
            uint8_t code[256];
            for (int e = 0; e < 256; ++e) code[e] = nvo_e2m1_rn(v[e] * r);
            for (int i = 0; i < 16; ++i) {
                int64_t rr = 16 * ti + i, cc = 16 * tj + i;
                for (int k = 0; k < 8; ++k) {
                    if (want_w)    /* row rr of W: elements (i, 2k), (i, 2k+1) of the tile */
                        codes_w[rr * (cols / 2) + 8 * tj + k] =
                            (uint8_t)(code[16 * i + 2 * k] | (code[16 * i + 2 * k + 1] << 4));
                    if (want_wt)   /* row cc of W^T: elements (2k, i), (2k+1, i) of the tile */
                        codes_wt[cc * (rows / 2) + 8 * ti + k] =
                            (uint8_t)(code[16 * (2 * k) + i] | (code[16 * (2 * k + 1) + i] << 4));
                }
                if (want_w) scales_w[rr * ntc + tj] = sb;
                if (want_wt) scales_wt[cc * ntr + ti] = sb;
            }
        }
    }
    return NVO_OK;
}

/* ------------------------------------------------------------------------------------------------------------
 * Four-over-six, row-wise 1x16, round-to-nearest, no RHT, rows [r_begin, r_end).  [P3]: every block is encoded
 * at the standard map-to-6 scale and at a 1.5x larger map-to-4 scale, both candidates are decoded, and the one
 * with the lower error is stored; the width-16 error reduction has a pinned order (a shuffle-down tree); the
 * recipe's sweep varies an error mode and a bound, which the page names without defining.
 * READINGS: candidate T in {6, 4} uses d_T = fl(T * g) in the block-scale rule above (bamax / (4g) is 1.5x
 * bamax / (6g) in exact arithmetic); decode xh = fl(fl(val(code) * decode(sb_T)) * g); d_i = fl(xh_i - x_i)
 * against the binary32 input.  The block error by err_mode:
 *   NVO_ERR_MSE    e_i = fl(d_i * d_i), summed by the tree p_i = e_i + e_{i+8} (i < 8), then strides 4, 2, 1;
 *   NVO_ERR_MAE    e_i = |d_i| (exact), summed by the same tree;
 *   NVO_ERR_MAXABS the largest |d_i| (no rounding, so no order), NaN if any d_i is NaN.
 * bound B (an integer 1..448) is the E4M3 value the tensor maximum's map-to-6 scale lands on: g = fl(A / (6 B)),
 * 6 B exact; B = 448 is the standard g = A / 2688, and B = 256 leaves the map-to-4 scale of every block
 * (at most 1.5 B = 384) below E4M3's 448, where with B = 448 the largest blocks' map-to-4 scales saturate.
 * Map-to-4 is kept only if its error is strictly lower, so ties and NaN keep map-to-6.  choice[] (optional)
 * receives 1 where map-to-4 was kept.
 * ---------------------------------------------------------------------------------------------------------- */
#define NVO_ERR_MSE 0
#define NVO_ERR_MAE 1
#define NVO_ERR_MAXABS 2

static float tree_sum16(const float e[16]) {
    float p[16];
    memcpy(p, e, sizeof p);
    for (int s = 8; s >= 1; s /= 2)
        for (int i = 0; i < s; ++i) p[i] = p[i] + p[i + s];
    return p[0];
}

/* The largest of n magnitudes, NaN if any is NaN. */
static float max_or_nan(const float* a, int n) {
    float m = 0.0f;
    for (int i = 0; i < n; ++i) {
        if (isnan(a[i])) return NAN;
        if (a[i] > m) m = a[i];
    }
    return m;
}

/* The error of 16 differences d under err_mode (the width-16 reduction above). */
static float error16(const float d[16], int err_mode) {
    float e[16];
    for (int i = 0; i < 16; ++i) e[i] = (err_mode == NVO_ERR_MSE) ? d[i] * d[i] : fabsf(d[i]);
    return (err_mode == NVO_ERR_MAXABS) ? max_or_nan(e, 16) : tree_sum16(e);
}

/* g = fl(A / (6 B)) for a bound B in 1..448 (6 B <= 2688 is exact). */
static float global_scale_bound(float amax, int bound) { return amax / (float)(6 * bound); }

static int knobs_ok(int err_mode, int bound) {
    return (err_mode == NVO_ERR_MSE || err_mode == NVO_ERR_MAE || err_mode == NVO_ERR_MAXABS) && bound >= 1 &&
           bound <= 448;
}

/* The input element (r, c): a bf16 pattern widened exactly, or a binary32 value as given.  [P3]: the reference
 * quantizer takes bf16 or fp32 inputs and its sweep covers both dtypes; every later step is the same. */
static float input_at(const uint16_t* xb, const float* xf, int64_t cols, int64_t r, int64_t c) {
    return xb ? nvo_bf16_to_f32(xb[r * cols + c]) : xf[r * cols + c];
}

static int quantize_4o6_rows(const uint16_t* xb, const float* xf, int64_t rows, int64_t cols, int gmode,
                             int err_mode, int bound, const float* amax, int64_t r_begin, int64_t r_end,
                             uint8_t* codes, uint8_t* scales, float* g, uint8_t* choice);

int nvo_quantize_4o6(const uint16_t* x, int64_t rows, int64_t cols, int gmode, int err_mode, int bound,
                     const float* amax, int64_t r_begin, int64_t r_end, uint8_t* codes, uint8_t* scales, float* g,
                     uint8_t* choice) {
    if (!x) return NVO_ERR_NULL;
    return quantize_4o6_rows(x, NULL, rows, cols, gmode, err_mode, bound, amax, r_begin, r_end, codes, scales, g,
                             choice);
}

/* Four-over-six of a binary32 input: nvo_quantize_4o6 on the values as given. */
int nvo_quantize_4o6_f32(const float* x, int64_t rows, int64_t cols, int gmode, int err_mode, int bound,
                         const float* amax, int64_t r_begin, int64_t r_end, uint8_t* codes, uint8_t* scales,
                         float* g, uint8_t* choice) {
    if (!x) return NVO_ERR_NULL;
    return quantize_4o6_rows(NULL, x, rows, cols, gmode, err_mode, bound, amax, r_begin, r_end, codes, scales, g,
                             choice);
}

/* Row-wise amax of a binary32 input (no transform), per tensor or per row: the largest magnitude as an integer
 * maximum of the magnitude bits, so NaN > inf > every finite value, as nvo_amax does for bf16. */
int nvo_amax_f32(const float* x, int64_t rows, int64_t cols, int gmode, float* amax) {
    if (!x || !amax) return NVO_ERR_NULL;
    if (rows < 0 || cols < 0 || cols % 16) return NVO_ERR_SHAPE;
    uint32_t total = 0;
    for (int64_t r = 0; r < rows; ++r) {
        uint32_t row_max = 0;
        for (int64_t c = 0; c < cols; ++c)
            if (absbits(x[r * cols + c]) > row_max) row_max = absbits(x[r * cols + c]);
        if (gmode == NVO_G_PER_ROW) amax[r] = f32_of(row_max);
        if (row_max > total) total = row_max;
    }
    if (gmode != NVO_G_PER_ROW) amax[0] = f32_of(total);
    return NVO_OK;
}

static int quantize_4o6_rows(const uint16_t* xb, const float* xf, int64_t rows, int64_t cols, int gmode,
                             int err_mode, int bound, const float* amax, int64_t r_begin, int64_t r_end,
                             uint8_t* codes, uint8_t* scales, float* g, uint8_t* choice) {
    if (!amax || !codes || !scales || !g) return NVO_ERR_NULL;
    if (rows < 0 || cols < 0 || cols % 16) return NVO_ERR_SHAPE;
    if (gmode != NVO_G_PER_TENSOR && gmode != NVO_G_PER_ROW) return NVO_ERR_UNSUPPORTED;
    if (!knobs_ok(err_mode, bound)) return NVO_ERR_UNSUPPORTED;
    if (r_begin < 0 || r_end > rows || r_begin > r_end) return NVO_ERR_SHAPE;
    int64_t nb = cols / 16;
    if (gmode == NVO_G_PER_TENSOR) g[0] = global_scale_bound(amax[0], bound);
    #pragma omp parallel for schedule(static)
    for (int64_t r = r_begin; r < r_end; ++r) {
        float gr = global_scale_bound(gmode == NVO_G_PER_ROW ? amax[r] : amax[0], bound);
        if (gmode == NVO_G_PER_ROW) g[r] = gr;
        for (int64_t b = 0; b < nb; ++b) {
            float xv[16];
            for (int i = 0; i < 16; ++i) xv[i] = input_at(xb, xf, cols, r, 16 * b + i);
            float bamax = max_of_block(xv, 16);
            uint8_t cand_code[2][16], cand_sb[2];
            float err[2];
            const float T[2] = {6.0f, 4.0f};
            for (int c = 0; c < 2; ++c) {
                float rr;
                nvo_block_scale(bamax, gr, T[c], &cand_sb[c], &rr);
                float sbf = nvo_e4m3_decode(cand_sb[c]);
                float d[16];
                for (int i = 0; i < 16; ++i) {
                    cand_code[c][i] = nvo_e2m1_rn(xv[i] * rr);
                    float xh = (nvo_e2m1_decode(cand_code[c][i]) * sbf) * gr;
                    d[i] = xh - xv[i];
                }
                err[c] = error16(d, err_mode);
            }
            int pick = (err[1] < err[0]) ? 1 : 0;
            for (int k = 0; k < 8; ++k)
                codes[r * (cols / 2) + 8 * b + k] =
                    (uint8_t)(cand_code[pick][2 * k] | (cand_code[pick][2 * k + 1] << 4));
            scales[r * nb + b] = cand_sb[pick];
            if (choice) choice[r * nb + b] = (uint8_t)pick;
        }
    }
    return NVO_OK;
}

/* ------------------------------------------------------------------------------------------------------------
 * Four-over-six with 16x16 blocks.  [P3]: the four-over-six reference quantizer takes 1x16 or 16x16 blocks, with a
 * per-tensor global scale for the 16x16 case here (a tile spans 16 rows, so a row-scaled g does not define one
 * tile scale).  Per 16x16 tile of X: tamax = the NaN-dominant maximum magnitude of its 256 values; for T in {6, 4}
 * the tile scale sb_T and the element codes follow the 1x16 rules with tamax in place of bamax; the decoded values
 * and their differences are as in the 1x16 case, with the same err_mode and bound.  READING (the pages pin only
 * the width-16 reduction): each of the tile's 16 rows is reduced as a 1x16 block is (error16), then the 16 row
 * errors (row 0 first) the same way: by the width-16 tree for MSE and MAE, as a maximum for MAXABS; map-to-4 is
 * kept only if its tile error is strictly lower.  The chosen codes are written in W (packed along X's rows) and/or
 * W^T (packed along X's columns) orientation, with the tile's scale repeated in each orientation's 1x16 scale
 * layout, exactly as nvo_quantize_16x16.  choice[tile] (optional, [rows/16, cols/16]) receives 1 for map-to-4.
 * ---------------------------------------------------------------------------------------------------------- */
static int quantize_4o6_tiles(const uint16_t* xb, const float* xf, int64_t rows, int64_t cols, int err_mode,
                              int bound, const float* amax, int64_t tr_begin, int64_t tr_end, uint8_t* codes_w,
                              uint8_t* scales_w, float* g_w, uint8_t* codes_wt, uint8_t* scales_wt, float* g_wt,
                              uint8_t* choice);

int nvo_quantize_4o6_16x16(const uint16_t* x, int64_t rows, int64_t cols, int err_mode, int bound,
                           const float* amax, int64_t tr_begin, int64_t tr_end, uint8_t* codes_w, uint8_t* scales_w,
                           float* g_w, uint8_t* codes_wt, uint8_t* scales_wt, float* g_wt, uint8_t* choice) {
    if (!x) return NVO_ERR_NULL;
    return quantize_4o6_tiles(x, NULL, rows, cols, err_mode, bound, amax, tr_begin, tr_end, codes_w, scales_w, g_w,
                              codes_wt, scales_wt, g_wt, choice);
}

/* The same for a binary32 input ([P3]: bf16 or fp32 inputs), on the values as given. */
int nvo_quantize_4o6_16x16_f32(const float* x, int64_t rows, int64_t cols, int err_mode, int bound,
                               const float* amax, int64_t tr_begin, int64_t tr_end, uint8_t* codes_w,
                               uint8_t* scales_w, float* g_w, uint8_t* codes_wt, uint8_t* scales_wt, float* g_wt,
                               uint8_t* choice) {
    if (!x) return NVO_ERR_NULL;
    return quantize_4o6_tiles(NULL, x, rows, cols, err_mode, bound, amax, tr_begin, tr_end, codes_w, scales_w, g_w,
                              codes_wt, scales_wt, g_wt, choice);
}

static int quantize_4o6_tiles(const uint16_t* xb, const float* xf, int64_t rows, int64_t cols, int err_mode,
                              int bound, const float* amax, int64_t tr_begin, int64_t tr_end, uint8_t* codes_w,
                              uint8_t* scales_w, float* g_w, uint8_t* codes_wt, uint8_t* scales_wt, float* g_wt,
                              uint8_t* choice) {
    if (!amax) return NVO_ERR_NULL;
    if (rows < 0 || cols < 0 || rows % 16 || cols % 16) return NVO_ERR_SHAPE;
    if (!knobs_ok(err_mode, bound)) return NVO_ERR_UNSUPPORTED;
    int want_w = codes_w != NULL, want_wt = codes_wt != NULL;
    if ((want_w && (!scales_w || !g_w)) || (want_wt && (!scales_wt || !g_wt)) || (!want_w && !want_wt))
        return NVO_ERR_NULL;
    int64_t ntr = rows / 16, ntc = cols / 16;
    if (tr_begin < 0 || tr_end > ntr || tr_begin > tr_end) return NVO_ERR_SHAPE;
    float g = global_scale_bound(amax[0], bound);
    if (want_w) g_w[0] = g;
    if (want_wt) g_wt[0] = g;
    #pragma omp parallel for schedule(static)
    for (int64_t ti = tr_begin; ti < tr_end; ++ti) {
        for (int64_t tj = 0; tj < ntc; ++tj) {
            float v[256];
            for (int i = 0; i < 16; ++i)
                for (int j = 0; j < 16; ++j) v[16 * i + j] = input_at(xb, xf, cols, 16 * ti + i, 16 * tj + j);
            float tamax = max_of_block(v, 256);
            uint8_t cand_code[2][256], cand_sb[2];
            float err[2];
            const float T[2] = {6.0f, 4.0f};
            for (int c = 0; c < 2; ++c) {
                float r;
                nvo_block_scale(tamax, g, T[c], &cand_sb[c], &r);
                float sbf = nvo_e4m3_decode(cand_sb[c]);
                float rowerr[16];
                for (int i = 0; i < 16; ++i) {
                    float d[16];
                    for (int j = 0; j < 16; ++j) {
                        uint8_t code = nvo_e2m1_rn(v[16 * i + j] * r);
                        cand_code[c][16 * i + j] = code;
                        float xh = (nvo_e2m1_decode(code) * sbf) * g;
                        d[j] = xh - v[16 * i + j];
                    }
                    rowerr[i] = error16(d, err_mode);
                }
                err[c] = (err_mode == NVO_ERR_MAXABS) ? max_or_nan(rowerr, 16) : tree_sum16(rowerr);
            }
            int pick = (err[1] < err[0]) ? 1 : 0;
            const uint8_t* code = cand_code[pick];
            uint8_t sb = cand_sb[pick];
            if (choice) choice[ti * ntc + tj] = (uint8_t)pick;
            for (int i = 0; i < 16; ++i) {
                int64_t rr = 16 * ti + i, cc = 16 * tj + i;
                for (int k = 0; k < 8; ++k) {
                    if (want_w)
                        codes_w[rr * (cols / 2) + 8 * tj + k] =
                            (uint8_t)(code[16 * i + 2 * k] | (code[16 * i + 2 * k + 1] << 4));
                    if (want_wt)
                        codes_wt[cc * (rows / 2) + 8 * ti + k] =
                            (uint8_t)(code[16 * (2 * k) + i] | (code[16 * (2 * k + 1) + i] << 4));
                }
                if (want_w) scales_w[rr * ntc + tj] = sb;
                if (want_wt) scales_wt[cc * ntr + ti] = sb;
            }
        }
    }
    return NVO_OK;
}

/* ------------------------------------------------------------------------------------------------------------
 * Standard NVFP4 decode.  [P3]: a recipe-agnostic decode of codes, block scales and global scale.
 * y = fl(fl(val(code) * decode(sb)) * g) in binary32 (the inner product is exact: at most 2 x 4 significant bits).
 * codes [rv, cv/2], scales [rv, cv/16], g [1] or [rv]; y [rv, cv] binary32.
 * ---------------------------------------------------------------------------------------------------------- */
int nvo_dequantize(const uint8_t* codes, const uint8_t* scales, const float* g, int64_t rv, int64_t cv, int gmode,
                   float* y) {
    if (!codes || !scales || !g || !y) return NVO_ERR_NULL;
    if (rv < 0 || cv < 0 || cv % 16) return NVO_ERR_SHAPE;
    if (gmode != NVO_G_PER_TENSOR && gmode != NVO_G_PER_ROW) return NVO_ERR_UNSUPPORTED;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rv; ++r) {
        float gr = (gmode == NVO_G_PER_ROW) ? g[r] : g[0];
        for (int64_t c = 0; c < cv; ++c) {
            uint8_t byte = codes[r * (cv / 2) + c / 2];
            uint8_t code = (c & 1) ? (byte >> 4) : (byte & 0xF);
            float sbf = nvo_e4m3_decode(scales[r * (cv / 16) + c / 16]);
            y[r * cv + c] = (nvo_e2m1_decode(code) * sbf) * gr;
        }
    }
    return NVO_OK;
}

/* binary32 -> bf16, round to nearest even on the 16 dropped bits.  READING (the pages name bf16 as the
 * high-precision format and never state a rounding for it): IEEE round-to-nearest-even, the usual conversion;
 * overflow rounds to infinity as in IEEE; every NaN becomes the quiet NaN 0x7FC0 (the sign of a NaN made by
 * arithmetic, such as inf - inf, differs between processors, so no NaN sign is part of the result).  Found by
 * comparing the candidate values: the two bf16 neighbours of x are the truncation t and the next pattern
 * t + 1 (same sign), and x goes to the nearer in exact binary64 arithmetic, to the even pattern on a tie. */
uint16_t nvo_f32_to_bf16(float x) {
    if (isnan(x)) return 0x7FC0;
    uint32_t u = bits_of(x);
    uint16_t t = (uint16_t)(u >> 16);                 /* truncation toward zero: |bf16(t)| <= |x| */
    if ((u & 0xFFFF) == 0) return t;                   /* exactly representable (includes +-0 and +-inf) */
    uint16_t up = (uint16_t)(t + 1);                   /* next magnitude (may become +-inf: exponent all ones) */
    double dx = fabs((double)x);
    double dt = fabs((double)f32_of((uint32_t)t << 16));
    double du = fabs((double)f32_of((uint32_t)up << 16));   /* +inf when t is the largest finite magnitude */
    double lo = dx - dt, hi = du - dx;                 /* both exact in binary64; hi is inf for du = inf */
    if (isinf(du)) {
        /* the gap above the largest finite bf16 is that of the binade below: ties and beyond go to inf */
        hi = dt + (dt - fabs((double)f32_of((uint32_t)(t - 1) << 16))) - dx;
    }
    if (lo < hi) return t;
    if (hi < lo) return up;
    return (t & 1) ? up : t;
}

/* Fused decode.  [P3]: the optimized decode is named as future kernel work; [P1, random Hadamard transform]:
 * blocks quantized after the rotation are brought back by its inverse.  Per 16-element block of a row:
 * d_i = fl(fl(val(code_i) * decode(sb)) * g) (as nvo_dequantize), then, when use_rht is set,
 * z = nvo_rht16_inverse(d, sign_mask), and the binary32 result is written as float (out_bf16 = 0) or rounded by
 * nvo_f32_to_bf16 (out_bf16 = 1).  y is [rv, cv] float or uint16 (bf16 bit patterns). */
int nvo_dequantize_fused(const uint8_t* codes, const uint8_t* scales, const float* g, int64_t rv, int64_t cv,
                         int gmode, int use_rht, uint16_t sign_mask, int out_bf16, void* y) {
    if (!codes || !scales || !g || !y) return NVO_ERR_NULL;
    if (rv < 0 || cv < 0 || cv % 16) return NVO_ERR_SHAPE;
    if (gmode != NVO_G_PER_TENSOR && gmode != NVO_G_PER_ROW) return NVO_ERR_UNSUPPORTED;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rv; ++r) {
        float gr = (gmode == NVO_G_PER_ROW) ? g[r] : g[0];
        for (int64_t b = 0; b < cv / 16; ++b) {
            float d[16], z[16];
            float sbf = nvo_e4m3_decode(scales[r * (cv / 16) + b]);
            for (int i = 0; i < 16; ++i) {
                uint8_t byte = codes[r * (cv / 2) + 8 * b + i / 2];
                uint8_t code = (i & 1) ? (byte >> 4) : (byte & 0xF);
                d[i] = (nvo_e2m1_decode(code) * sbf) * gr;
            }
            if (use_rht) nvo_rht16_inverse(d, sign_mask, z);
            else memcpy(z, d, sizeof z);
            for (int i = 0; i < 16; ++i) {
                int64_t k = r * cv + 16 * b + i;
                if (out_bf16) ((uint16_t*)y)[k] = nvo_f32_to_bf16(z[i]);
                else ((float*)y)[k] = z[i];
            }
        }
    }
    return NVO_OK;
}

/* ------------------------------------------------------------------------------------------------------------
 * Tiled scale layout for the FP4 GEMM ([P2, approach]: the quantized operands go to the FP4 GEMM with 1x16 block
 * scales in the SWIZZLE_32_4_4 layout; [P2, results]: that swizzle is part of the per-call wrapper overhead).
 * READING (the pages name the layout only): the scale matrix [rv, nb] (nb = scales per row) is cut into tiles of
 * 128 rows x 4 scale columns, padded with zero bytes to whole tiles; tiles are stored one after another, row tile
 * major (tile (R, B) at byte 512 * (R * ceil(nb/4) + B)), and inside a tile the 512 bytes are the [32][4][4] array
 * the name spells out: byte 16 a + 4 b + c holds the scale of row 128 R + 32 b + a, column 4 B + c.  This is the
 * layout of the 1D block-scaling factors in the cuBLAS documentation.  out holds
 * ceil(rv/128) * 128 * ceil(nb/4) * 4 bytes.
 * ---------------------------------------------------------------------------------------------------------- */
int nvo_swizzle_scales(const uint8_t* scales, int64_t rv, int64_t nb, uint8_t* out) {
    if (!out || (rv * nb > 0 && !scales)) return NVO_ERR_NULL;
    if (rv < 0 || nb < 0) return NVO_ERR_SHAPE;
    int64_t rt = (rv + 127) / 128, bt = (nb + 3) / 4;
    memset(out, 0, (size_t)(rt * bt * 512));
    for (int64_t m = 0; m < rv; ++m) {
        for (int64_t k = 0; k < nb; ++k) {
            int64_t tile = (m / 128) * bt + k / 4;
            int64_t a = m % 32, b = (m % 128) / 32, c = k % 4;
            out[tile * 512 + 16 * a + 4 * b + c] = scales[m * nb + k];
        }
    }
    return NVO_OK;
}
