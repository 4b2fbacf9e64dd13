/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 training quantizer.
 *
 * Pages cited (title, then the section):
 *   [P1] "在 RTX 5090 (SM120) 上补全 NVFP4 量化相关 kernel" -- blog post on polyfilling NVFP4 quantization kernels
 *        for the RTX 5090 (harrychen.xyz, 2026-04-14).
 *   [P2] "nvfp4-sm120" repository README.
 *   [P3] pytorch/ao pull request #4852, "Add a CuTe DSL fast-path kernel for four-over-six quantize".
 *
 * The method.  A bf16 tensor is quantized to NVFP4: E2M1 4-bit codes (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
 * [P1, FP4 quantization techniques]) with one E4M3 scale per block of 16 consecutive elements (or per 16x16
 * tile) on top of one FP32 global scale g = amax / (6 * 448) per tensor or per row ([P2, layout]; [P3]).
 * Rounding is round-to-nearest-even or stochastic rounding with Philox random bytes ([P1, stochastic rounding]);
 * optionally each 16-element block is first rotated by a 16x16 Hadamard matrix with random signs
 * ([P1, random Hadamard transform]).  Four-over-six ([P3]) encodes every block at the map-to-6 and the
 * 1.5x-scale map-to-4 scale and keeps the one with lower squared error.
 *
 * Conventions shared by every entry point
 *   - Every tensor argument is DEVICE memory owned by the caller.  The library never allocates, frees or
 *     synchronises; every call is asynchronous on `stream` (a hipStream_t; NULL = the default stream).
 *     The global amax stays on the device: nothing is read back to the host ([P2, results: a host sync on the
 *     amax dominated quantization time]).
 *   - Inputs are bf16 bit patterns (uint16), row-major and contiguous, [rows, cols]; the *_f32 calls take
 *     binary32 instead.
 *   - "View" V: row-wise quantization works on V = X ([rows, cols]); column-wise on V = X^T ([cols, rows]),
 *     read directly from X without a transposed copy.  Blocks are 16 consecutive elements of a row of V.
 *   - Outputs of a quantization (struct nvfp4_out, all device pointers):
 *       codes  [Rv, Cv/2] uint8: byte k of a row holds element 2k in its low nibble and 2k+1 in its high nibble;
 *              a code is sign << 3 | m, m indexing the magnitude list above;
 *       scales [Rv, Cv/16] uint8: E4M3 ("fn": bias 7, max 448, 0x7F = NaN) block scales, or the FP4 GEMM's
 *              tiled layout when scale_layout is NVFP4_SCALES_TILED (see nvfp4_scale_layout);
 *       g      [1] (per tensor) or [Rv] (per row of V) float: the global scale amax / 2688 actually used.
 *   - Element scaling: with T = 6, s = bamax / fl(T g) (correctly rounded), sb = E4M3(s) (round to nearest even,
 *     saturating at 448, NaN -> 0x7F), S = fl(decode(sb) g), r = fl(1 / S) (r = 0 if S = 0, NaN if S is NaN,
 *     FLT_MAX if it overflows), q_i = fl(y_i r); E2M1(q_i) saturates at +-6 and maps NaN to 0x7.
 *   - NaN propagates: the amax is the integer maximum of the magnitude bit patterns, so one NaN (or inf) makes
 *     the amax NaN (or inf) and every block of that tensor (or row) decodes to NaN ([P1, RHT GEMM rewrite and
 *     vibe-coding sections: dropping NaN in min/max was a bug]).
 *   - Errors: arguments are validated on the host before anything is enqueued.  On an error the call returns a
 *     non-zero nvfp4_status and enqueues nothing; there is no fallback path.  NVFP4_ERR_HIP reports a failed
 *     launch (the kernels may then not have run).
 *   - Alignment: x, codes, scales and y must be 16-byte aligned; amax and g 4-byte aligned.
 *   - Sizes: rows, cols >= 0; rows * cols < 2^35.  Column-wise views and 16x16 blocks also need cols < 2^25.
 *     A zero-sized tensor is valid: its amax is 0 and a quantize call only writes g.
 *   - Calls on different streams may run concurrently; they share no state (nvfp4_amax_quantize: see it).
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NVFP4_OK = 0,
    NVFP4_ERR_NULL = 1,        /* a required pointer is NULL */
    NVFP4_ERR_SHAPE = 2,       /* a size is negative, too large, or not the multiple of 16 (or 8) required */
    NVFP4_ERR_ALIGN = 3,       /* a pointer is not aligned as required */
    NVFP4_ERR_UNSUPPORTED = 4, /* an unknown enum value or an unsupported combination */
    NVFP4_ERR_HIP = 5          /* the HIP runtime reported an error when launching */
} nvfp4_status;

typedef enum { NVFP4_ROWWISE = 1, NVFP4_COLWISE = 2, NVFP4_BOTH = 3 } nvfp4_orient;
typedef enum { NVFP4_BLOCK_1X16 = 0, NVFP4_BLOCK_16X16 = 1 } nvfp4_block;
typedef enum { NVFP4_G_PER_TENSOR = 0, NVFP4_G_PER_ROW = 1 } nvfp4_gmode;
typedef enum {
    NVFP4_ROUND_RN = 0,
    NVFP4_ROUND_SR = 1,
    NVFP4_ROUND_RHT_SR = 2,
    NVFP4_ROUND_4O6 = 3   /* four-over-six: grouped calls only (nvfp4_quantize_4o6 for one tensor) */
} nvfp4_rounding;

/* Layout of an output's scale codes.  NVFP4_SCALES_TILED is the FP4 GEMM's tiled layout (see
 * nvfp4_swizzle_scales: nvfp4_swizzled_scales_size(Rv, Cv/16) bytes, padding written as zero), written by the
 * quantize kernels themselves; it is taken by the 1x16 quantize calls (nvfp4_quantize_rn with NVFP4_BLOCK_1X16,
 * nvfp4_quantize_sr, nvfp4_quantize_rht_sr and nvfp4_amax_quantize, either orientation).  The 16x16, four-over-six
 * and grouped calls return NVFP4_ERR_UNSUPPORTED for it (their scales can be re-laid by nvfp4_swizzle_scales). */
typedef enum { NVFP4_SCALES_ROWMAJOR = 0, NVFP4_SCALES_TILED = 1 } nvfp4_scale_layout;

/* Four-over-six error measure ([P3]: the recipe's sweep varies an error mode, named there without a definition).
 * With d_i = fl(xhat_i - x_i), xhat the candidate's decoded value: NVFP4_4O6_MSE sums fl(d_i * d_i), NVFP4_4O6_MAE
 * sums |d_i| (both by the width-16 tree: (i, i+8), then strides 4, 2, 1), NVFP4_4O6_MAXABS takes the largest |d_i|
 * (NaN if any d_i is NaN).  A 16x16 tile combines its 16 row errors the same way (tree, or maximum). */
typedef enum { NVFP4_4O6_MSE = 0, NVFP4_4O6_MAE = 1, NVFP4_4O6_MAXABS = 2 } nvfp4_4o6_error;

/* Four-over-six bound ([P3]: the sweep's "bound", named without a definition): the E4M3 value B (an integer,
 * 1 <= B <= 448) that the tensor maximum's map-to-6 scale lands on, g = fl(amax / (6 B)) with 6 B exact.
 * NVFP4_4O6_BOUND_STD (448) is the standard g = amax / 2688; NVFP4_4O6_BOUND_HEADROOM (256) keeps every map-to-4
 * scale (at most 1.5 B = 384) below E4M3's 448, where with 448 the largest blocks' map-to-4 scales saturate. */
#define NVFP4_4O6_BOUND_STD 448
#define NVFP4_4O6_BOUND_HEADROOM 256

typedef struct {
    uint8_t* codes;       /* [Rv, Cv/2] */
    uint8_t* scales;      /* [Rv, Cv/16] (NVFP4_SCALES_ROWMAJOR) or the tiled layout */
    float* g;             /* [1] or [Rv] */
    int32_t scale_layout; /* nvfp4_scale_layout; zero-initialised = row-major */
} nvfp4_out;

/* One tensor of a grouped call (row-wise view, 1x16 blocks).  All pointers are device memory. */
#define NVFP4_MAX_GROUP 32
typedef struct {
    const uint16_t* x;   /* [rows, cols] bf16 */
    int64_t rows, cols;  /* cols % 16 == 0 */
    float* amax;         /* [1] or [rows] (gmode): written by nvfp4_amax_grouped, read by nvfp4_quantize_grouped */
    nvfp4_out out;       /* codes [rows, cols/2], scales [rows, cols/16], g [1] or [rows]; unused by the amax call */
    uint16_t sign_mask;  /* the random signs of the transform (RHT+SR, and the amax with use_rht) */
    uint64_t seed;       /* Philox key (SR, RHT+SR) */
    uint64_t offset;     /* Philox offset (SR, RHT+SR) */
} nvfp4_group_item;

/* Absolute maximum ([P2, results: per-tensor amax kept on the device]; [P3]: row-scaled global scales).
 *   x [rows, cols] bf16; orient NVFP4_ROWWISE or NVFP4_COLWISE selects the view V;
 *   gmode NVFP4_G_PER_TENSOR writes amax[0], NVFP4_G_PER_ROW writes amax[Rv] (one per row of V);
 *   use_rht != 0: the maximum is taken over the Hadamard-transformed blocks (same sign_mask as the quantize call).
 *   Shape: the same rules as the quantize call it feeds: row-wise cols % 16 == 0; column-wise rows % 16 == 0
 *   (any cols below 2^25). */
nvfp4_status nvfp4_amax(const uint16_t* x, int64_t rows, int64_t cols, nvfp4_orient orient, nvfp4_gmode gmode,
                        int use_rht, uint16_t sign_mask, float* amax, void* stream);

/* Round-to-nearest quantization ([P1, stochastic rounding: IEEE round-to-nearest is the hardware default];
 * [P2, layout and results: forward activations and both weight orientations use round-to-nearest]).
 *   block NVFP4_BLOCK_1X16: orient ROWWISE writes *row_out, COLWISE writes *col_out (the other may be NULL).
 *   block NVFP4_BLOCK_16X16 ([P2, intro: 2D weight scaling]; [P3]: 16x16 blocks): one E4M3 scale per 16x16 tile
 *     of X, per-tensor g only; orient ROWWISE writes W to *row_out ([rows, cols/2] codes, [rows, cols/16] scales),
 *     COLWISE writes W^T to *col_out ([cols, rows/2], [cols, rows/16]), BOTH writes both from one read of X.
 *     Each tile's scale is repeated in the 1x16 scale layout of each orientation (16 entries per tile).
 *   amax: [1] or [Rv] device floats from nvfp4_amax (without RHT).
 *   Shape: 1x16 row-wise needs cols % 16 == 0; column-wise rows % 16 == 0 (any cols below 2^25: the blocked
 *   dimension is the only one the method constrains); 16x16 needs both rows and cols multiples of 16.
 *   Unsupported: 16x16 with per-row g; 1x16 with BOTH. */
nvfp4_status nvfp4_quantize_rn(const uint16_t* x, int64_t rows, int64_t cols, nvfp4_block block,
                               nvfp4_orient orient, nvfp4_gmode gmode, const float* amax, const nvfp4_out* row_out,
                               const nvfp4_out* col_out, void* stream);

/* Stochastic-rounding quantization, 1x16 blocks ([P1, stochastic rounding]: P(up) = (x - a) / (b - a); the
 * random source is 8 bits per element).  Element j of the block with row-major index n in V rounds up iff
 * rho < floor(256 (t - a) / (b - a)), rho = byte (j % 4) of word (j / 4) of Philox4x32-10 with
 * key = (seed lo, seed hi) and counter = (n lo, n hi, offset lo, offset hi).  A new offset per call gives fresh
 * randomness; the same (seed, offset) reproduces the same bits.
 *   orient ROWWISE or COLWISE (writes *out).  amax from nvfp4_amax without RHT. */
nvfp4_status nvfp4_quantize_sr(const uint16_t* x, int64_t rows, int64_t cols, nvfp4_orient orient,
                               nvfp4_gmode gmode, const float* amax, uint64_t seed, uint64_t offset,
                               const nvfp4_out* out, void* stream);

/* Random Hadamard Transform + stochastic rounding, 1x16 blocks ([P1, random Hadamard transform and RHT GEMM
 * rewrite]: the fused rotate-and-quantize used for weight-gradient operands, [P2, results: Wgrad RHT+SR]).
 * Each 16-element block v of V becomes y = (1/4) H16 diag(s) v (Sylvester H16, s_i = -1 where bit i of
 * sign_mask is set), evaluated as the butterfly with strides 1, 2, 4, 8 in binary32 followed by one multiply
 * by 0.25; y is then quantized as in nvfp4_quantize_sr.
 *   amax: from nvfp4_amax with use_rht = 1 and the same sign_mask (the amax of the transformed values). */
nvfp4_status nvfp4_quantize_rht_sr(const uint16_t* x, int64_t rows, int64_t cols, nvfp4_orient orient,
                                   nvfp4_gmode gmode, const float* amax, uint16_t sign_mask, uint64_t seed,
                                   uint64_t offset, const nvfp4_out* out, void* stream);

/* The amax pass and a 1x16 quantization with a per-tensor g in one call ([P2, results: amax and quantization
 * with no host round trip]).  The result equals nvfp4_amax (per tensor, use_rht = rounding is RHT_SR) followed by
 * nvfp4_quantize_rn / _sr / _rht_sr with the same arguments, and amax[0] is written too.
 *   A tensor that the chip can hold in registers is read from memory once: column-wise (cols % 4 == 0) up to two
 *   256-row x 256-column tiles per CU, row-wise up to 8192 blocks per CU (8192 x 4096 either way on MI355X).
 *   Each workgroup keeps its share in registers, publishes its maximum in a slot and waits for every other
 *   workgroup's; larger tensors run the two passes.
 *   For callers that cannot allocate (code under HIP graph capture, tight serving loops, harnesses that forbid
 *   hipMalloc): this call allocates nothing.  Its only scratch is the exchange slots, a 2 MiB array in the library's
 *   own device memory (one per GPU, held until the process ends; 8 regions of 16 copies of 2048 slots), whose
 *   address the library looks up on a device's first call; launches never need more, whatever the tensor size.
 *   Each launch tags its slots with a fresh 32-bit epoch and takes one of the 8 regions in turn.  Calls that overlap
 *   on one GPU (other streams, graph replays) may share a region: a workgroup never takes a slot that carries
 *   another launch's epoch, so sharing costs time, never correctness.  The wait is bounded: after 100 us with some
 *   workgroup of the launch not yet started (not all resident, e.g. CUs held by other work), or after 2 ms in any
 *   case, a waiting workgroup reads the tiles whose maxima it has not seen from the tensor itself, so the result
 *   never changes, only the time.
 *   rounding: NVFP4_ROUND_RN, _SR or _RHT_SR; sign_mask is used with RHT, seed and offset with SR.
 *   amax: [1] device float (output).  Shapes and outputs as for the quantize calls. */
nvfp4_status nvfp4_amax_quantize(const uint16_t* x, int64_t rows, int64_t cols, nvfp4_orient orient,
                                 nvfp4_rounding rounding, uint16_t sign_mask, uint64_t seed, uint64_t offset,
                                 float* amax, const nvfp4_out* out, void* stream);

/* Four-over-six quantization ([P3]): row-wise 1x16 blocks, round-to-nearest, no RHT.  g = fl(amax / (6 bound)).
 * Each block is encoded with T = 6 and with T = 4 (scale bamax / fl(4 g), 1.5x the map-to-6 scale); both are
 * decoded as fl(fl(val * decode(sb)) * g); their errors are measured by err_mode (nvfp4_4o6_error); map-to-4 is
 * kept only if its error is strictly smaller (ties and NaN keep 6).
 *   amax: [1] or [rows] from nvfp4_amax (row-wise, no RHT).  Shape: cols % 16 == 0.
 *   err_mode outside nvfp4_4o6_error or bound outside 1..448: NVFP4_ERR_UNSUPPORTED. */
nvfp4_status nvfp4_quantize_4o6(const uint16_t* x, int64_t rows, int64_t cols, nvfp4_gmode gmode,
                                nvfp4_4o6_error err_mode, int32_t bound, const float* amax, const nvfp4_out* out,
                                void* stream);

/* Four-over-six of a binary32 tensor ([P3]: the reference quantizer takes bf16 or fp32 inputs, and its sweep covers
 * both): nvfp4_quantize_4o6 with x [rows, cols] binary32 (16-byte aligned) in place of bf16; every step is the same,
 * on the binary32 values as given.  amax: [1] or [rows] from nvfp4_amax_f32. */
nvfp4_status nvfp4_quantize_4o6_f32(const float* x, int64_t rows, int64_t cols, nvfp4_gmode gmode,
                                    nvfp4_4o6_error err_mode, int32_t bound, const float* amax,
                                    const nvfp4_out* out, void* stream);

/* Row-wise amax of a binary32 tensor (no transform): the NaN-dominant maximum magnitude per tensor (amax[0]) or per
 * row (amax[rows]), for nvfp4_quantize_4o6_f32.  x [rows, cols] binary32, 16-byte aligned; cols % 16 == 0. */
nvfp4_status nvfp4_amax_f32(const float* x, int64_t rows, int64_t cols, nvfp4_gmode gmode, float* amax, void* stream);

/* Four-over-six with 16x16 tiles ([P3]: the reference quantizer takes 1x16 or 16x16 blocks; [P2, results]: weights
 * are quantized in both orientations).  One E4M3 scale per 16x16 tile of X from the tile's maximum; both candidates
 * (T = 6, 4) are formed as in nvfp4_quantize_4o6 with the tile maximum; the tile's error combines its rows' errors
 * (each row by err_mode over its 16 differences, then the 16 row errors the same way, row 0 first); map-to-4 is
 * kept only if strictly lower.  Per-tensor g = fl(amax / (6 bound)).
 *   orient NVFP4_ROWWISE writes W to *row_out: codes [rows, cols/2] packed along X's rows, scales [rows, cols/16]
 *   (each tile's scale repeated in its 16 rows), g [1]; NVFP4_COLWISE writes W^T to *col_out: codes [cols, rows/2]
 *   packed along X's columns, scales [cols, rows/16], g [1]; NVFP4_BOTH writes both from one read of X.
 *   amax: [1] from nvfp4_amax (row-wise, per tensor, no RHT).  Shape: rows % 16 == 0 and cols % 16 == 0.
 *   err_mode outside nvfp4_4o6_error, bound outside 1..448, or another orient: NVFP4_ERR_UNSUPPORTED. */
nvfp4_status nvfp4_quantize_4o6_16x16(const uint16_t* x, int64_t rows, int64_t cols, nvfp4_orient orient,
                                      nvfp4_4o6_error err_mode, int32_t bound, const float* amax,
                                      const nvfp4_out* row_out, const nvfp4_out* col_out, void* stream);

/* nvfp4_quantize_4o6_16x16 for a binary32 tensor ([P3]: bf16 or fp32 inputs): x [rows, cols] binary32, 16-byte
 * aligned; amax [1] from nvfp4_amax_f32 (per tensor).  Every step is the same, on the values as given. */
nvfp4_status nvfp4_quantize_4o6_16x16_f32(const float* x, int64_t rows, int64_t cols, nvfp4_orient orient,
                                          nvfp4_4o6_error err_mode, int32_t bound, const float* amax,
                                          const nvfp4_out* row_out, const nvfp4_out* col_out, void* stream);

/* Scale matrix to the tiled layout of the FP4 GEMM ([P2, approach]: the quantized operands reach the FP4 GEMM with
 * 1x16 block scales in the SWIZZLE_32_4_4 layout; [P2, results]: the swizzle is part of the per-call wrapper
 * overhead).  The scale matrix [rv, nb] (row-major, nb scales per row, as written by the quantize calls) is cut into
 * tiles of 128 rows x 4 scale columns, zero-padded to whole tiles; tile (R, B) is stored at byte
 * 512 * (R * ceil(nb/4) + B), and inside it byte 16 a + 4 b + c holds the scale of row 128 R + 32 b + a, column
 * 4 B + c (a [32][4][4] array; the layout of the 1D block-scaling factors in the cuBLAS documentation).
 *   scales: device, any alignment; out: device, 16-byte aligned, nvfp4_swizzled_scales_size(rv, nb) bytes, every
 *   byte written (padding = 0).  rv * nb < 2^31.  Errors: NVFP4_ERR_SHAPE, _NULL, _ALIGN; nothing is enqueued then. */
nvfp4_status nvfp4_swizzle_scales(const uint8_t* scales, int64_t rv, int64_t nb, uint8_t* out, void* stream);

/* Bytes of the tiled layout of an [rv, nb] scale matrix: ceil(rv/128) * 128 * ceil(nb/4) * 4 (0 for negative
 * sizes).  Host only; no GPU call. */
int64_t nvfp4_swizzled_scales_size(int64_t rv, int64_t nb);

/* Standard NVFP4 decode ([P3]: the recipe-agnostic decode): y = fl(fl(val(code) * decode(sb)) * g) as binary32.
 *   in: a quantization's outputs (device pointers, as written by the quantize calls): in->codes [rv, cv/2],
 *   in->scales [rv, cv/16] row-major (in->scale_layout NVFP4_SCALES_ROWMAJOR; the tiled layout returns
 *   NVFP4_ERR_UNSUPPORTED), in->g [1] or [rv] (gmode).  y [rv, cv] float (device).  Shape: cv % 16 == 0.
 *   Alignment as for the quantize calls' outputs (codes, scales 16 bytes, g 4) and y 16 bytes.  in is read on the
 *   host during the call only. */
nvfp4_status nvfp4_dequantize(const nvfp4_out* in, int64_t rv, int64_t cv, nvfp4_gmode gmode, float* y, void* stream);

/* Grouped calls ([P3]: grouped variants of the quantizer are named there as future kernel work): up to
 * NVFP4_MAX_GROUP row-wise tensors of any shapes, one launch for all of them.  items is a HOST array of count
 * descriptors (read during the call; the descriptors travel as kernel arguments, nothing is allocated).  The result
 * for item i is exactly that of the single-tensor call on it:
 *   nvfp4_amax_grouped     = nvfp4_amax(x, rows, cols, NVFP4_ROWWISE, gmode, use_rht, sign_mask, amax);
 *   nvfp4_quantize_grouped = nvfp4_quantize_rn / _sr / _rht_sr (row-wise, with the item's sign_mask, seed, offset)
 *                            or nvfp4_quantize_4o6 (rounding NVFP4_ROUND_4O6, with err_mode and bound; both are
 *                            ignored for the other roundings), reading the item's amax.
 *   Errors: count < 0 or > NVFP4_MAX_GROUP -> NVFP4_ERR_SHAPE; items NULL with count > 0 -> NVFP4_ERR_NULL; every
 *   item is checked as the single-tensor call would check it, and the first failing item's status is returned
 *   (nothing is enqueued then).  count == 0 is a no-op.  The tensors' buffers must not overlap one another. */
nvfp4_status nvfp4_amax_grouped(const nvfp4_group_item* items, int32_t count, nvfp4_gmode gmode, int use_rht,
                                void* stream);
nvfp4_status nvfp4_quantize_grouped(const nvfp4_group_item* items, int32_t count, nvfp4_gmode gmode,
                                    nvfp4_rounding rounding, nvfp4_4o6_error err_mode, int32_t bound,
                                    void* stream);

/* Fused decode ([P3]: an optimized decode is named there as future kernel work; [P1, random Hadamard transform]:
 * a block quantized after the rotation is brought back by the rotation's inverse, its transpose).  For each block of
 * 16 elements of a row: d_i = fl(fl(val(code_i) * decode(sb)) * g), as nvfp4_dequantize; with use_rht != 0, the
 * inverse of the transform of nvfp4_quantize_rht_sr with the same sign_mask: the butterfly with strides 1, 2, 4, 8,
 * (a, b) -> (a + b, a - b) in binary32, one multiply by 0.25, and element i negated where bit i of sign_mask is set.
 * The binary32 result is written as float (out_bf16 = 0) or as bf16 bit patterns (out_bf16 != 0) rounded to nearest
 * even, overflowing to infinity, with every NaN written as 0x7FC0.
 *   in: as for nvfp4_dequantize (row-major scales).  y [rv, cv] float or uint16, 16-byte aligned.
 *   Shape: cv % 16 == 0.  A column-wise quantization decodes to V = X^T. */
nvfp4_status nvfp4_dequantize_fused(const nvfp4_out* in, int64_t rv, int64_t cv, nvfp4_gmode gmode, int use_rht,
                                    uint16_t sign_mask, int out_bf16, void* y, void* stream);

/* Human-readable name of a status code (static storage). */
const char* nvfp4_status_str(nvfp4_status status);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
