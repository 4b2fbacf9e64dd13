// nvfp4_kernels.hip -- HIP kernels of the NVFP4 training quantizer for MI355X (gfx950, wave64).
//
// Pages cited (title, then section):
//   [P1] "在 RTX 5090 (SM120) 上补全 NVFP4 量化相关 kernel" -- blog post on polyfilling NVFP4 quantization kernels for
//        the RTX 5090 (harrychen.xyz, 2026-04-14).
//   [P2] "nvfp4-sm120" repository README.
//   [P3] pytorch/ao pull request #4852, "Add a CuTe DSL fast-path kernel for four-over-six quantize".
//   Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11.
//
// Design (MI355X-first):
//   * The op is O(|X|) and HBM-bound ([P1, random Hadamard transform]: not a real GEMM).  A 16-point transform is
//     far too narrow for MFMA, so the Hadamard product is an in-register butterfly; nothing is staged in LDS.
//   * Every lane owns whole 16-element blocks, so block maxima, scales, Philox and packing need no cross-lane
//     traffic.  Row-wise: a lane loads one block (two 16-byte loads).  Column-wise (blocks run down columns of X):
//     a lane loads 16 rows x 8 columns with 16 coalesced 16-byte loads and transposes in registers, which yields 8
//     complete column blocks; the 4 waves of a workgroup are stacked along rows so each output row of X^T receives
//     a contiguous multi-line run from one CU.
//   * Bit-exact rounding: every step is one IEEE binary32 operation (built with -ffp-contract=off, no fast-math,
//     denormals kept); the divisions are HIP's correctly rounded ones.  E2M1/E4M3 encodes are integer
//     manipulations of the binary32 pattern that reproduce round-to-nearest-even / the SR rule exactly.
//   * No host synchronisation: the global scale is computed on the device from the amax buffer ([P2, results]).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_launch.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr float kFltMax = 3.402823466e38f;

__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// ------------------------------------------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC'11).  Multipliers and Weyl increments are the published constants.  The key
// is uniform across the launch, so its schedule lives in scalar registers.
// ------------------------------------------------------------------------------------------------------------
constexpr uint32_t kPhiloxMulA = 0xD2511F53u;  // multiplies counter word 0
constexpr uint32_t kPhiloxMulB = 0xCD9E8D57u;  // multiplies counter word 2
constexpr uint32_t kPhiloxWeylA = 0x9E3779B9u;
constexpr uint32_t kPhiloxWeylB = 0xBB67AE85u;

struct Rand4 {
    uint32_t w[4];
};

__device__ __forceinline__ Rand4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                               uint32_t k1) {
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint64_t pa = (uint64_t)kPhiloxMulA * c0;
        const uint64_t pb = (uint64_t)kPhiloxMulB * c2;
        const uint32_t n0 = (uint32_t)(pb >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(pa >> 32) ^ c3 ^ k1;
        c1 = (uint32_t)pb;
        c3 = (uint32_t)pa;
        c0 = n0;
        c2 = n2;
        k0 += kPhiloxWeylA;
        k1 += kPhiloxWeylB;
    }
    return Rand4{{c0, c1, c2, c3}};
}

// Random bytes of the 1x16 block with row-major index n in the quantized view ([P1, vibe-coding and timeline
// sections]: the counter layout is part of the semantics): key = seed, counter = (n, offset) as 32-bit words.
struct RngArgs {
    uint32_t k0, k1, o0, o1;
};

__device__ __forceinline__ Rand4 block_rand(const RngArgs& a, uint64_t n) {
    return philox4x32_10((uint32_t)n, (uint32_t)(n >> 32), a.o0, a.o1, a.k0, a.k1);
}

// ------------------------------------------------------------------------------------------------------------
// E4M3 ("fn") block scale.  [P2, layout]: E4M3 per-block scale over an FP32 global scale.  Round to nearest even,
// saturate above 448 (the "satfinite" convention of the conversions in [P1]), NaN -> 0x7F, s <= 0 -> 0.
// ------------------------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
    if (s != s) return 0x7Fu;
    if (!(s > 0.0f)) return 0u;
    if (s > 448.0f) return 0x7Eu;
    const uint32_t b = as_u(s);
    if (b >= 0x3C800000u) {                             // s >= 2^-6: normal; round 23 mantissa bits to 3 (RNE)
        const uint32_t u = b + 0x7FFFFu + ((b >> 20) & 1u);
        return (u >> 20) - 960u;                        // ((e - 127 + 7) << 3) | m
    }
    return (uint32_t)__builtin_rintf(s * 512.0f);      // subnormal range: a multiple of 2^-9 (8 = min normal)
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {  // c in [0, 0x7F]
    if (c == 0x7Fu) return __builtin_nanf("");
    const uint32_t e = c >> 3, m = c & 7u;
    if (e == 0) return (float)m * 0.001953125f;         // m * 2^-9, exact
    return as_f(((e + 120u) << 23) | (m << 20));
}

// Block scale and element multiplier: s = bamax / d (d = fl(T g)), sb = E4M3(s), S = fl(decode(sb) g),
// r = fl(1 / S) with r = 0 for S = 0, NaN for NaN S, FLT_MAX when the reciprocal overflows.
struct BlockScale {
    uint32_t sb;
    float r;
};

__device__ __forceinline__ BlockScale block_scale(float bamax, float d, float g) {
    const float s = (bamax == 0.0f) ? 0.0f : bamax / d;
    const uint32_t sb = e4m3_encode(s);
    const float S = e4m3_decode(sb) * g;
    float r;
    if (S != S) {
        r = S;
    } else if (S == 0.0f) {
        r = 0.0f;
    } else {
        r = 1.0f / S;
        if (__builtin_isinf(r)) r = kFltMax;
    }
    return BlockScale{sb, r};
}

// ------------------------------------------------------------------------------------------------------------
// E2M1 magnitude index (0..7 for 0, 0.5, 1, 1.5, 2, 3, 4, 6; [P1, FP4 quantization techniques]) of t >= 0.
// t is clamped to 6 first (satfinite); NaN must be handled by the caller (fminf drops it).
//   t >= 1: d = bits(t) - bits(0.5) puts the E2M1 exponent/mantissa pair in bits 22..24 (value index 2..7);
//           the 22 bits below are the fraction of the way to the next grid point.
//   t <  1: the grid is uniform with step 0.5.
// ------------------------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e2m1_rn_mag(float t) {
    t = __builtin_fminf(t, 6.0f);
    const uint32_t d = as_u(t) - 0x3F000000u;
    const uint32_t hi = (d + 0x1FFFFFu + ((d >> 22) & 1u)) >> 22;   // round to nearest, ties to even
    const uint32_t lo = (uint32_t)__builtin_rintf(t + t);           // 2t rounded to nearest even: 0, 1, 2
    return ((int32_t)d < 0x800000) ? lo : hi;
}

// Stochastic rounding ([P1, stochastic rounding]): up iff rho < floor(256 * frac).  rinv = (255 - rho) << 14;
// adding it to the 22 fraction bits carries into bit 22 exactly when frac's top 8 bits exceed rho.
// For t < 1, floor(t * 2^23) has the same layout (step 0.5 = 2^22 units).
__device__ __forceinline__ uint32_t e2m1_sr_mag(float t, uint32_t rinv) {
    t = __builtin_fminf(t, 6.0f);
    const uint32_t d = as_u(t) - 0x3F000000u;
    const uint32_t lo = (uint32_t)(t * 8388608.0f);
    return ((((int32_t)d < 0x800000) ? lo : d) + rinv) >> 22;
}

template <bool SR>
__device__ __forceinline__ uint32_t e2m1_code_fast(float y, float r, uint32_t rinv) {
    // valid for finite r > 0: q = y r has the sign of y and is NaN only if y is, which cannot happen here
    // (a NaN in the block makes its scale NaN)
    const float t = __builtin_fabsf(y) * r;
    const uint32_t m = SR ? e2m1_sr_mag(t, rinv) : e2m1_rn_mag(t);
    return m | ((as_u(y) >> 28) & 8u);
}

template <bool SR>
__device__ __forceinline__ uint32_t e2m1_code_general(float y, float r, uint32_t rinv) {
    const float q = y * r;
    if (q != q) return 7u;
    const float t = __builtin_fabsf(q);
    const uint32_t m = SR ? e2m1_sr_mag(t, rinv) : e2m1_rn_mag(t);
    return m | ((as_u(q) >> 28) & 8u);
}

__device__ __forceinline__ uint32_t rinv_of(const Rand4& rnd, int i) {
    return ((~rnd.w[i >> 2] >> (8 * (i & 3))) & 0xFFu) << 14;
}

// Quantize 16 binary32 values: block amax (integer max of magnitude bits, NaN dominant), scale, E2M1 codes
// packed 8 per dword with element 2k in the low nibble of byte k.
template <bool SR>
__device__ __forceinline__ void quantize16(const float (&y)[16], float d6, float g, const Rand4& rnd, uint32_t& lo,
                                           uint32_t& hi, uint32_t& sb) {
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = umax(mx, as_u(y[i]) & 0x7FFFFFFFu);
    const BlockScale sc = block_scale(as_f(mx), d6, g);
    sb = sc.sb;
    uint32_t c0 = 0, c1 = 0;
    if (sc.r > 0.0f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) c0 |= e2m1_code_fast<SR>(y[i], sc.r, SR ? rinv_of(rnd, i) : 0u) << (4 * i);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            c1 |= e2m1_code_fast<SR>(y[8 + i], sc.r, SR ? rinv_of(rnd, 8 + i) : 0u) << (4 * i);
    } else {  // r is 0, negative or NaN (degenerate amax or NaN block)
#pragma unroll
        for (int i = 0; i < 8; ++i) c0 |= e2m1_code_general<SR>(y[i], sc.r, SR ? rinv_of(rnd, i) : 0u) << (4 * i);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            c1 |= e2m1_code_general<SR>(y[8 + i], sc.r, SR ? rinv_of(rnd, 8 + i) : 0u) << (4 * i);
    }
    lo = c0;
    hi = c1;
}

// ------------------------------------------------------------------------------------------------------------
// 16-point Random Hadamard Transform ([P1, random Hadamard transform]): y = (1/4) H16 diag(s) v with the
// Sylvester H16, evaluated as the butterfly with strides 1, 2, 4, 8 ((a, b) -> (a + b, a - b)), then a multiply
// by 0.25.  The random signs are applied by the caller on the packed bf16 words (an exact sign-bit flip).
// ------------------------------------------------------------------------------------------------------------
__device__ __forceinline__ void fwht16(float (&w)[16]) {
#pragma unroll
    for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if ((i & h) == 0) {
                const float a = w[i], b = w[i + h];
                w[i] = a + b;
                w[i + h] = a - b;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = 0.25f * w[i];
}

// XOR patterns that flip the bf16 sign bits of elements (2k, 2k+1) held in packed word k of a row-wise block.
__device__ __forceinline__ uint32_t sign_word(uint32_t mask, int k) {
    return (((mask >> (2 * k)) & 1u) << 15) | (((mask >> (2 * k + 1)) & 1u) << 31);
}

// 16-byte load of 8 bf16 values (the address is 16-byte aligned by the shape rules).
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return as_f(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return as_f(w & 0xFFFF0000u); }

// n / d for 32-bit n with a precomputed multiplier (Granlund-Montgomery "round-up" method).
struct FastDiv {
    uint32_t d, m, s;
};

FastDiv make_fastdiv(uint32_t d) {
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    const uint64_t m = ((((1ull << s) - d) << 32) / d) + 1;
    return FastDiv{d, (uint32_t)m, s};
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
    return (uint32_t)(((uint64_t)__umulhi(n, f.m) + n) >> f.s);
}

__device__ __forceinline__ float global_scale(float amax) { return amax / 2688.0f; }

// ------------------------------------------------------------------------------------------------------------
// Row-wise 1x16 quantization: one block (32 bytes of bf16) per lane per iteration, grid-stride.
// ------------------------------------------------------------------------------------------------------------
template <int MODE, bool PER_ROW>
__global__ void __launch_bounds__(kThreads)
k_quant_rowwise(const uint4* __restrict__ x, uint32_t total_blocks, FastDiv per_row, const float* __restrict__ amax,
                uint32_t sign_mask, RngArgs rng, uint2* __restrict__ codes, uint8_t* __restrict__ scales,
                float* __restrict__ gout) {
    constexpr bool SR = MODE != kRN;
    float g = 0.0f, d6 = 0.0f;
    if (!PER_ROW) {
        g = global_scale(amax[0]);
        d6 = 6.0f * g;
        if (blockIdx.x == 0 && threadIdx.x == 0) gout[0] = g;
    }
    const uint32_t stride = gridDim.x * kThreads;
    for (uint32_t n = blockIdx.x * kThreads + threadIdx.x; n < total_blocks; n += stride) {
        if (PER_ROW) {
            const uint32_t row = fdiv(n, per_row);
            g = global_scale(amax[row]);
            d6 = 6.0f * g;
            if (n == row * per_row.d) gout[row] = g;
        }
        uint4 a = ld16(x + 2 * (size_t)n);
        uint4 b = ld16(x + 2 * (size_t)n + 1);
        if (MODE == kRHTSR) {
            a.x ^= sign_word(sign_mask, 0);
            a.y ^= sign_word(sign_mask, 1);
            a.z ^= sign_word(sign_mask, 2);
            a.w ^= sign_word(sign_mask, 3);
            b.x ^= sign_word(sign_mask, 4);
            b.y ^= sign_word(sign_mask, 5);
            b.z ^= sign_word(sign_mask, 6);
            b.w ^= sign_word(sign_mask, 7);
        }
        float y[16] = {bf16_lo(a.x), bf16_hi(a.x), bf16_lo(a.y), bf16_hi(a.y), bf16_lo(a.z), bf16_hi(a.z),
                       bf16_lo(a.w), bf16_hi(a.w), bf16_lo(b.x), bf16_hi(b.x), bf16_lo(b.y), bf16_hi(b.y),
                       bf16_lo(b.z), bf16_hi(b.z), bf16_lo(b.w), bf16_hi(b.w)};
        if (MODE == kRHTSR) fwht16(y);
        Rand4 rnd{{0, 0, 0, 0}};
        if (SR) rnd = block_rand(rng, n);
        uint32_t lo, hi, sb;
        quantize16<SR>(y, d6, g, rnd, lo, hi, sb);
        codes[n] = make_uint2(lo, hi);
        scales[n] = (uint8_t)sb;
    }
}

// ------------------------------------------------------------------------------------------------------------
// Column-wise 1x16 quantization (V = X^T; a block is 16 consecutive rows of one column of X).
// Lane (rb, cg) of a wave owns row-block rb (16 rows) and column group cg (8 columns): 16 loads of 16 bytes,
// 8 complete blocks.  RBW row-blocks x (64 / RBW) column groups per wave; the 4 waves of a workgroup are stacked
// along rows, so a workgroup covers 4*RBW row-blocks x 8*(64/RBW) columns.
// ------------------------------------------------------------------------------------------------------------
template <int MODE, bool PER_ROW, int RBW>
__global__ void __launch_bounds__(kThreads)
k_quant_colwise(const uint16_t* __restrict__ x, uint32_t rows, uint32_t cols, uint32_t col_tiles,
                uint32_t total_tiles, const float* __restrict__ amax, uint32_t sign_mask, RngArgs rng,
                uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gout) {
    constexpr bool SR = MODE != kRN;
    constexpr int CGW = 64 / RBW;                 // column groups per wave
    constexpr int TILE_COLS = 8 * CGW;
    constexpr int TILE_RB = 4 * RBW;              // row-blocks per workgroup tile
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t rbl = lane % RBW, cgl = lane / RBW;
    const uint32_t nrb = rows >> 4;               // blocks per row of V
    float g = 0.0f, d6 = 0.0f;
    if (!PER_ROW) {
        g = global_scale(amax[0]);
        d6 = 6.0f * g;
        if (blockIdx.x == 0 && threadIdx.x == 0) gout[0] = g;
    }
    for (uint32_t t = blockIdx.x; t < total_tiles; t += gridDim.x) {
        const uint32_t tr = t / col_tiles, tc = t - tr * col_tiles;
        const uint32_t rb = tr * TILE_RB + wave * RBW + rbl;
        const uint32_t c8 = (tc * TILE_COLS) + 8 * cgl;
        if (rb >= nrb || c8 >= cols) continue;
        const uint16_t* src = x + (size_t)(16 * rb) * cols + c8;
        uint4 v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = ld16(src + (size_t)k * cols);
        if (MODE == kRHTSR) {
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const uint32_t f = ((sign_mask >> k) & 1u) ? 0x80008000u : 0u;
                v[k].x ^= f;
                v[k].y ^= f;
                v[k].z ^= f;
                v[k].w ^= f;
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t c = c8 + j;
            float y[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const uint32_t w = (j >> 1) == 0 ? v[k].x : (j >> 1) == 1 ? v[k].y : (j >> 1) == 2 ? v[k].z : v[k].w;
                y[k] = (j & 1) ? bf16_hi(w) : bf16_lo(w);
            }
            if (MODE == kRHTSR) fwht16(y);
            if (PER_ROW) {
                g = global_scale(amax[c]);
                d6 = 6.0f * g;
                if (rb == 0) gout[c] = g;
            }
            const uint64_t n = (uint64_t)c * nrb + rb;
            Rand4 rnd{{0, 0, 0, 0}};
            if (SR) rnd = block_rand(rng, n);
            uint32_t lo, hi, sb;
            quantize16<SR>(y, d6, g, rnd, lo, hi, sb);
            *reinterpret_cast<uint2*>(codes + (size_t)c * (rows >> 1) + 8 * (size_t)rb) = make_uint2(lo, hi);
            scales[(size_t)c * nrb + rb] = (uint8_t)sb;
        }
    }
}

// ------------------------------------------------------------------------------------------------------------
// 16x16 RN quantization, W and/or W^T from one read ([P2, intro: 2D weight scaling; results: both weight
// orientations]).  Lane pair (2m, 2m+1) owns tile column tj (columns 16 tj + 8h .. +7 for half h); each lane
// loads 16 rows x 16 bytes; the tile amax is the max over the pair.  Waves of a workgroup are stacked along tile
// rows, each wave loops over TR tile rows.
// ------------------------------------------------------------------------------------------------------------
template <bool WANT_W, bool WANT_WT, int TR>
__global__ void __launch_bounds__(kThreads)
k_quant_16x16(const uint16_t* __restrict__ x, uint32_t rows, uint32_t cols, uint32_t col_groups,
              uint32_t total_groups, const float* __restrict__ amax, uint8_t* __restrict__ cw,
              uint8_t* __restrict__ sw, float* __restrict__ gw, uint8_t* __restrict__ ct, uint8_t* __restrict__ st,
              float* __restrict__ gt) {
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t h = lane & 1u;
    const uint32_t ntr = rows >> 4, ntc = cols >> 4;
    const float g = global_scale(amax[0]);
    const float d6 = 6.0f * g;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (WANT_W) gw[0] = g;
        if (WANT_WT) gt[0] = g;
    }
    for (uint32_t grp = blockIdx.x; grp < total_groups; grp += gridDim.x) {
        const uint32_t gr = grp / col_groups, gc = grp - gr * col_groups;
        const uint32_t tj = gc * 32 + (lane >> 1);
        const bool col_ok = tj < ntc;
        for (int it = 0; it < TR; ++it) {
            const uint32_t ti = (gr * 4 + wave) * TR + it;
            // both lanes of a pair share ti and tj, so the pair is active or idle together (needed by the shuffle)
            const bool ok = col_ok && ti < ntr;
            uint4 v[16];
            uint32_t m16 = 0;  // integer max of the bf16 magnitude bits of this half tile
            if (ok) {
                const uint16_t* src = x + (size_t)(16 * ti) * cols + 16 * tj + 8 * h;
#pragma unroll
                for (int k = 0; k < 16; ++k) v[k] = ld16(src + (size_t)k * cols);
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const uint32_t ws[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) m16 = umax(m16, umax(ws[q] & 0x7FFFu, (ws[q] >> 16) & 0x7FFFu));
                }
            }
            m16 = umax(m16, (uint32_t)__shfl_xor((int)m16, 1));
            if (!ok) continue;
            const BlockScale sc = block_scale(as_f(m16 << 16), d6, g);
            uint32_t wt[8][2];
#pragma unroll
            for (int j = 0; j < 8; ++j) wt[j][0] = wt[j][1] = 0;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const uint32_t ws[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
                uint32_t rowc = 0;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float y = (j & 1) ? bf16_hi(ws[j >> 1]) : bf16_lo(ws[j >> 1]);
                    const uint32_t code = sc.r > 0.0f ? e2m1_code_fast<false>(y, sc.r, 0u)
                                                      : e2m1_code_general<false>(y, sc.r, 0u);
                    rowc |= code << (4 * j);
                    wt[j][k >> 3] |= code << (4 * (k & 7));
                }
                if (WANT_W)
                    *reinterpret_cast<uint32_t*>(cw + (size_t)(16 * ti + k) * (cols >> 1) + 8 * tj + 4 * h) = rowc;
            }
            if (WANT_W) {
#pragma unroll
                for (int k = 0; k < 8; ++k) sw[(size_t)(16 * ti + 8 * h + k) * ntc + tj] = (uint8_t)sc.sb;
            }
            if (WANT_WT) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t c = 16 * tj + 8 * h + j;
                    *reinterpret_cast<uint2*>(ct + (size_t)c * (rows >> 1) + 8 * ti) = make_uint2(wt[j][0], wt[j][1]);
                    st[(size_t)c * ntr + ti] = (uint8_t)sc.sb;
                }
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------------------
// Four-over-six ([P3]): row-wise 1x16 RN; candidates T = 6 and T = 4; decode, squared errors, pinned tree sum
// (i, i+8), then strides 4, 2, 1; map-to-4 kept only if strictly lower.
// ------------------------------------------------------------------------------------------------------------
__device__ __forceinline__ float e2m1_value(uint32_t code) {
    const uint32_t m = code & 7u;
    // m >= 2: exponent field (m >> 1) + 126 and mantissa bit m & 1, i.e. (m + 252) << 22; m = 1 is 0.5
    const uint32_t mag = m >= 2u ? ((m + 252u) << 22) : (m == 1u ? 0x3F000000u : 0u);
    return as_f(mag | ((code & 8u) << 28));
}

template <bool PER_ROW>
__global__ void __launch_bounds__(kThreads)
k_quant_4o6(const uint4* __restrict__ x, uint32_t total_blocks, FastDiv per_row, const float* __restrict__ amax,
            uint2* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gout) {
    float g = 0.0f;
    if (!PER_ROW) {
        g = global_scale(amax[0]);
        if (blockIdx.x == 0 && threadIdx.x == 0) gout[0] = g;
    }
    const uint32_t stride = gridDim.x * kThreads;
    for (uint32_t n = blockIdx.x * kThreads + threadIdx.x; n < total_blocks; n += stride) {
        if (PER_ROW) {
            const uint32_t row = fdiv(n, per_row);
            g = global_scale(amax[row]);
            if (n == row * per_row.d) gout[row] = g;
        }
        const uint4 a = ld16(x + 2 * (size_t)n);
        const uint4 b = ld16(x + 2 * (size_t)n + 1);
        const float xv[16] = {bf16_lo(a.x), bf16_hi(a.x), bf16_lo(a.y), bf16_hi(a.y), bf16_lo(a.z), bf16_hi(a.z),
                              bf16_lo(a.w), bf16_hi(a.w), bf16_lo(b.x), bf16_hi(b.x), bf16_lo(b.y), bf16_hi(b.y),
                              bf16_lo(b.z), bf16_hi(b.z), bf16_lo(b.w), bf16_hi(b.w)};
        uint32_t mx = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = umax(mx, as_u(xv[i]) & 0x7FFFFFFFu);
        const float bamax = as_f(mx);
        uint32_t cand_lo[2], cand_hi[2], cand_sb[2];
        float err[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const float d = (c == 0 ? 6.0f : 4.0f) * g;
            const BlockScale sc = block_scale(bamax, d, g);
            const float sbf = e4m3_decode(sc.sb);
            float e[16];
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t code = sc.r > 0.0f ? e2m1_code_fast<false>(xv[i], sc.r, 0u)
                                                  : e2m1_code_general<false>(xv[i], sc.r, 0u);
                if (i < 8) lo |= code << (4 * i);
                else hi |= code << (4 * (i - 8));
                const float xh = (e2m1_value(code) * sbf) * g;
                const float df = xh - xv[i];
                e[i] = df * df;
            }
#pragma unroll
            for (int s = 8; s >= 1; s >>= 1)
#pragma unroll
                for (int i = 0; i < s; ++i) e[i] = e[i] + e[i + s];
            cand_lo[c] = lo;
            cand_hi[c] = hi;
            cand_sb[c] = sc.sb;
            err[c] = e[0];
        }
        const int pick = (err[1] < err[0]) ? 1 : 0;
        codes[n] = make_uint2(cand_lo[pick], cand_hi[pick]);
        scales[n] = (uint8_t)cand_sb[pick];
    }
}

// ------------------------------------------------------------------------------------------------------------
// Standard NVFP4 decode ([P3]): y = fl(fl(val(code) * decode(sb)) * g); one 16-element block per lane.
// ------------------------------------------------------------------------------------------------------------
template <bool PER_ROW>
__global__ void __launch_bounds__(kThreads)
k_dequantize(const uint2* __restrict__ codes, const uint8_t* __restrict__ scales, const float* __restrict__ g,
             uint32_t total_blocks, FastDiv per_row, float4* __restrict__ y) {
    const uint32_t stride = gridDim.x * kThreads;
    for (uint32_t n = blockIdx.x * kThreads + threadIdx.x; n < total_blocks; n += stride) {
        const float gr = PER_ROW ? g[fdiv(n, per_row)] : g[0];
        const float sbf = e4m3_decode(scales[n] & 0x7Fu) ;
        const float sbf_signed = (scales[n] & 0x80u) ? -sbf : sbf;
        const uint2 c = codes[n];
        float out[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t code = ((i < 8 ? c.x : c.y) >> (4 * (i & 7))) & 0xFu;
            out[i] = (e2m1_value(code) * sbf_signed) * gr;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            y[4 * (size_t)n + q] = make_float4(out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]);
    }
}

// ------------------------------------------------------------------------------------------------------------
// amax kernels.  The maximum is an integer maximum over magnitude bit patterns (NaN > inf > finite).
// ------------------------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = umax(v, (uint32_t)__shfl_xor((int)v, off));
    return v;
}

__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* lds) {
    v = wave_max(v);
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    if (lane == 0) lds[wave] = v;
    __syncthreads();
    uint32_t r = 0;
    if (threadIdx.x == 0) {
        for (int w = 0; w < kThreads / 64; ++w) r = umax(r, lds[w]);
    }
    __syncthreads();
    return r;  // valid in thread 0
}

__global__ void k_fill_zero(uint32_t* __restrict__ p, uint32_t n) {
    for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < n; i += gridDim.x * kThreads) p[i] = 0u;
}

// g = amax / 2688 for n entries (used when the tensor to quantize is empty, so no block writes g).
__global__ void k_write_g(const float* __restrict__ amax, float* __restrict__ g, uint32_t n) {
    for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < n; i += gridDim.x * kThreads) g[i] = global_scale(amax[i]);
}

// Max magnitude bits of one row-wise block (optionally transformed).
template <bool RHT>
__device__ __forceinline__ uint32_t block_absmax_rowwise(const uint4* x, size_t n, uint32_t sign_mask) {
    uint4 a = ld16(x + 2 * n);
    uint4 b = ld16(x + 2 * n + 1);
    if (!RHT) {
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint32_t m = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) m = umax(m, umax(w[q] & 0x7FFFu, (w[q] >> 16) & 0x7FFFu));
        return m << 16;
    }
    a.x ^= sign_word(sign_mask, 0);
    a.y ^= sign_word(sign_mask, 1);
    a.z ^= sign_word(sign_mask, 2);
    a.w ^= sign_word(sign_mask, 3);
    b.x ^= sign_word(sign_mask, 4);
    b.y ^= sign_word(sign_mask, 5);
    b.z ^= sign_word(sign_mask, 6);
    b.w ^= sign_word(sign_mask, 7);
    float y[16] = {bf16_lo(a.x), bf16_hi(a.x), bf16_lo(a.y), bf16_hi(a.y), bf16_lo(a.z), bf16_hi(a.z),
                   bf16_lo(a.w), bf16_hi(a.w), bf16_lo(b.x), bf16_hi(b.x), bf16_lo(b.y), bf16_hi(b.y),
                   bf16_lo(b.z), bf16_hi(b.z), bf16_lo(b.w), bf16_hi(b.w)};
    fwht16(y);
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = umax(m, as_u(y[i]) & 0x7FFFFFFFu);
    return m;
}

// Row-wise, per tensor: grid-stride over blocks, one atomic max per workgroup into a zeroed amax[0].
template <bool RHT>
__global__ void __launch_bounds__(kThreads)
k_amax_rowwise_tensor(const uint4* __restrict__ x, uint32_t total_blocks, uint32_t sign_mask, uint32_t* amax_bits) {
    __shared__ uint32_t lds[kThreads / 64];
    uint32_t m = 0;
    for (uint32_t n = blockIdx.x * kThreads + threadIdx.x; n < total_blocks; n += gridDim.x * kThreads)
        m = umax(m, block_absmax_rowwise<RHT>(x, n, sign_mask));
    m = block_max(m, lds);
    if (threadIdx.x == 0) atomicMax(amax_bits, m);
}

// Row-wise, per row: one workgroup per row (grid-stride over rows), direct store.
template <bool RHT>
__global__ void __launch_bounds__(kThreads)
k_amax_rowwise_rows(const uint4* __restrict__ x, uint32_t rows, uint32_t blocks_per_row, uint32_t sign_mask,
                    uint32_t* __restrict__ amax_bits) {
    __shared__ uint32_t lds[kThreads / 64];
    for (uint32_t r = blockIdx.x; r < rows; r += gridDim.x) {
        uint32_t m = 0;
        for (uint32_t b = threadIdx.x; b < blocks_per_row; b += kThreads)
            m = umax(m, block_absmax_rowwise<RHT>(x, (size_t)r * blocks_per_row + b, sign_mask));
        m = block_max(m, lds);
        if (threadIdx.x == 0) amax_bits[r] = m;
    }
}

// Column-wise (V = X^T): same lane tiling as k_quant_colwise.  Per tensor: one atomic per workgroup; per row of V
// (= per column of X): lanes sharing a column group reduce over row-blocks, then one atomic per column per wave.
template <bool RHT, bool PER_ROW, int RBW>
__global__ void __launch_bounds__(kThreads)
k_amax_colwise(const uint16_t* __restrict__ x, uint32_t rows, uint32_t cols, uint32_t col_tiles,
               uint32_t total_tiles, uint32_t sign_mask, uint32_t* __restrict__ amax_bits) {
    constexpr int CGW = 64 / RBW;
    constexpr int TILE_COLS = 8 * CGW;
    constexpr int TILE_RB = 4 * RBW;
    __shared__ uint32_t lds[kThreads / 64];
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t rbl = lane % RBW, cgl = lane / RBW;
    const uint32_t nrb = rows >> 4;
    uint32_t total = 0;
    for (uint32_t t = blockIdx.x; t < total_tiles; t += gridDim.x) {
        const uint32_t tr = t / col_tiles, tc = t - tr * col_tiles;
        const uint32_t rb = tr * TILE_RB + wave * RBW + rbl;
        const uint32_t c8 = tc * TILE_COLS + 8 * cgl;
        const bool ok = rb < nrb && c8 < cols;
        uint32_t colmax[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (ok) {
            const uint16_t* src = x + (size_t)(16 * rb) * cols + c8;
            uint4 v[16];
#pragma unroll
            for (int k = 0; k < 16; ++k)
                v[k] = ld16(src + (size_t)k * cols);
            if (!RHT) {
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const uint32_t ws[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        colmax[j] = umax(colmax[j], ((j & 1) ? (ws[j >> 1] >> 16) : ws[j >> 1]) & 0x7FFFu);
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) colmax[j] <<= 16;
            } else {
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const uint32_t f = ((sign_mask >> k) & 1u) ? 0x80008000u : 0u;
                    v[k].x ^= f;
                    v[k].y ^= f;
                    v[k].z ^= f;
                    v[k].w ^= f;
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    float y[16];
#pragma unroll
                    for (int k = 0; k < 16; ++k) {
                        const uint32_t w =
                            (j >> 1) == 0 ? v[k].x : (j >> 1) == 1 ? v[k].y : (j >> 1) == 2 ? v[k].z : v[k].w;
                        y[k] = (j & 1) ? bf16_hi(w) : bf16_lo(w);
                    }
                    fwht16(y);
#pragma unroll
                    for (int k = 0; k < 16; ++k) colmax[j] = umax(colmax[j], as_u(y[k]) & 0x7FFFFFFFu);
                }
            }
        }
        if (PER_ROW) {
            // lanes with the same cgl are RBW consecutive lanes: reduce over rbl with xor offsets < RBW
#pragma unroll
            for (int j = 0; j < 8; ++j) {
#pragma unroll
                for (int off = RBW / 2; off >= 1; off >>= 1)
                    colmax[j] = umax(colmax[j], (uint32_t)__shfl_xor((int)colmax[j], off));
            }
            if (rbl == 0 && c8 < cols) {
#pragma unroll
                for (int j = 0; j < 8; ++j) atomicMax(amax_bits + c8 + j, colmax[j]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) total = umax(total, colmax[j]);
        }
    }
    if (!PER_ROW) {
        total = block_max(total, lds);
        if (threadIdx.x == 0) atomicMax(amax_bits, total);
    }
}

// ------------------------------------------------------------------------------------------------------------
// Launch helpers
// ------------------------------------------------------------------------------------------------------------
int cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

uint32_t grid_for(uint64_t work_items, uint32_t per_group, uint32_t groups_per_cu) {
    const uint64_t need = (work_items + per_group - 1) / per_group;
    const uint64_t cap = (uint64_t)cu_count() * groups_per_cu;
    const uint64_t g = need < cap ? need : cap;
    return (uint32_t)(g == 0 ? 1 : g);
}

RngArgs rng_args(Philox p) {
    return RngArgs{(uint32_t)p.seed, (uint32_t)(p.seed >> 32), (uint32_t)p.offset, (uint32_t)(p.offset >> 32)};
}

constexpr int kColRBW = 8;  // row-blocks per wave in the column-wise kernels

hipError_t write_empty_g(const float* amax, float* g, uint32_t n, hipStream_t stream) {
    if (n) k_write_g<<<grid_for(n, kThreads, 1), kThreads, 0, stream>>>(amax, g, n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_amax(const uint16_t* x, int64_t rows, int64_t cols, bool colwise, bool per_row, bool use_rht,
                       uint32_t sign_mask, float* amax, hipStream_t stream) {
    uint32_t* bits = reinterpret_cast<uint32_t*>(amax);
    const int64_t rv = colwise ? cols : rows;
    const bool atomic = !per_row || colwise;
    if (atomic || rows == 0 || cols == 0) {
        const uint32_t n = per_row ? (uint32_t)rv : 1u;
        if (n) k_fill_zero<<<grid_for(n, kThreads, 1), kThreads, 0, stream>>>(bits, n);
    }
    if (rows == 0 || cols == 0) return hipGetLastError();
    if (!colwise) {
        const uint32_t bpr = (uint32_t)(cols / 16);
        const uint32_t total = (uint32_t)(rows * bpr);
        if (per_row) {
            const uint32_t grid = (uint32_t)(rows < 65536 * 16 ? rows : 65536 * 16);
            if (use_rht)
                k_amax_rowwise_rows<true><<<grid, kThreads, 0, stream>>>(reinterpret_cast<const uint4*>(x),
                                                                           (uint32_t)rows, bpr, sign_mask, bits);
            else
                k_amax_rowwise_rows<false><<<grid, kThreads, 0, stream>>>(reinterpret_cast<const uint4*>(x),
                                                                            (uint32_t)rows, bpr, sign_mask, bits);
        } else {
            const uint32_t grid = grid_for(total, kThreads * 4, 8);
            if (use_rht)
                k_amax_rowwise_tensor<true><<<grid, kThreads, 0, stream>>>(reinterpret_cast<const uint4*>(x), total,
                                                                             sign_mask, bits);
            else
                k_amax_rowwise_tensor<false><<<grid, kThreads, 0, stream>>>(reinterpret_cast<const uint4*>(x),
                                                                              total, sign_mask, bits);
        }
    } else {
        constexpr int RBW = kColRBW;
        const uint32_t tile_cols = 8 * (64 / RBW), tile_rb = 4 * RBW;
        const uint32_t col_tiles = (uint32_t)((cols + tile_cols - 1) / tile_cols);
        const uint32_t row_tiles = (uint32_t)((rows / 16 + tile_rb - 1) / tile_rb);
        const uint32_t total = col_tiles * row_tiles;
        const uint32_t grid = grid_for(total, 1, 8);
#define NVFP4_AMAX_COL(R, P)                                                                                     \
    k_amax_colwise<R, P, RBW><<<grid, kThreads, 0, stream>>>(x, (uint32_t)rows, (uint32_t)cols, col_tiles, total, \
                                                             sign_mask, bits)
        if (use_rht && per_row) NVFP4_AMAX_COL(true, true);
        else if (use_rht) NVFP4_AMAX_COL(true, false);
        else if (per_row) NVFP4_AMAX_COL(false, true);
        else NVFP4_AMAX_COL(false, false);
#undef NVFP4_AMAX_COL
    }
    return hipGetLastError();
}

hipError_t launch_quant_1x16(const uint16_t* x, int64_t rows, int64_t cols, bool colwise, bool per_row, Mode mode,
                             const float* amax, uint32_t sign_mask, Philox rng, uint8_t* codes, uint8_t* scales,
                             float* g, hipStream_t stream) {
    const RngArgs ra = rng_args(rng);
    const int64_t rv = colwise ? cols : rows;
    if (rows == 0 || cols == 0) return write_empty_g(amax, g, per_row ? (uint32_t)rv : 1u, stream);
    if (!colwise) {
        const uint32_t bpr = (uint32_t)(cols / 16);
        const uint32_t total = (uint32_t)(rows * bpr);
        const FastDiv fd = make_fastdiv(bpr);
        const uint32_t grid = grid_for(total, kThreads, 16);
        const uint4* xv = reinterpret_cast<const uint4*>(x);
        uint2* cv = reinterpret_cast<uint2*>(codes);
#define NVFP4_ROW(M, P) \
    k_quant_rowwise<M, P><<<grid, kThreads, 0, stream>>>(xv, total, fd, amax, sign_mask, ra, cv, scales, g)
        switch (mode) {
            case kRN: if (per_row) NVFP4_ROW(kRN, true); else NVFP4_ROW(kRN, false); break;
            case kSR: if (per_row) NVFP4_ROW(kSR, true); else NVFP4_ROW(kSR, false); break;
            case kRHTSR: if (per_row) NVFP4_ROW(kRHTSR, true); else NVFP4_ROW(kRHTSR, false); break;
        }
#undef NVFP4_ROW
    } else {
        constexpr int RBW = kColRBW;
        const uint32_t tile_cols = 8 * (64 / RBW), tile_rb = 4 * RBW;
        const uint32_t col_tiles = (uint32_t)((cols + tile_cols - 1) / tile_cols);
        const uint32_t row_tiles = (uint32_t)((rows / 16 + tile_rb - 1) / tile_rb);
        const uint32_t total = col_tiles * row_tiles;
        const uint32_t grid = grid_for(total, 1, 16);
#define NVFP4_COL(M, P)                                                                                       \
    k_quant_colwise<M, P, RBW><<<grid, kThreads, 0, stream>>>(x, (uint32_t)rows, (uint32_t)cols, col_tiles, \
                                                              total, amax, sign_mask, ra, codes, scales, g)
        switch (mode) {
            case kRN: if (per_row) NVFP4_COL(kRN, true); else NVFP4_COL(kRN, false); break;
            case kSR: if (per_row) NVFP4_COL(kSR, true); else NVFP4_COL(kSR, false); break;
            case kRHTSR: if (per_row) NVFP4_COL(kRHTSR, true); else NVFP4_COL(kRHTSR, false); break;
        }
#undef NVFP4_COL
    }
    return hipGetLastError();
}

hipError_t launch_quant_16x16(const uint16_t* x, int64_t rows, int64_t cols, const float* amax, uint8_t* codes_w,
                              uint8_t* scales_w, float* g_w, uint8_t* codes_wt, uint8_t* scales_wt, float* g_wt,
                              hipStream_t stream) {
    if (rows == 0 || cols == 0) {
        hipError_t e = hipSuccess;
        if (codes_w) e = write_empty_g(amax, g_w, 1u, stream);
        if (e == hipSuccess && codes_wt) e = write_empty_g(amax, g_wt, 1u, stream);
        return e;
    }
    constexpr int TR = 4;
    const uint32_t ntr = (uint32_t)(rows / 16), ntc = (uint32_t)(cols / 16);
    const uint32_t col_groups = (ntc + 31) / 32;
    const uint32_t row_groups = (ntr + 4 * TR - 1) / (4 * TR);
    const uint32_t total = col_groups * row_groups;
    const uint32_t grid = grid_for(total, 1, 16);
#define NVFP4_2D(W, T)                                                                                          \
    k_quant_16x16<W, T, TR><<<grid, kThreads, 0, stream>>>(x, (uint32_t)rows, (uint32_t)cols, col_groups, total, \
                                                           amax, codes_w, scales_w, g_w, codes_wt, scales_wt, g_wt)
    if (codes_w && codes_wt) NVFP4_2D(true, true);
    else if (codes_w) NVFP4_2D(true, false);
    else NVFP4_2D(false, true);
#undef NVFP4_2D
    return hipGetLastError();
}

hipError_t launch_quant_4o6(const uint16_t* x, int64_t rows, int64_t cols, bool per_row, const float* amax,
                            uint8_t* codes, uint8_t* scales, float* g, hipStream_t stream) {
    if (rows == 0 || cols == 0) return write_empty_g(amax, g, per_row ? (uint32_t)rows : 1u, stream);
    const uint32_t bpr = (uint32_t)(cols / 16);
    const uint32_t total = (uint32_t)(rows * bpr);
    const FastDiv fd = make_fastdiv(bpr);
    const uint32_t grid = grid_for(total, kThreads, 16);
    if (per_row)
        k_quant_4o6<true><<<grid, kThreads, 0, stream>>>(reinterpret_cast<const uint4*>(x), total, fd, amax,
                                                          reinterpret_cast<uint2*>(codes), scales, g);
    else
        k_quant_4o6<false><<<grid, kThreads, 0, stream>>>(reinterpret_cast<const uint4*>(x), total, fd, amax,
                                                           reinterpret_cast<uint2*>(codes), scales, g);
    return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* g, int64_t rv, int64_t cv,
                             bool per_row, float* y, hipStream_t stream) {
    if (rv == 0 || cv == 0) return hipSuccess;
    const uint32_t bpr = (uint32_t)(cv / 16);
    const uint32_t total = (uint32_t)(rv * bpr);
    const FastDiv fd = make_fastdiv(bpr);
    const uint32_t grid = grid_for(total, kThreads, 16);
    if (per_row)
        k_dequantize<true><<<grid, kThreads, 0, stream>>>(reinterpret_cast<const uint2*>(codes), scales, g, total, fd,
                                                          reinterpret_cast<float4*>(y));
    else
        k_dequantize<false><<<grid, kThreads, 0, stream>>>(reinterpret_cast<const uint2*>(codes), scales, g, total,
                                                           fd, reinterpret_cast<float4*>(y));
    return hipGetLastError();
}

}  // namespace nvfp4
