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
//   * The op is O(|X|) and memory-bound ([P1, random Hadamard transform]: not a real GEMM).  A 16-point transform is
//     far too narrow for MFMA, so the Hadamard product is an in-register butterfly; nothing is staged in LDS.
//   * Every lane owns whole 16-element blocks, so block maxima, scales, Philox and packing need no cross-lane
//     traffic.  Column-wise (blocks run down columns of X): a lane loads 16 rows x 8 columns with 16 loads of 16
//     bytes (a wave reads 1 KiB contiguous per row) and transposes in registers into 8 complete column blocks.
//   * Persistent waves: each wave walks a contiguous run of tiles with the next tile's loads in flight while the
//     current one is computed (double-buffered registers), so HBM streaming overlaps the VALU work.
//   * E2M1 rounding uses the gfx950 FP4 conversions with a unit scale: v_cvt_scalef32_pk_fp4_f32 rounds to nearest
//     even and saturates at +-6; v_cvt_scalef32_sr_pk_fp4_f32 rounds the first element of its pair up exactly when
//     the element's fraction (in grid steps) plus the seed's top bits carries, so the seed (255 - rho) << 24 makes it
//     round up iff rho < floor(256 * frac) -- the stochastic-rounding rule [P1, stochastic rounding] with one random
//     byte per element.  Both agree with the definition on every non-NaN binary32 input; NaN is patched to 0x7.
//   * Bit-exact arithmetic: every step is one IEEE binary32 operation (built with -ffp-contract=off, no fast-math,
//     denormals kept); divisions are HIP's correctly rounded ones.
//   * No host synchronisation: the global scale is computed on the device from the amax buffer ([P2, results]).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <atomic>

#include "nvfp4_launch.h"




namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerGroup = kThreads / 64;
constexpr int kThreads16 = 1024;                  // 16x16 four-over-six workgroups
constexpr int kWavesPerGroup16 = kThreads16 / 64;
constexpr float kFltMax = 3.402823466e38f;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// NaN-propagating maximum of magnitudes (v_maximum3_f32 with |.| modifiers).  On non-NaN inputs it equals the
// integer maximum of the magnitude bit patterns; any NaN input gives NaN.
__device__ __forceinline__ float absmax3(float m, float a, float b) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(m, __builtin_fabsf(a)), __builtin_fabsf(b));
}

// ------------------------------------------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC'11): published multipliers and Weyl increments; the key schedule is uniform
// and lives in scalar registers; each output word's three-way xor is one v_bitop3.
// ------------------------------------------------------------------------------------------------------------
constexpr uint32_t kPhiloxMulA = 0xD2511F53u;  // multiplies counter word 0
constexpr uint32_t kPhiloxMulB = 0xCD9E8D57u;  // multiplies counter word 2
constexpr uint32_t kPhiloxWeylA = 0x9E3779B9u;
constexpr uint32_t kPhiloxWeylB = 0xBB67AE85u;

struct Rand4 {
    uint32_t w[4];
};

__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// Philox4x32-10 of counter (c0, c1, c2, c3) and key (k0, k1), returning the bitwise complement of the four output
// words (the SR seeds need 255 - rho); the complement is folded into the last round's three-way xors where
// possible.
__device__ __forceinline__ Rand4 philox4x32_10_inv(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                   uint32_t k1) {
#pragma unroll
    for (int round = 0; round < 9; ++round) {
        const uint64_t pa = (uint64_t)kPhiloxMulA * c0;
        const uint64_t pb = (uint64_t)kPhiloxMulB * c2;
        const uint32_t n0 = xor3((uint32_t)(pb >> 32), c1, k0);
        const uint32_t n2 = xor3((uint32_t)(pa >> 32), c3, k1);
        c1 = (uint32_t)pb;
        c3 = (uint32_t)pa;
        c0 = n0;
        c2 = n2;
        k0 += kPhiloxWeylA;
        k1 += kPhiloxWeylB;
    }
    const uint64_t pa = (uint64_t)kPhiloxMulA * c0;
    const uint64_t pb = (uint64_t)kPhiloxMulB * c2;
    return Rand4{{(uint32_t)__builtin_amdgcn_bitop3_b32((uint32_t)(pb >> 32), c1, k0, 0x69), ~(uint32_t)pb,
                  (uint32_t)__builtin_amdgcn_bitop3_b32((uint32_t)(pa >> 32), c3, k1, 0x69), ~(uint32_t)pa}};
}

// Random bytes of the 1x16 block with row-major index n in the quantized view ([P1, vibe-coding and timeline
// sections]: the counter layout is part of the semantics): key = seed, counter = (n, offset) as 32-bit words.
struct RngArgs {
    uint32_t k0, k1, o0, o1;
};

// Complemented random words of the block (bytes 255 - rho).  Block indices stay below 2^31 (a tensor holds fewer
// than 2^35 elements), so the high counter word is zero; with the offset words uniform, the first round's product of
// counter word 2 and the second round's product of word 0 are then the same in every lane and are formed by the
// scalar unit.
__device__ __forceinline__ Rand4 block_rand_inv(const RngArgs& a, uint32_t n) {
    return philox4x32_10_inv(n, 0u, a.o0, a.o1, a.k0, a.k1);
}

// ------------------------------------------------------------------------------------------------------------
// E4M3 ("fn") block scale.  [P2, layout]: E4M3 per-block scale over an FP32 global scale.  Round to nearest even,
// saturate above 448 (the "satfinite" convention of the conversions in [P1]), NaN -> 0x7F, s <= 0 -> 0.
// gfx950's fp32 -> E4M3 conversion rounds to nearest even; clamping to [0, 448] first (NaN-propagating min/max)
// supplies the saturation and the zero floor, and NaN is mapped to 0x7F explicitly.  Verified against the
// definition on all 2^32 binary32 inputs; the E4M3 -> fp32 conversion equals the exact decode on all 256 codes.
// ------------------------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
    const float c = __builtin_elementwise_minimum(__builtin_elementwise_maximum(s, 0.0f), 448.0f);
    const uint32_t code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, 0.0f, 0, false);   // byte 1 is fp8(0) = 0
    return (s != s) ? 0x7Fu : code;
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {  // any byte: sign bit, 0x7F/0xFF are NaN
    return __builtin_amdgcn_cvt_f32_fp8((int)c, 0);
}

// Element multiplier of block scale code sb: S = fl(decode(sb) g), r = fl(1 / S), with r = 0 for S = 0, NaN for a
// NaN S and FLT_MAX when the reciprocal overflows.
__device__ __forceinline__ float scale_multiplier(uint32_t sb, float g) {
    const float S = e4m3_decode(sb) * g;
    float r = 1.0f / S;
    r = __builtin_isinf(r) ? kFltMax : r;
    r = (S == 0.0f) ? 0.0f : r;
    return (S != S) ? S : r;
}

// Divisor of the block-scale quotient s = fl(bamax / d), d = fl(T g).  The quotient is formed with Markstein's
// method (P. Markstein, "Computation of elementary functions on the IBM RISC System/6000 processor", IBM J. Res.
// Dev. 34(1), 1990): from y = fl(1/d) and q = fl(bamax y), which is within one ulp of bamax/d, the exact FMA
// residual e = bamax - q d gives the correctly rounded quotient fl(q + e y), provided no step underflows or
// overflows.  That holds for 2^-60 <= d <= 2^60 and 2^-20 <= q <= 2^64.  Below that window of q the result stays
// within a few units of the (sub)normal grid of a quotient under 2^-20, so the code is 0 either way; q is clamped to
// 2^20 from above, where the code saturates either way (an infinite or NaN bamax still yields inf or NaN).  Other d
// use the division.
struct Divisor {
    float d, y;
    bool fast;
};

__device__ __forceinline__ Divisor make_divisor(float d) {
    return Divisor{d, 1.0f / d, d >= 0x1p-60f && d <= 0x1p60f};
}

// A value equal in every lane, moved to a scalar register.
__device__ __forceinline__ float uniform_f(float v) {
    return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(v)));
}

// The same for a d that is equal in every lane: the branch on fast becomes a scalar one.
__device__ __forceinline__ Divisor make_divisor_uniform(float d) {
    const Divisor v = make_divisor(d);
    return Divisor{v.d, v.y, __builtin_amdgcn_readfirstlane((uint32_t)v.fast) != 0};
}

// Block scale code: sb = E4M3(fl(bamax / d)), with s = 0 for bamax = 0 (which the Markstein branch gives by itself:
// y is finite there).
__device__ __forceinline__ uint32_t scale_code(float bamax, const Divisor& dv) {
    float s;
    if (dv.fast) {
        const float q = __builtin_fminf(bamax * dv.y, 0x1p20f);
        s = __builtin_fmaf(__builtin_fmaf(-q, dv.d, bamax), dv.y, q);
    } else {
        s = bamax == 0.0f ? 0.0f : bamax / dv.d;
    }
    return e4m3_encode(s);
}

// NaN-propagating maximum of the 16 magnitudes (a depth-3 tree of v_maximum3).
__device__ __forceinline__ float absmax16(const float (&w)[16]) {
    const float m0 = absmax3(__builtin_fabsf(w[0]), w[1], w[2]);
    const float m1 = absmax3(__builtin_fabsf(w[3]), w[4], w[5]);
    const float m2 = absmax3(__builtin_fabsf(w[6]), w[7], w[8]);
    const float m3 = absmax3(__builtin_fabsf(w[9]), w[10], w[11]);
    const float m4 = absmax3(__builtin_fabsf(w[12]), w[13], w[14]);
    const float m5 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m0, m1), m2);
    const float m6 = absmax3(__builtin_elementwise_maximum(m3, m4), w[15], w[15]);
    return __builtin_elementwise_maximum(m5, m6);
}

// The value held by the other lane of this lane's pair (lanes 2m, 2m + 1): DPP quad permutation [1, 0, 3, 2].
__device__ __forceinline__ float pair_swap(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}

// Maxima over a wave / workgroup of magnitude bit patterns (integer maximum: NaN > inf > finite).
// The wave's maximum, equal in every lane (every lane active): DPP steps within each 16-lane row (the quad's lanes
// i ^ 1 and i ^ 2, then the mirrored half row and the mirrored row), then the four rows' results read into scalar
// registers, so no step goes through LDS (cross-lane shuffles are LDS permutes, which queue behind the LDS traffic
// of the other workgroups on the CU).  A source lane outside the row or disabled yields the lane's own value.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
    v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));    // quad [1,0,3,2]
    v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));    // quad [2,3,0,1]
    v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false));   // row_half_mirror
    v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false));   // row_mirror
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return umax(umax(a, b), umax(c, d));
}

template <int WAVES = kWavesPerGroup>
__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* lds) {
    v = wave_max(v);
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    if (lane == 0) lds[wave] = v;
    __syncthreads();
    uint32_t r = 0;
    if (threadIdx.x == 0) {
        for (int w = 0; w < WAVES; ++w) r = umax(r, lds[w]);
    }
    __syncthreads();
    return r;  // valid in thread 0
}

// Fast-path multiplier of a block whose scale multiplier is r: what w is multiplied by directly (0.25 r with the
// RHT, where w is the value before the transform's final 0.25), or NaN where the fast path might not reproduce the
// definition's codes, so that the block takes the general path (which maps NaN products to 0x7).  A finite r > 0
// is exact without the RHT (a zero r can meet an infinite value: inf * 0).  With it, fl(w fl(0.25 r)) and
// fl(fl(0.25 w) r) give the same code for 2^-124 <= r < 2^117: they are equal when 0.25 w is exact, and both are
// below 2^-9 (code 0 with the sign of w) when it is not.  Negative and NaN r (degenerate g) go general too.
template <bool RHT>
__device__ __forceinline__ float fast_multiplier(float r) {
    const float nan = __builtin_nanf("");
    if (RHT) return (r >= 0x1p-124f && r < 0x1p117f) ? 0.25f * r : nan;
    return (r > 0.0f && r <= kFltMax) ? r : nan;
}

// Per-tensor g: the multipliers of the 128 scale codes are tabulated once per workgroup in LDS, as r and as the
// fast-path multiplier.
struct RTable {
    float r[128];
    float rq[128];
};

template <bool RHT>
__device__ __forceinline__ void fill_rtable_entry(RTable& t, uint32_t c, float g) {
    const float r = scale_multiplier(c, g);
    t.r[c] = r;
    t.rq[c] = fast_multiplier<RHT>(r);
}

template <bool RHT>
__device__ __forceinline__ void fill_rtable(RTable& t, float g) {
    if (threadIdx.x < 128) fill_rtable_entry<RHT>(t, threadIdx.x, g);
    __syncthreads();
}

// Sources of the block multipliers: a per-tensor table, or computed per block from a per-row g.
struct TableMul {
    const RTable& t;
    __device__ float rq(uint32_t c) const { return t.rq[c]; }
    __device__ float r(uint32_t c) const { return t.r[c]; }
};

template <bool RHT>
struct RowMul {
    float g;
    __device__ float rq(uint32_t c) const { return fast_multiplier<RHT>(scale_multiplier(c, g)); }
    __device__ float r(uint32_t c) const { return scale_multiplier(c, g); }
};

// ------------------------------------------------------------------------------------------------------------
// E2M1 encoding with the gfx950 conversions (unit scale).  Element 2k goes to the low nibble of byte k.
// ------------------------------------------------------------------------------------------------------------
// Byte sel of d replaced by the codes of (a, b); the other bytes kept.
__device__ __forceinline__ uint32_t cvt_fp4_byte(int sel, uint32_t d, float a, float b) {
    switch (sel) {
        case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, a, b, 1.0f, 0);
        case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, a, b, 1.0f, 1);
        case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, a, b, 1.0f, 2);
        default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, a, b, 1.0f, 3);
    }
}

__device__ __forceinline__ uint32_t pack8_rn(const float (&q)[8]) {
    uint32_t d = 0;
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, q[0], q[1], 1.0f, 0);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, q[2], q[3], 1.0f, 1);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, q[4], q[5], 1.0f, 2);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, q[6], q[7], 1.0f, 3);
    return d;
}

// Stochastic rounding, one conversion per element on the natural pair (q[2k], q[2k+1]): the first slot draws its
// random byte from seed bits 31..24, the second slot from bits 30..23 (the instruction shifts the seed left by one
// for it).  Element 2k uses seed (255 - rho) << 24 and keeps the low nibble; element 2k+1 uses (255 - rho) << 23
// and keeps the high nibble; the other nibble of each conversion is discarded by the final bit-select.
// Byte b of w shifted left by 24 (first slot) or 23 (second slot), the other bits zero: one SDWA shift each.
#define NVFP4_SEED(name, SHIFT, SEL)                                                                        \
    __device__ __forceinline__ uint32_t name(uint32_t w) {                                                  \
        uint32_t r;                                                                                         \
        asm("v_lshlrev_b32_sdwa %0, " #SHIFT ", %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "     \
            "src1_sel:" SEL                                                                                 \
            : "=v"(r) : "v"(w));                                                                            \
        return r;                                                                                           \
    }
NVFP4_SEED(seed_first_b0, 24, "BYTE_0")
NVFP4_SEED(seed_first_b2, 24, "BYTE_2")
NVFP4_SEED(seed_second_b1, 23, "BYTE_1")
NVFP4_SEED(seed_second_b3, 23, "BYTE_3")
#undef NVFP4_SEED

// The byte-select chain needs the accumulator tied to the destination (each conversion writes one byte and keeps
// the other three); the compiler's lowering of the SR conversion builtin does not carry that operand, so the
// instruction is written out with a tied operand here.
#define NVFP4_SR_PAIR(acc, k, seed, OPSEL)                                                \
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 " OPSEL                             \
        : "+v"(acc)                                                                       \
        : "v"(f32x2{q[2 * (k)], q[2 * (k) + 1]}), "v"(seed))
// the first conversion of a chain: the bytes it keeps are all overwritten later, so no initial value is needed
#define NVFP4_SR_FIRST(acc, seed)                                                         \
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0"                                    \
        : "=v"(acc)                                                                       \
        : "v"(f32x2{q[0], q[1]}), "v"(seed))

__device__ __forceinline__ uint32_t pack8_sr(const float (&q)[8], uint32_t inv_lo, uint32_t inv_hi) {
    // inv_lo holds the complemented random bytes of elements 0..3, inv_hi of elements 4..7
    uint32_t e, o;
    NVFP4_SR_FIRST(e, seed_first_b0(inv_lo));
    NVFP4_SR_FIRST(o, seed_second_b1(inv_lo));
    NVFP4_SR_PAIR(e, 1, seed_first_b2(inv_lo), "op_sel:[0,0,1,0]");
    NVFP4_SR_PAIR(o, 1, seed_second_b3(inv_lo), "op_sel:[0,0,1,0]");
    NVFP4_SR_PAIR(e, 2, seed_first_b0(inv_hi), "op_sel:[0,0,0,1]");
    NVFP4_SR_PAIR(o, 2, seed_second_b1(inv_hi), "op_sel:[0,0,0,1]");
    NVFP4_SR_PAIR(e, 3, seed_first_b2(inv_hi), "op_sel:[0,0,1,1]");
    NVFP4_SR_PAIR(o, 3, seed_second_b3(inv_hi), "op_sel:[0,0,1,1]");
    return (e & 0x0F0F0F0Fu) | (o & 0xF0F0F0F0u);
}
#undef NVFP4_SR_FIRST
#undef NVFP4_SR_PAIR

// NaN elements encode to 0x7 (the hardware keeps the NaN's sign).
__device__ __forceinline__ uint32_t patch_nan8(uint32_t d, const float (&q)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (q[i] != q[i]) d = (d & ~(0xFu << (4 * i))) | (0x7u << (4 * i));
    return d;
}

// Sources of a block's complemented random words: held in registers (Rand4), or read from LDS half a block at a
// time (LdsRand), so that only the two words of the half being encoded are live.
__device__ __forceinline__ uint2 rand_lo(const Rand4& r) { return make_uint2(r.w[0], r.w[1]); }
__device__ __forceinline__ uint2 rand_hi(const Rand4& r) { return make_uint2(r.w[2], r.w[3]); }
struct LdsRand {
    const uint4* p;
};
__device__ __forceinline__ uint2 rand_lo(const LdsRand& r) { return reinterpret_cast<const uint2*>(r.p)[0]; }
__device__ __forceinline__ uint2 rand_hi(const LdsRand& r) { return reinterpret_cast<const uint2*>(r.p)[1]; }

// Quantize one 16-element block; w[] is consumed (the scaled values are formed in its place).  w[] are the values
// before the final 0.25 of the transform when RHT is set (y = fl(0.25 w)), the values themselves otherwise; m is
// the block's absmax16(w); mul gives the multipliers of a scale code (fast_multiplier).  Which path a block takes
// depends only on its scale code, so it is decided before the multiply: the fast path q = fl(w rq), or the
// definition step by step, q = fl(fl(0.25 w) r) (RHT) or fl(w r), with NaN products patched to code 0x7.
template <bool SR, bool RHT, typename Mul, typename R>
__device__ __forceinline__ void quantize_block_m(float (&w)[16], float m, const Divisor& d6, const Mul& mul,
                                                 const R& inv, uint32_t& lo, uint32_t& hi, uint32_t& sb) {
    const float bamax = RHT ? 0.25f * m : m;       // max_i fl(0.25 |w_i|) = fl(0.25 max_i |w_i|)
    sb = scale_code(bamax, d6);
    const float rq = mul.rq(sb);
    const bool fast = rq == rq;
    const float r = fast ? rq : mul.r(sb);
    if (SR) {
        // The SR conversion reads its operands as aligned register pairs, so the products are formed in pairs of
        // their own, half a block at a time (fewer registers live than forming all 16 next to w).
        float q[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (fast) [[likely]] {
#pragma unroll
                for (int i = 0; i < 8; ++i) q[i] = w[8 * h + i] * r;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) q[i] = (RHT ? 0.25f * w[8 * h + i] : w[8 * h + i]) * r;
            }
            const uint2 rw = h ? rand_hi(inv) : rand_lo(inv);
            uint32_t d = pack8_sr(q, rw.x, rw.y);
            if (!fast) [[unlikely]] d = patch_nan8(d, q);
            (h ? hi : lo) = d;
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        if (fast) [[likely]] {
#pragma unroll
            for (int i = 0; i < 16; ++i) w[i] = w[i] * r;
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) w[i] = (RHT ? 0.25f * w[i] : w[i]) * r;
        }
        lo = pack8_rn(*reinterpret_cast<const float(*)[8]>(&w[0]));
        hi = pack8_rn(*reinterpret_cast<const float(*)[8]>(&w[8]));
        if (!fast) [[unlikely]] {
            lo = patch_nan8(lo, *reinterpret_cast<const float(*)[8]>(&w[0]));
            hi = patch_nan8(hi, *reinterpret_cast<const float(*)[8]>(&w[8]));
        }
    }
}

template <bool SR, bool RHT, typename Mul, typename R>
__device__ __forceinline__ void quantize_block(float (&w)[16], const Divisor& d6, const Mul& mul,
                                               const R& inv, uint32_t& lo, uint32_t& hi, uint32_t& sb) {
    quantize_block_m<SR, RHT>(w, absmax16(w), d6, mul, inv, lo, hi, sb);
}

// ------------------------------------------------------------------------------------------------------------
// 16-point Walsh-Hadamard butterfly, strides 1, 2, 4, 8, (a, b) -> (a + b, a - b) in binary32; the final 0.25 is
// applied by the caller ([P1, random Hadamard transform]; y = (1/4) H16 diag(s) v, Sylvester order).
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
}

// bf16 halves of a packed word to binary32, with the random sign applied as an exact sign-bit flip
// (flip = 0 or 0x80000000).
__device__ __forceinline__ float bf16_lo(uint32_t w, uint32_t flip) { return as_f((w << 16) + flip); }
__device__ __forceinline__ float bf16_hi(uint32_t w, uint32_t flip) { return as_f((w & 0xFFFF0000u) ^ flip); }
__device__ __forceinline__ uint32_t flip_bit(uint32_t mask, int i) { return ((mask >> i) & 1u) << 31; }

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Output stores are non-temporal: the outputs are not read again by the kernel, and streaming them past the L2
// avoids a write-back burst at the end of the launch (1-1.3 us off the column-wise quantizers).
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st_nt(void* p, uint2 v) {
    __builtin_nontemporal_store(u32x2v{v.x, v.y}, reinterpret_cast<u32x2v*>(p));
}
__device__ __forceinline__ void st_nt(void* p, uint32_t v) { __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p)); }
__device__ __forceinline__ void st_nt(void* p, uint8_t v) { __builtin_nontemporal_store(v, reinterpret_cast<uint8_t*>(p)); }
__device__ __forceinline__ void st_nt(void* p, uint4 v) {
    typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(u32x4v{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4v*>(p));
}

__device__ __forceinline__ void st_nt(void* p, float4 v) {
    __builtin_nontemporal_store(f32x4v{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4v*>(p));
}

// Row-wise block: 16 consecutive bf16 of a row (two 16-byte words) -> binary32 (sign-flipped when RHT).
template <bool RHT>
__device__ __forceinline__ void widen_row_block(const uint4& a, const uint4& b, uint32_t mask, float (&w)[16]) {
    const uint32_t ws[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        w[2 * k] = bf16_lo(ws[k], RHT ? flip_bit(mask, 2 * k) : 0u);
        w[2 * k + 1] = bf16_hi(ws[k], RHT ? flip_bit(mask, 2 * k + 1) : 0u);
    }
    if (RHT) fwht16(w);
}

// Columns 2p and 2p+1 of a lane's 16 x 8 tile (the two halves of packed word p) -> two column blocks.
template <bool RHT>
__device__ __forceinline__ void widen_col_pair(const uint4 (&v)[16], int p, uint32_t mask, float (&wa)[16],
                                               float (&wb)[16]) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const uint32_t word = p == 0 ? v[k].x : p == 1 ? v[k].y : p == 2 ? v[k].z : v[k].w;
        const uint32_t f = RHT ? flip_bit(mask, k) : 0u;
        wa[k] = bf16_lo(word, f);
        wb[k] = bf16_hi(word, f);
    }
    if (RHT) {
        fwht16(wa);
        fwht16(wb);
    }
}

// Column j (0..7) of a lane's 16 x 8 tile -> the 16 values of one column block.
template <bool RHT>
__device__ __forceinline__ void widen_col_block(const uint4 (&v)[16], int j, uint32_t mask, float (&w)[16]) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const uint32_t word = (j >> 1) == 0 ? v[k].x : (j >> 1) == 1 ? v[k].y : (j >> 1) == 2 ? v[k].z : v[k].w;
        const uint32_t f = RHT ? flip_bit(mask, k) : 0u;
        w[k] = (j & 1) ? bf16_hi(word, f) : bf16_lo(word, f);
    }
    if (RHT) fwht16(w);
}

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

// Four-over-six global scale g = fl(amax / (6 B)) for the bound B (gden = 6 B, exact); B = 448 is global_scale.
__device__ __forceinline__ float global_scale_den(float amax, float gden) { return amax / gden; }

// ------------------------------------------------------------------------------------------------------------
// Row-wise 1x16 quantization: one 16-element block per lane per step; lanes walk the blocks with a grid stride
// and keep the next block's two loads in flight.
// ------------------------------------------------------------------------------------------------------------
// Byte offset of view row r, scale column b in the tiled scale layout of the FP4 GEMM (tiles of 128 rows x 4 scale
// columns, each a [32][4][4] byte array: byte 16 a + 4 i + j = row 32 i + a, scale column j; bt tiles per row tile).
__device__ __forceinline__ size_t tiled_scale_offset(uint32_t r, uint32_t b, uint32_t bt) {
    return ((size_t)(r >> 7) * bt + (b >> 2)) * 512 + 16 * (r & 31u) + 4 * ((r >> 5) & 3u) + (b & 3u);
}
// The work of workgroup wg of nwg on one tensor (a kernel's own grid, or its share of a grouped launch).
template <int MODE, bool PER_ROW>
// tbt != 0: the scales in the tiled layout of the FP4 GEMM (tbt scale-column tiles per row tile) when it has no
// padding (rows a multiple of 128, blocks per row a multiple of 4): each block's byte goes to its place in the tiles
// as a cached store, so the 4-byte pieces of a tile row meet in L2.  per_row divides by the blocks per row.
__device__ __forceinline__ void quant_rowwise_wg(const uint4* __restrict__ x, uint32_t total_blocks, FastDiv per_row,
                                                 const float* __restrict__ amax, uint32_t sign_mask, RngArgs rng,
                                                 uint2* __restrict__ codes, uint8_t* __restrict__ scales,
                                                 float* __restrict__ gout, uint32_t wg, uint32_t nwg, RTable& tab,
                                                 uint32_t tbt = 0) {
    constexpr bool SR = MODE != kRN;
    constexpr bool RHT = MODE == kRHTSR;
    // the first block's loads go out before the amax read and the table fill (RN at 8192 x 4096: 17.3 -> 16.4 us)
    const uint32_t stride = nwg * kThreads;
    uint32_t n = wg * kThreads + threadIdx.x;
    uint4 a{}, b{};
    if (n < total_blocks) {
        a = ld16(x + 2 * (size_t)n);
        b = ld16(x + 2 * (size_t)n + 1);
    }
    float g = 0.0f;
    Divisor d6{};
    if (!PER_ROW) {
        g = global_scale(amax[0]);
        d6 = make_divisor_uniform(6.0f * g);
        if (wg == 0 && threadIdx.x == 0) gout[0] = g;
        fill_rtable<RHT>(tab, g);
    }
    if (n >= total_blocks) return;
    for (; n < total_blocks; n += stride) {
        const uint32_t nn = n + stride;
        uint4 a2 = a, b2 = b;
        if (nn < total_blocks) {
            a2 = ld16(x + 2 * (size_t)nn);
            b2 = ld16(x + 2 * (size_t)nn + 1);
        }
        float w[16];
        widen_row_block<RHT>(a, b, sign_mask, w);
        Rand4 rnd{{0, 0, 0, 0}};
        if (SR) rnd = block_rand_inv(rng, n);
        uint32_t lo, hi, sb;
        if (PER_ROW) {
            const uint32_t row = fdiv(n, per_row);
            const float gr = global_scale(amax[row]);
            if (n == row * per_row.d) gout[row] = gr;
            quantize_block<SR, RHT>(w, make_divisor(6.0f * gr), RowMul<RHT>{gr}, rnd, lo, hi, sb);
        } else {
            quantize_block<SR, RHT>(w, d6, TableMul{tab}, rnd, lo, hi, sb);
        }
        st_nt(codes + n, make_uint2(lo, hi));
        if (tbt) {
            const uint32_t row = fdiv(n, per_row);
            scales[tiled_scale_offset(row, n - row * per_row.d, tbt)] = (uint8_t)sb;
        } else {
            st_nt(scales + n, (uint8_t)sb);
        }
        a = a2;
        b = b2;
    }
}

template <int MODE, bool PER_ROW>
__global__ void __launch_bounds__(kThreads)
k_quant_rowwise(const uint4* __restrict__ x, uint32_t total_blocks, FastDiv per_row, const float* __restrict__ amax,
                uint32_t sign_mask, RngArgs rng, uint2* __restrict__ codes, uint8_t* __restrict__ scales,
                float* __restrict__ gout, uint32_t tbt) {
    __shared__ RTable tab;
    quant_rowwise_wg<MODE, PER_ROW>(x, total_blocks, per_row, amax, sign_mask, rng, codes, scales, gout, blockIdx.x,
                                    gridDim.x, tab, tbt);
}

// ------------------------------------------------------------------------------------------------------------
// Row-wise quantization with the scales in the FP4 GEMM's tiled layout (128 x 4 tiles, each a [32][4][4] byte
// array: byte 16 a + 4 b + c = row 32 b + a, scale column c; row-tile major; zero padding).  A tile needs 128 rows,
// so these kernels give each workgroup item a 128-row x 64-block piece of V (16 tiles of scales): slice j = 0..7 of
// the item is rows 16 j .. 16 j + 15, wave w takes row 16 j + w and lane l block l, so a wave reads 2 KiB of a row
// and writes 512 contiguous bytes of codes; the scale bytes are collected in LDS and written as 16 whole tiles
// (8 KiB, contiguous).
// ------------------------------------------------------------------------------------------------------------
struct RowTileItem {
    uint32_t row0;   // first row of V
    uint32_t blk0;   // first block of those rows
};

__device__ __forceinline__ RowTileItem row_tile_item(uint32_t item, uint32_t items_per_band) {
    const uint32_t band = item / items_per_band;
    return RowTileItem{128 * band, 64 * (item - band * items_per_band)};
}

// Writes the item's 16 tiles (8 KiB, contiguous); get(r, c) is the scale byte of row r (0..127) and block c (0..63)
// of the item.  Thread t < 512 takes tile row a = t % 32 of tile t / 32: four 4-byte pieces of rows a, a + 32,
// a + 64, a + 96.  Rows past rows and blocks past nb are written as zero; tiles past the last scale column are not
// written.
template <typename F>
__device__ __forceinline__ void row_write_scales_tiled(const RowTileItem& it, uint32_t rows, uint32_t nb,
                                                       uint8_t* __restrict__ scales, F get) {
    if (threadIdx.x >= 512) return;
    const uint32_t tb = threadIdx.x >> 5, a = threadIdx.x & 31u;
    const uint32_t bt = (nb + 3) / 4, B = it.blk0 / 4 + tb;
    if (B >= bt) return;
    uint32_t w[4];
#pragma unroll
    for (uint32_t b = 0; b < 4; ++b) {
        const uint32_t r = 32 * b + a;
        uint32_t v = 0;
        if (it.row0 + r < rows) {
#pragma unroll
            for (uint32_t c = 0; c < 4; ++c)
                if (it.blk0 + 4 * tb + c < nb) v |= (uint32_t)get(r, 4 * tb + c) << (8 * c);
        }
        w[b] = v;
    }
    st_nt(scales + ((size_t)(it.row0 / 128) * bt + B) * 512 + 16 * a, make_uint4(w[0], w[1], w[2], w[3]));
}

// Amax given: 512-thread workgroups loop over the items; wave w takes rows 8 j + w (j = 0..15) of the item, block l
// in lane l, with the next block's loads in flight.  The LDS scale stage is double-buffered, so one barrier per item
// separates its writes from the read-out of the item before.
constexpr uint32_t kThreadsRT = 512;

template <int MODE, bool PER_ROW>
__global__ void __launch_bounds__(kThreadsRT)
k_quant_rowwise_tiled(const uint4* __restrict__ x, uint32_t rows, uint32_t nb, uint32_t items_per_band, uint32_t items,
                      const float* __restrict__ amax, uint32_t sign_mask, RngArgs rng, uint2* __restrict__ codes,
                      uint8_t* __restrict__ scales, float* __restrict__ gout) {
    constexpr bool SR = MODE != kRN;
    constexpr bool RHT = MODE == kRHTSR;
    __shared__ RTable tab;
    __shared__ uint8_t sc[2][128][68];
    float g = 0.0f;
    Divisor d6{};
    if (!PER_ROW) {
        g = uniform_f(global_scale(amax[0]));   // uniform values kept in scalar registers
        d6 = make_divisor_uniform(6.0f * g);
        d6.d = uniform_f(d6.d);
        d6.y = uniform_f(d6.y);
        if (blockIdx.x == 0 && threadIdx.x == 0) gout[0] = g;
        fill_rtable<RHT>(tab, g);
    }
    const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63u;
    uint32_t buf = 0;
    for (uint32_t item = blockIdx.x; item < items; item += gridDim.x, buf ^= 1u) {
        const RowTileItem it = row_tile_item(item, items_per_band);
        const uint32_t blk = it.blk0 + lane;
        auto row_of = [&](uint32_t j) { return it.row0 + 8 * j + wave; };
        auto valid = [&](uint32_t j) { return blk < nb && row_of(j) < rows; };
        uint4 a = {}, b = {};
        if (valid(0)) {
            const size_t n = (size_t)row_of(0) * nb + blk;
            a = ld16(x + 2 * n);
            b = ld16(x + 2 * n + 1);
        }
#pragma unroll 2
        for (uint32_t j = 0; j < 16; ++j) {
            uint4 a2 = a, b2 = b;
            if (j + 1 < 16 && valid(j + 1)) {
                const size_t nn = (size_t)row_of(j + 1) * nb + blk;
                a2 = ld16(x + 2 * nn);
                b2 = ld16(x + 2 * nn + 1);
            }
            if (valid(j)) {
                const uint32_t row = row_of(j);
                const size_t n = (size_t)row * nb + blk;
                float w[16];
                widen_row_block<RHT>(a, b, sign_mask, w);
                Rand4 rnd{{0, 0, 0, 0}};
                if (SR) rnd = block_rand_inv(rng, (uint32_t)n);
                uint32_t lo, hi, sb;
                if (PER_ROW) {
                    const float gr = global_scale(amax[row]);
                    if (blk == 0) gout[row] = gr;
                    quantize_block<SR, RHT>(w, make_divisor(6.0f * gr), RowMul<RHT>{gr}, rnd, lo, hi, sb);
                } else {
                    quantize_block<SR, RHT>(w, d6, TableMul{tab}, rnd, lo, hi, sb);
                }
                st_nt(codes + n, make_uint2(lo, hi));
                sc[buf][8 * j + wave][lane] = (uint8_t)sb;
            }
            a = a2;
            b = b2;
        }
        __syncthreads();
        row_write_scales_tiled(it, rows, nb, scales, [&](uint32_t r, uint32_t c) { return sc[buf][r][c]; });
    }
}

// ------------------------------------------------------------------------------------------------------------
// Column-wise kernels (quantize, amax, 16x16).  A workgroup covers 16 row-blocks (256 rows) by a strip of 512
// columns; each of its 16 waves takes one row-block (16 rows) of the strip, and lane l owns columns 8l..8l+7, so one
// load instruction reads 1 KiB of a row.  A lane keeps its 16 rows x 8 columns in registers (word p of row k holds
// its columns 2p and 2p+1) and transposes them into 8 column blocks there.  Workgroups are numbered strip-fastest
// with the strip rotated by the row group: workgroups are dealt round-robin to the 8 XCDs, and the rotation makes
// every XCD read every strip (without it, with 8 strips, each XCD would read one fixed 1 KiB column range of every
// row, and the XCDs' read rates differ by a third).  Results are staged in LDS and written out so that every output
// row of X^T receives its 16 row-blocks (128 bytes of codes, 16 bytes of scales) as contiguous stores; stores of
// 8-byte pieces straight from the waves run at half the speed.
// ------------------------------------------------------------------------------------------------------------
constexpr int kColRB = 16;                     // row-blocks per workgroup (one per wave)
constexpr int kColThreads = 64 * kColRB;       // 1024

// LDS staging of RB row-blocks' codes and scales, [j][lane][row-block] with rows of RB + 1 entries.
template <int RB>
struct ColStage {
    uint2 codes[8 * 64 * (RB + 1)];            // 8 codes bytes per block
    // the tile scale codes of a 16x16 item (RB row-blocks x 32 tile columns), in both orders: a W scale row takes 32
    // contiguous tile columns of one row-block, a W^T scale row 16 contiguous row-blocks of one tile column
    __align__(16) uint8_t tsw[RB][32];
    __align__(16) uint8_t tst[32][RB];
};

struct ColGrid {
    uint32_t nrb;      // row-blocks (rows / 16)
    uint32_t nstrips;  // strips of 512 columns
    uint32_t ntiles;   // workgroup tiles: ceil(nrb / RB) * nstrips, RB row-blocks per workgroup
};

struct ColPos {
    uint32_t group;  // row group (RB row-blocks)
    uint32_t strip;  // 512-column strip
    uint32_t rb;     // this wave's row-block
    uint32_t lane;
    uint32_t c8;     // first of the lane's 8 columns
};

template <int RB = kColRB>
__device__ __forceinline__ ColPos col_position(const ColGrid& g, uint32_t tile) {
    ColPos p;
    p.group = tile / g.nstrips;
    const uint32_t s = tile - p.group * g.nstrips + p.group % g.nstrips;
    p.strip = s >= g.nstrips ? s - g.nstrips : s;
    p.rb = p.group * RB + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    p.lane = threadIdx.x & 63u;
    p.c8 = p.strip * 512 + 8 * p.lane;
    return p;
}

// Issues the 16 loads of the lane's 16 x 8 tile (cols is a multiple of 8: a lane's columns exist all or none).  The
// loads go through a buffer resource over the wave's 16 rows (a wave-uniform base): the lane offset is one 32-bit
// register and the row offset a scalar, where 64-bit addresses would take two registers per load in flight.  The
// row-block spans 32 cols bytes, below 2^32 by the column-wise size limit.
__device__ __forceinline__ void load_col_tile(const uint16_t* x, uint32_t cols, const ColPos& p, uint4 (&v)[16]) {
    const uint16_t* base = x + (size_t)(16 * p.rb) * cols;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, (int)(32u * cols), 0x00020000);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(2u * p.c8), (int)(2u * k * cols), 0);
        v[k] = make_uint4(t.x, t.y, t.z, t.w);
    }
}

template <int RB>
__device__ __forceinline__ uint32_t stage_index(uint32_t j, uint32_t lane, uint32_t rbl) {
    return (j * 64 + lane) * (RB + 1) + rbl;
}

// Writes the staged codes of the workgroup (64 RB threads): (column, row-block) pairs with the row-block fastest, so
// RB consecutive threads store one output row's 8 RB contiguous bytes of codes.
template <int RB>
__device__ __forceinline__ void col_write_out(const ColStage<RB>& st, const ColPos& p, uint32_t rows, uint32_t cols,
                                              uint32_t nrb, uint8_t* __restrict__ codes) {
    const uint32_t col0 = p.strip * 512;
    const uint32_t ncol = min(512u, cols - col0), nr = min((uint32_t)RB, nrb - p.group * RB);
    const uint32_t rbl = threadIdx.x % RB, rb = p.group * RB + rbl;
    if (rbl >= nr) return;
    for (uint32_t cl = threadIdx.x / RB; cl < ncol; cl += 64) {
        const uint32_t si = stage_index<RB>(cl & 7, cl >> 3, rbl);
        st_nt(codes + (size_t)(col0 + cl) * (rows >> 1) + 8 * (size_t)rb, st.codes[si]);
    }
}

// The first n (<= 16) bytes of v to dst: one 16-byte store when whole is set (n == 16, dst 16-byte aligned), else
// byte by byte (straight-line predicated stores: a loop with a variable trip count here raised the register pressure
// of the 16x16 kernel into spills).
__device__ __forceinline__ void store_piece16(uint8_t* __restrict__ dst, const uint4& v, uint32_t n, bool whole) {
    if (whole) {
        *reinterpret_cast<uint4*>(dst) = v;
        return;
    }
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (uint32_t i = 0; i < 16; ++i)
        if (i < n) dst[i] = (uint8_t)(w[i >> 2] >> (8 * (i & 3u)));
}

// The W scale rows of one row-block of a 16x16 item, written by its wave: row 16 rb + k takes the item's 32 tile
// columns, two 16-byte pieces, one per lane 0..31 (lane 2 k + half).  The wave's lane pairs have put their scale codes
// in its row of tsw; the wave reads back what its own lanes wrote, so a wavefront-scope fence (the wait for its LDS
// writes) stands in for a workgroup barrier.  Ordinary (cached) stores, so that the pieces that the items of
// neighbouring strips write into one line can meet in L2.  Pieces that are not whole, or not 16-byte aligned in the
// output (cols % 256 != 0), are written byte by byte.
template <int RB>
__device__ __forceinline__ void write_w_scales(const ColStage<RB>& st, const ColPos& p, uint32_t cols,
                                               uint8_t* __restrict__ sw) {
    const uint32_t ntc = cols >> 4, tc0 = p.strip * 32, ntcs = min(32u, ntc - tc0);
    const uint32_t rbl = p.rb - p.group * RB, k = p.lane >> 1, half = p.lane & 1u;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (p.lane >= 32 || 16 * half >= ntcs) return;
    uint8_t* dst = sw + (size_t)(16 * p.rb + k) * ntc + tc0 + 16 * half;
    const uint8_t* src = &st.tsw[rbl][16 * half];
    const uint32_t n = min(16u, ntcs - 16 * half);
    store_piece16(dst, *reinterpret_cast<const uint4*>(src), n, n == 16 && (ntc & 15u) == 0);
}

// The W^T scale rows of a 16x16 item (after the workgroup barrier; threads 512 .. 1023 of 1024): output row c takes the
// 16 row-blocks of its tile column, one 16-byte piece.  Ordinary (cached) stores; pieces that are not whole, or not
// 16-byte aligned in the output (rows % 256 != 0), are written byte by byte.
template <int RB>
__device__ __forceinline__ void write_wt_scales(const ColStage<RB>& st, const ColPos& p, uint32_t cols, uint32_t nrb,
                                                uint8_t* __restrict__ st_scales) {
    static_assert(RB == 16, "one 16-byte piece per row needs 16 row-blocks");
    const uint32_t col0 = p.strip * 512, nr = min((uint32_t)RB, nrb - p.group * RB);
    const uint32_t cl = threadIdx.x - 512;
    if (threadIdx.x < 512 || cl >= min(512u, cols - col0)) return;
    uint8_t* dst = st_scales + (size_t)(col0 + cl) * nrb + p.group * RB;
    const uint8_t* src = &st.tst[cl >> 4][0];
    store_piece16(dst, *reinterpret_cast<const uint4*>(src), nr, nr == 16 && (nrb & 15u) == 0);
}

// LDS of a column-wise workgroup that generates every block's random words ahead of the data: entry (wave, j,
// lane) first holds the four Philox words of the lane's block j, then that block's codes (x, y) and scale (z).  A
// wave's region is padded by one entry so that the write-out, which reads the 16 row-blocks (= waves) of one
// column, hits 16 different bank groups.
struct ColStash {
    uint4 e[kColRB][8 * 64 + 1];
};

// Column-wise quantization with a device-resident amax.  The workgroup tile is the same 16 row-blocks x 512 columns,
// but split among the waves so that the four waves that receive their data together finish a complete piece of the
// output: wave w = 4 q + i covers columns 128 q .. 128 q + 127 of the strip and row-blocks 4 i .. 4 i + 3 (lanes
// 16 s .. 16 s + 15 take row-block 4 i + s, 8 columns each), so waves 4 q .. 4 q + 3 hold all 16 row-blocks of 128
// columns.  Waves of a workgroup are dispatched in order to the four SIMDs, which serve their oldest wave first, and
// the memory system answers in about the order of the requests: waves 0-3 get their data first, then 4-7, and so on.
// Each quad's last wave to finish (an LDS counter) writes the quad's 128 output rows of 128 bytes of codes and 16 of
// scales, so those stores overlap the later quads' loads and arithmetic instead of following a workgroup barrier.
struct QuadPos {
    uint32_t group;  // row group (16 row-blocks)
    uint32_t strip;  // 512-column strip
    uint32_t q;      // column quarter of the strip (128 columns) = the wave's quad
    uint32_t i;      // the wave's four row-blocks within the group: 4 i .. 4 i + 3
    uint32_t s;      // the lane's row-block within those four
    uint32_t lane;
    uint32_t rb0;    // first row-block of the wave (wave-uniform)
    uint32_t rb;     // the lane's row-block
    uint32_t c8;     // first of the lane's 8 columns
};

__device__ __forceinline__ QuadPos quad_position(const ColGrid& g, uint32_t tile) {
    QuadPos p;
    p.group = tile / g.nstrips;
    const uint32_t s = tile - p.group * g.nstrips + p.group % g.nstrips;
    p.strip = s >= g.nstrips ? s - g.nstrips : s;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    p.q = wave >> 2;
    p.i = wave & 3u;
    p.lane = threadIdx.x & 63u;
    p.s = p.lane >> 4;
    p.rb0 = p.group * kColRB + 4 * p.i;
    p.rb = p.rb0 + p.s;
    p.c8 = p.strip * 512 + 128 * p.q + 8 * (p.lane & 15u);
    return p;
}

// The lane's 16 rows x 8 columns (row k of its row-block in v[k]); one load instruction reads 256 contiguous bytes
// of a row in each of the wave's four row-blocks.  Offsets from the wave's first row-block stay below 128 cols bytes,
// which the column-wise size limit (cols < 2^25) keeps below 2^32.
__device__ __forceinline__ void load_quad_tile(const uint16_t* x, uint32_t rows, uint32_t cols, const QuadPos& p,
                                               uint4 (&v)[16]) {
    const uint16_t* base = x + (size_t)(16 * p.rb0) * cols;
    const uint64_t span = (uint64_t)(rows - 16 * p.rb0) * cols * 2;
    const uint32_t nrec = span > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)span;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, (int)nrec, 0x00020000);
    const uint32_t voff = p.s * 32u * cols + 2u * p.c8;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff, (int)(2u * k * cols), 0);
        v[k] = make_uint4(t.x, t.y, t.z, t.w);
    }
}

// LDS of the quad-mapped kernel: entry (wave, j, lane) first holds the Philox words of the lane's block j, then its
// codes (x, y); the scale codes go to sc[quad][column within the quarter][row-block]; cnt counts finished waves per
// quad.
struct QuadStash {
    uint4 e[kColRB][8 * 64 + 1];
    uint8_t sc[4][128][kColRB];
    uint32_t cnt[4];
};

// Writes quad q's 128 columns x nr row-blocks (one wave).  Codes: instruction t covers output rows 8 t .. 8 t + 7 of
// the quarter, 8 lanes per row, each lane 16 bytes = row-blocks 2 p and 2 p + 1.  Scales (unless scales is null):
// one lane per output row, 16 bytes.
__device__ __forceinline__ void quad_write_out(const QuadStash& st, const QuadPos& pos, uint32_t rows, uint32_t cols,
                                               uint32_t nrb, uint8_t* __restrict__ codes,
                                               uint8_t* __restrict__ scales) {
    const uint32_t col0 = pos.strip * 512 + 128 * pos.q;
    const uint32_t rbg = pos.group * kColRB;
    const uint32_t nr = min((uint32_t)kColRB, nrb - rbg);
    const uint32_t p = pos.lane & 7u, cl = pos.lane >> 3;
    const uint32_t wv = 4 * pos.q + (p >> 1), s0 = 2 * (p & 1u);   // slots of row-blocks 2p, 2p + 1
    const bool aligned16 = (rows & 31u) == 0;   // 16-byte stores need (rows / 2) % 16 == 0
#pragma unroll 4
    for (uint32_t t = 0; t < 16; ++t) {
        const uint32_t cc = 8 * t + cl, c = col0 + cc;
        if (c < cols && 2 * p < nr) {
            const uint32_t jj = cc & 7u, ln = cc >> 3;
            const uint4 a = st.e[wv][jj * 64 + 16 * s0 + ln];
            uint8_t* dst = codes + (size_t)c * (rows >> 1) + 8 * (size_t)(rbg + 2 * p);
            if (2 * p + 1 < nr) {
                const uint4 b = st.e[wv][jj * 64 + 16 * (s0 + 1) + ln];
                if (aligned16) {
                    st_nt(dst, make_uint4(a.x, a.y, b.x, b.y));
                } else {
                    st_nt(dst, make_uint2(a.x, a.y));
                    st_nt(dst + 8, make_uint2(b.x, b.y));
                }
            } else {
                st_nt(dst, make_uint2(a.x, a.y));
            }
        }
    }
    if (!scales) return;   // tiled scales: quad_write_scales_tiled
#pragma unroll
    for (uint32_t t = 0; t < 2; ++t) {
        const uint32_t cc = 64 * t + pos.lane, c = col0 + cc;
        if (c < cols) {
            uint8_t* dst = scales + (size_t)c * nrb + rbg;
            if (nr == kColRB && (nrb & 15u) == 0) {
                st_nt(dst, *reinterpret_cast<const uint4*>(&st.sc[pos.q][cc][0]));
            } else {
                for (uint32_t r = 0; r < nr; ++r) st_nt(dst + r, st.sc[pos.q][cc][r]);
            }
        }
    }
}

// The scale codes of quad q in the tiled layout of the FP4 GEMM (tiles of 128 rows x 4 scale columns, each a
// [32][4][4] byte array: byte 16 a + 4 b + c = row 32 b + a, scale column c; row-tile major; zero padding).  The
// quad's 128 columns of X are exactly the 128 rows of row tile col0 / 128 of V, and its 16 row-blocks the 4 tiles
// 4 group .. 4 group + 3 of that row tile, so the quad writes 2 KiB contiguously: lane l takes tile row
// a = l % 32 of tiles l / 32 and 2 + l / 32 (16 bytes: four 4-byte pieces of rows a, a + 32, a + 64, a + 96).
// Rows past cols and scale columns past nrb are written as zero.
__device__ __forceinline__ void quad_write_scales_tiled(const QuadStash& st, const QuadPos& pos, uint32_t cols,
                                                        uint32_t nrb, uint8_t* __restrict__ scales) {
    const uint32_t col0 = pos.strip * 512 + 128 * pos.q;
    if (col0 >= cols) return;
    const uint32_t nr = min((uint32_t)kColRB, nrb - pos.group * kColRB);
    const uint32_t bt = (nrb + 3) / 4;
    uint8_t* base = scales + ((size_t)(col0 / 128) * bt + 4 * pos.group) * 512;
#pragma unroll
    for (uint32_t t = 0; t < 2; ++t) {
        const uint32_t id = 64 * t + pos.lane, tb = id >> 5, a = id & 31u;
        if (4 * tb < nr) {
            const uint32_t keep = nr >= 4 * tb + 4 ? 0xFFFFFFFFu : (1u << (8 * (nr - 4 * tb))) - 1u;
            uint32_t w[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint32_t cc = 32 * b + a;
                w[b] = col0 + cc < cols ? *reinterpret_cast<const uint32_t*>(&st.sc[pos.q][cc][4 * tb]) & keep : 0u;
            }
            st_nt(base + (size_t)tb * 512 + 16 * a, make_uint4(w[0], w[1], w[2], w[3]));
        }
    }
}

template <int MODE, bool PER_ROW>
__global__ void __launch_bounds__(kColThreads)
k_quant_colwise(const uint16_t* __restrict__ x, uint32_t rows, uint32_t cols, ColGrid cg,
                const float* __restrict__ amax, uint32_t sign_mask, RngArgs rng, uint8_t* __restrict__ codes,
                uint8_t* __restrict__ scales, float* __restrict__ gout, uint32_t tiled) {
    constexpr bool SR = MODE != kRN;
    constexpr bool RHT = MODE == kRHTSR;
    __shared__ QuadStash st;
    __shared__ RTable tab;
    if (threadIdx.x < 4) st.cnt[threadIdx.x] = 0;
    float g = 0.0f;
    Divisor d6{};
    if (!PER_ROW) {
        g = global_scale(amax[0]);
        d6 = make_divisor_uniform(6.0f * g);
        if (blockIdx.x == 0 && threadIdx.x == 0) gout[0] = g;
        fill_rtable<RHT>(tab, g);   // its barrier also orders the counters' reset
    } else {
        __syncthreads();
    }
    const QuadPos pos = quad_position(cg, blockIdx.x);
    const uint32_t wave = threadIdx.x >> 6;
    if (pos.rb < cg.nrb && pos.c8 < cols) {
        uint4 v[16];
        load_quad_tile(x, rows, cols, pos, v);
        // The random words do not depend on the data: they are generated while the loads are in flight and parked
        // in LDS (registers are full with the tile).
        if (SR) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const Rand4 r = block_rand_inv(rng, (pos.c8 + j) * cg.nrb + pos.rb);
                st.e[wave][j * 64 + pos.lane] = make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]);
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint4& slot = st.e[wave][j * 64 + pos.lane];
            Rand4 inv{{0, 0, 0, 0}};
            if (SR) {
                const uint4 r = slot;
                inv = Rand4{{r.x, r.y, r.z, r.w}};
            }
            float w[16];
            widen_col_block<RHT>(v, j, sign_mask, w);
            uint32_t lo, hi, sb;
            if (PER_ROW) {
                const uint32_t c = pos.c8 + j;
                const float gr = global_scale(amax[c]);
                if (pos.rb == 0) gout[c] = gr;
                quantize_block<SR, RHT>(w, make_divisor(6.0f * gr), RowMul<RHT>{gr}, inv, lo, hi, sb);
            } else {
                quantize_block<SR, RHT>(w, d6, TableMul{tab}, inv, lo, hi, sb);
            }
            slot = make_uint4(lo, hi, 0u, 0u);
            st.sc[pos.q][8 * (pos.lane & 15u) + j][4 * pos.i + pos.s] = (uint8_t)sb;
            if (j & 1) __builtin_amdgcn_sched_barrier(0);   // two blocks at a time bounds the live registers
        }
    }
    // Every wave counts itself in (active or not); the last of the quad writes the quad's output.  The release half
    // of the atomic orders this wave's LDS writes before it, the acquire half the writer's reads after it.
    uint32_t before = 0;
    if (pos.lane == 0)
        before = __hip_atomic_fetch_add(&st.cnt[pos.q], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (__builtin_amdgcn_readfirstlane(before) == 3) {
        quad_write_out(st, pos, rows, cols, cg.nrb, codes, tiled ? nullptr : scales);
        if (tiled) quad_write_scales_tiled(st, pos, cols, cg.nrb, scales);
    }
}

// ------------------------------------------------------------------------------------------------------------
// Column-wise kernels with narrow lane tiles: a lane holds 16 rows x 4 columns (16 loads of 8 bytes, 32 VGPRs) and
// a 1024-thread workgroup 16 row-blocks x 256 columns (wave w = row-block w), so that two workgroups fit on a CU: 8
// waves per SIMD instead of 4.  The VALU work per element is the same, but twice the waves are there to issue it
// while others wait for memory, and each wave's share (4 blocks) is half as long, which shortens the tail after
// the last data arrives.  At 8192 x 4096 the 512 workgroups are all resident at once.  Codes and scales are staged
// in LDS and written per output row of X^T: 128 contiguous bytes of codes (16 row-blocks) and 16 of scales.
// ------------------------------------------------------------------------------------------------------------
constexpr uint32_t kStrip4 = 256;   // columns of X per narrow workgroup tile

struct Col4Pos {
    uint32_t group;  // row group (16 row-blocks)
    uint32_t strip;  // 256-column strip
    uint32_t rb;     // this wave's row-block
    uint32_t lane;
    uint32_t c4;     // first of the lane's 4 columns
};

// Workgroup b -> (row group, strip), strip-fastest with the strip rotated by the row group (every XCD reads every
// strip); ns divides by the strip count (uniform values, so the divisions stay on the scalar unit).  octets: the 8 row groups 8 o .. 8 o + 7 of a strip go to one XCD (workgroups are dealt to the 8 XCDs in
// turn), so that their 16-byte pieces of each row-major scale row meet in one L2 as whole lines; needs whole
// octets and a multiple of 8 (octet, strip) pairs, else the usual order.
// n / d for a uniform n (scalar unit): the multiply-high of FastDiv on 64-bit scalar arithmetic.
__device__ __forceinline__ uint32_t sfdiv(uint32_t n, const FastDiv& f) {
    n = __builtin_amdgcn_readfirstlane(n);
    return __builtin_amdgcn_readfirstlane((uint32_t)((((uint64_t)n * f.m >> 32) + n) >> f.s));
}

__device__ __forceinline__ Col4Pos col4_at(uint32_t group, uint32_t strip) {
    Col4Pos p;
    p.group = group;
    p.strip = strip;
    p.rb = group * kColRB + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    p.lane = threadIdx.x & 63u;
    p.c4 = strip * kStrip4 + 4 * p.lane;
    return p;
}

__device__ __forceinline__ Col4Pos col4_position(uint32_t nrb, const FastDiv& ns, uint32_t b, bool octets) {
    const uint32_t nstrips = ns.d;
    const uint32_t ngroups = (nrb + kColRB - 1) / kColRB;
    const uint32_t pairs = (ngroups / 8) * nstrips;
    uint32_t group, strip;
    b = __builtin_amdgcn_readfirstlane(b);
    if (octets && (ngroups & 7u) == 0 && (pairs & 7u) == 0) {
        const uint32_t x = b & 7u, i = b >> 3;
        const uint32_t pr = (i >> 3) * 8 + x, o = sfdiv(pr, ns);
        group = 8 * o + (i & 7u);
        strip = pr - o * nstrips;
    } else {
        group = sfdiv(b, ns);
        const uint32_t s = b - group * nstrips + (group - sfdiv(group, ns) * nstrips);
        strip = s >= nstrips ? s - nstrips : s;
    }
    return col4_at(__builtin_amdgcn_readfirstlane(group), __builtin_amdgcn_readfirstlane(strip));
}

// The lane's 16 rows x 4 columns: v[k] = row k of the wave's row-block, columns c4 .. c4 + 3 (cols % 4 == 0).  A
// buffer resource over the row-block: one 32-bit lane offset, the row offset in a scalar.
__device__ __forceinline__ void load_col4_tile(const uint16_t* x, uint32_t cols, const Col4Pos& p, uint2 (&v)[16]) {
    const uint16_t* base = x + (size_t)(16 * p.rb) * cols;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, (int)(32u * cols), 0x00020000);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)(2u * p.c4), (int)(2u * k * cols), 0);
        v[k] = make_uint2(t.x, t.y);
    }
}

// Column j (0..3) of the lane's 16 x 4 tile -> the 16 values of its column block (sign-flipped and transformed with
// RHT).
template <bool RHT>
__device__ __forceinline__ void widen_col4_block(const uint2 (&v)[16], int j, uint32_t mask, float (&w)[16]) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const uint32_t word = (j >> 1) ? v[k].y : v[k].x;
        const uint32_t f = RHT ? flip_bit(mask, k) : 0u;
        w[k] = (j & 1) ? bf16_hi(word, f) : bf16_lo(word, f);
    }
    if (RHT) fwht16(w);
}

// The random signs applied to the packed words of a lane's tile: row k of a column block is element k, so both
// halves of the words of row k are negated where bit k of mask is set (exact sign-bit flips).
__device__ __forceinline__ void flip_col4_tile(uint2 (&v)[16], uint32_t mask) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const uint32_t f = ((mask >> k) & 1u) ? 0x80008000u : 0u;
        v[k].x ^= f;
        v[k].y ^= f;
        asm volatile("" : "+v"(v[k].x), "+v"(v[k].y));   // the flipped words replace the loaded ones
    }
}

// LDS of a narrow column-wise workgroup: entry (wave, j, lane) first holds the Philox words of the lane's block j,
// then its codes (x, y) and scale (z).  A wave's region is padded by one entry.
struct Col4Stash {
    uint4 e[kColRB][4 * 64 + 1];
};

__device__ __forceinline__ const uint4& col4_entry(const Col4Stash& st, uint32_t rbl, uint32_t cl) {
    return st.e[rbl][(cl & 3u) * 64 + (cl >> 2)];   // column cl (0..255) of the strip = block cl % 4 of lane cl / 4
}

// Writes the workgroup's staged codes: thread t takes column 128 r + t / 8 of the strip (r = 0, 1) and row-blocks
// 2 (t % 8), 2 (t % 8) + 1, so 8 consecutive threads write one output row's 128 contiguous bytes.
__device__ __forceinline__ void col4_write_codes(const Col4Stash& st, const Col4Pos& p, uint32_t rows, uint32_t cols,
                                                 uint32_t nrb, uint8_t* __restrict__ codes) {
    const uint32_t nr = min((uint32_t)kColRB, nrb - p.group * kColRB);
    const uint32_t q = threadIdx.x & 7u, rb0 = p.group * kColRB + 2 * q;
    const bool aligned16 = (rows & 31u) == 0;   // 16-byte stores need (rows / 2) % 16 == 0
#pragma unroll
    for (uint32_t r = 0; r < 2; ++r) {
        const uint32_t cl = 128 * r + (threadIdx.x >> 3), c = p.strip * kStrip4 + cl;
        if (c < cols && 2 * q < nr) {
            const uint4 a = col4_entry(st, 2 * q, cl);
            uint8_t* dst = codes + (size_t)c * (rows >> 1) + 8 * (size_t)rb0;
            if (2 * q + 1 < nr) {
                const uint4 b = col4_entry(st, 2 * q + 1, cl);
                if (aligned16) {
                    st_nt(dst, make_uint4(a.x, a.y, b.x, b.y));
                } else {
                    st_nt(dst, make_uint2(a.x, a.y));
                    st_nt(dst + 8, make_uint2(b.x, b.y));
                }
            } else {
                st_nt(dst, make_uint2(a.x, a.y));
            }
        }
    }
}

// The workgroup's scale codes, row-major: thread t < 256 writes the 16 bytes (row-blocks of the group) of output row
// strip * 256 + t with one store when they form a whole aligned 16-byte piece, byte by byte otherwise.  The 16-byte
// stores are ordinary (cached) ones, so that the pieces of an octet's row groups (one XCD) meet in L2 as whole lines.
__device__ __forceinline__ void col4_write_scales_rows(const Col4Stash& st, const Col4Pos& p, uint32_t cols,
                                                       uint32_t nrb, uint8_t* __restrict__ scales) {
    if (threadIdx.x >= kStrip4) return;
    const uint32_t cl = threadIdx.x, c = p.strip * kStrip4 + cl;
    if (c >= cols) return;
    const uint32_t nr = min((uint32_t)kColRB, nrb - p.group * kColRB);
    uint8_t* dst = scales + (size_t)c * nrb + p.group * kColRB;
    if (nr == kColRB && (nrb & 15u) == 0) {
        uint32_t w[4];
#pragma unroll
        for (uint32_t q = 0; q < 4; ++q) {
            w[q] = 0;
#pragma unroll
            for (uint32_t k = 0; k < 4; ++k) w[q] |= (col4_entry(st, 4 * q + k, cl).z & 0xFFu) << (8 * k);
        }
        *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
        for (uint32_t r = 0; r < nr; ++r) st_nt(dst + r, (uint8_t)col4_entry(st, r, cl).z);
    }
}

// The workgroup's scale codes in the tiled layout of the FP4 GEMM: its 256 columns of X are 2 row tiles of V and its
// 16 row-blocks 4 scale-column tiles; thread t < 256 takes tile row a = t % 32 of tile (t / 128, (t / 32) % 4).
// Rows past cols and scale columns past nrb are written as zero.
__device__ __forceinline__ void col4_write_scales_tiled(const Col4Stash& st, const Col4Pos& p, uint32_t cols,
                                                        uint32_t nrb, uint8_t* __restrict__ scales) {
    if (threadIdx.x >= kStrip4) return;
    const uint32_t rt = threadIdx.x >> 7, tb = (threadIdx.x >> 5) & 3u, a = threadIdx.x & 31u;
    const uint32_t col0 = p.strip * kStrip4 + 128 * rt;
    const uint32_t nr = min((uint32_t)kColRB, nrb - p.group * kColRB);
    if (col0 >= cols || 4 * tb >= nr) return;
    const uint32_t bt = (nrb + 3) / 4;
    uint32_t w[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t cl = 128 * rt + 32 * b + a;
        w[b] = 0;
        if (p.strip * kStrip4 + cl < cols) {
#pragma unroll
            for (uint32_t c = 0; c < 4; ++c)
                if (4 * tb + c < nr) w[b] |= (col4_entry(st, 4 * tb + c, cl).z & 0xFFu) << (8 * c);
        }
    }
    st_nt(scales + ((size_t)(col0 / 128) * bt + 4 * p.group + tb) * 512 + 16 * a, make_uint4(w[0], w[1], w[2], w[3]));
}

// Column-wise quantization with a device-resident per-tensor amax, narrow lane tiles (cols % 4 == 0).  The Philox
// words are generated while the loads are in flight and parked in LDS; each block's codes and scale replace its
// words; after one workgroup barrier the output rows are written.  (Per-row g needs two divisions per block, whose
// temporaries do not fit the 64 registers; it keeps the wide-tile kernel.)
template <int MODE>
__global__ void __launch_bounds__(kColThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
k_quant_colwise4(const uint16_t* __restrict__ x, uint32_t rows, uint32_t cols, uint32_t nrb, FastDiv ns,
                 const float* __restrict__ amax, uint32_t sign_mask, RngArgs rng, uint8_t* __restrict__ codes,
                 uint8_t* __restrict__ scales, float* __restrict__ gout, uint32_t tiled) {
    constexpr bool SR = MODE != kRN;
    constexpr bool RHT = MODE == kRHTSR;
    __shared__ Col4Stash st;
    __shared__ RTable tab;
    const Col4Pos pos = col4_position(nrb, ns, blockIdx.x, !tiled);
    const uint32_t wave = threadIdx.x >> 6;
    const bool active = pos.rb < nrb && pos.c4 < cols;
    uint2 v[16];
    // RN: the tile's loads go out before the amax read and the table fill (19.3 -> 18.1 us at 8192 x 4096); with SR
    // they follow the table and the Philox words are generated while they are in flight (loads first measured 0.9 us
    // slower there)
    if (!SR && active) load_col4_tile(x, cols, pos, v);
    const float g = global_scale(amax[0]);
    const Divisor d6 = make_divisor_uniform(6.0f * g);
    if (blockIdx.x == 0 && threadIdx.x == 0) gout[0] = g;
    fill_rtable<RHT>(tab, g);
    if (active) {
        if (SR) load_col4_tile(x, cols, pos, v);
        if (SR) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const Rand4 r = block_rand_inv(rng, (pos.c4 + j) * nrb + pos.rb);
                st.e[wave][j * 64 + pos.lane] = make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]);
                __builtin_amdgcn_sched_barrier(0);   // one call at a time: the tile's registers are in flight
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint4& slot = st.e[wave][j * 64 + pos.lane];
            const LdsRand inv{&slot};
            float w[16];
            widen_col4_block<RHT>(v, j, sign_mask, w);
            uint32_t lo, hi, sb;
            quantize_block<SR, RHT>(w, d6, TableMul{tab}, inv, lo, hi, sb);
            slot = make_uint4(lo, hi, sb, 0u);
            __builtin_amdgcn_sched_barrier(0);   // one block at a time bounds the live registers
        }
    }
    __syncthreads();
    col4_write_codes(st, pos, rows, cols, nrb, codes);
    if (tiled) col4_write_scales_tiled(st, pos, cols, nrb, scales);
    else col4_write_scales_rows(st, pos, cols, nrb, scales);
}

// ------------------------------------------------------------------------------------------------------------
// Single-read amax + column-wise 1x16 quantization of a tensor that the chip can hold: every workgroup keeps its
// tile in registers, publishes its tile maximum in a slot of its own, waits until every workgroup has published,
// reduces the slots to the tensor amax and quantizes the tile it still holds.  The tensor is read from HBM once
// instead of twice.
//   The exchange.  Every launch carries a nonzero 32-bit tag (its epoch, from a host counter) and uses slot region
// epoch % kSlotRegions; workgroup b owns slot b of the region, written to kSlotCopies copies.  A slot holds 0 or
// (epoch << 32) | v, where v = kArrived once the workgroup has started and v = its tile maximum (magnitude bits,
// <= 0x7FFFFFFF) once that is known.  Readers take only values that carry their own epoch: a slot holding another
// launch's value (a launch sharing the region, or a stale one) reads as absent, never as a maximum.
//   The wait is bounded twice: once arrive_ticks have passed with some slot still absent (its workgroup has not
// started, so not every workgroup is resident at once), or once wait_ticks have passed in any case, the workgroup
// stops waiting and computes the maxima of the tiles it has not seen from the tensor itself (the slow route).  The
// result is the same on every route; only the time changes.
//   Each workgroup clears its slot as its last action with a compare-and-swap of its own value, so a slot taken over
// by another launch keeps that launch's value, and launches that follow one another (replays of a captured graph
// repeat their epoch) find the region clear.
//   Workgroup b polls copy b % kSlotCopies: with one copy, every workgroup polls the same few cache lines while it
// waits for the last one, and those reads queue behind each other (the exchange then took ~2.5 us against a one-way
// latency of ~0.6 us between XCDs).
// ------------------------------------------------------------------------------------------------------------
constexpr uint32_t kFusedMaxGrid = 2048;
constexpr uint32_t kSlotCopies = 16;
constexpr uint32_t kSlotRegions = 8;
constexpr uint32_t kSlotsPerRegion = kSlotCopies * kFusedMaxGrid;
constexpr uint32_t kArrived = 0xFFFFFFFFu;     // low word of a slot whose workgroup has started
// Wait bounds in ticks of the 100 MHz wall clock.  At 8192 x 4096 the last workgroup publishes ~16 us after the
// launch and the exchange completes within ~2 us of that; a workgroup starts waiting only after its own loads, by
// which time every co-resident workgroup has long started.
constexpr uint64_t kWaitTicks = 200000;        // 2 ms: the whole wait
constexpr uint64_t kArriveTicks = 10000;       // 100 us: the wait for workgroups that have not started

// The exchange slots of every single-read launch on a GPU (2 MiB): region r, copy c, slot b at
// scratch[r * kSlotsPerRegion + c * kFusedMaxGrid + b].  Host code hands its device address (hipGetSymbolAddress,
// once per device) to the kernels.
static __device__ __align__(256) uint64_t scratch[kSlotRegions * kSlotsPerRegion];

struct Exchange {
    uint64_t* region;        // this launch's slot region: kSlotCopies copies of kFusedMaxGrid slots
    uint32_t epoch;          // the launch's tag, nonzero
    uint32_t pad;
    uint64_t wait_ticks;     // bound of the whole wait
    uint64_t arrive_ticks;   // bound of the wait while some workgroup has not started
};

__device__ __forceinline__ uint64_t* slot_copy(const Exchange& ex, uint32_t copy) {
    return ex.region + (size_t)copy * kFusedMaxGrid;
}

// Copy `copy` of this workgroup's own slot (the workgroup index taken as a scalar, so that the address stays a
// scalar base plus the lane's copy offset).
__device__ __forceinline__ uint64_t* own_slot(const Exchange& ex, uint32_t copy) {
    return ex.region + __builtin_amdgcn_readfirstlane(blockIdx.x) + (size_t)copy * kFusedMaxGrid;
}

// The first action of a single-read kernel: this workgroup's slot says it has started.
__device__ __forceinline__ void announce(const Exchange& ex) {
    if (threadIdx.x < kSlotCopies)
        __hip_atomic_store(own_slot(ex, threadIdx.x), ((uint64_t)ex.epoch << 32) | kArrived, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// The cross-workgroup step of the single-read kernels (1024-thread workgroups).  The workgroup maximum of mbits
// (magnitude bits) goes to this workgroup's slot (kept in s_own for release_slot), and wave 0 then reads the
// slots of every workgroup (lane l watches slots l + 64 k, up to eight loads in flight together: each read is a round
// trip to memory, since the slots are shared by all XCDs; a slot once seen with its maximum is not read again),
// reduces them and, when none is missing, fills tab for g = amax / 2688, while the other waves wait at the one
// barrier that follows.  Returns the maximum over the slots seen, equal in every thread; missing[l] (l < 64) gets
// bit k set for each slot l + 64 k not seen, and nmissing (uniform) is nonzero if any is (then tab is not filled).  Uses
// red[16].
template <bool RHT>
__device__ uint32_t exchange_max(uint32_t mbits, const Exchange& ex, uint32_t* red, uint32_t* missing,
                                 uint32_t* s_own, RTable& tab, uint32_t& nmissing) {
    __shared__ uint32_t s_max, s_nmiss;
    const uint32_t lane = threadIdx.x & 63u;
    mbits = wave_max(mbits);
    if (lane == 0) red[threadIdx.x >> 6] = mbits;
    __syncthreads();
    uint32_t m = 0;
    if (threadIdx.x < 64) {
        m = wave_max(lane < kColRB ? red[lane] : 0u);
        if (lane == 0) *s_own = m;
        if (lane < kSlotCopies)
            __hip_atomic_store(own_slot(ex, lane), ((uint64_t)ex.epoch << 32) | m, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    if (threadIdx.x < 64) {
        const uint64_t* copy = slot_copy(ex, __builtin_amdgcn_readfirstlane(blockIdx.x) % kSlotCopies);
        const uint32_t nk = (gridDim.x + 63) / 64;   // slots per lane, <= 32
        uint32_t pending = 0, absent = 0;            // bit k: slot lane + 64 k not seen yet / last read foreign
        for (uint32_t k = 0; k < nk; ++k)
            if (lane + 64 * k < gridDim.x) pending |= 1u << k;
        m = 0;
        const uint64_t t0 = wall_clock64();
        while (true) {
            for (uint32_t k0 = 0; k0 < nk; k0 += 8) {
                uint64_t sv[8];
#pragma unroll
                for (uint32_t kk = 0; kk < 8; ++kk) {
                    const uint32_t k = k0 + kk;
                    sv[kk] = (k < nk && ((pending >> k) & 1u))
                                 ? __hip_atomic_load(&copy[lane + 64 * k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                 : 0ull;
                }
#pragma unroll
                for (uint32_t kk = 0; kk < 8; ++kk) {
                    const uint32_t k = k0 + kk;
                    if (k < nk && ((pending >> k) & 1u)) {
                        const bool ours = (uint32_t)(sv[kk] >> 32) == ex.epoch;
                        const uint32_t v = (uint32_t)sv[kk];
                        absent = ours ? absent & ~(1u << k) : absent | (1u << k);
                        if (ours && v != kArrived) {
                            m = umax(m, v);
                            pending &= ~(1u << k);
                        }
                    }
                }
            }
            if (__ballot(pending != 0) == 0) break;
            const uint64_t dt = wall_clock64() - t0;
            if (dt >= ex.wait_ticks || (dt >= ex.arrive_ticks && __ballot(absent != 0) != 0)) break;
            __builtin_amdgcn_s_sleep(1);
        }
        m = wave_max(m);
        missing[lane] = pending;
        const uint32_t cnt = __ballot(pending != 0) != 0 ? 1u : 0u;   // whether any slot is missing
        if (cnt == 0) {
            const float g = global_scale(as_f(m));
#pragma unroll 1
            for (uint32_t c = lane; c < 128; c += 64) fill_rtable_entry<RHT>(tab, c, g);
        }
        if (lane == 0) {
            s_max = m;
            s_nmiss = cnt;
        }
    }
    __syncthreads();
    nmissing = __builtin_amdgcn_readfirstlane(s_nmiss);
    return __builtin_amdgcn_readfirstlane(s_max);
}

// Whether slot s was missing in the exchange (missing as written by exchange_max).
__device__ __forceinline__ bool slot_missing(const uint32_t* missing, uint32_t s) {
    return (missing[s & 63u] >> (s >> 6)) & 1u;
}

// Clears this workgroup's slot if it still holds this launch's value: the last action of a single-read kernel
// (every other workgroup of the launch has read the slot by then, or has stopped waiting and taken the slow route).
__device__ __forceinline__ void release_slot(const Exchange& ex, uint32_t own) {
    uint32_t copy = threadIdx.x;
    asm volatile("" : "+v"(copy));   // formed here, not kept in a register from the start of the kernel
    if (copy < kSlotCopies) {
        uint64_t expect = ((uint64_t)ex.epoch << 32) | own;
        __hip_atomic_compare_exchange_strong(own_slot(ex, copy), &expect, 0ull, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ------------------------------------------------------------------------------------------------------------
// Single-read amax + column-wise quantization with narrow lane tiles (16 rows x 4 columns per lane, cols % 4 == 0):
// two 1024-thread workgroups per CU, 8 waves per SIMD, so a tensor of up to 512 tiles of 16 row-blocks x 256 columns
// (8192 x 4096 on MI355X) stays in registers.  Phase 2 is bound by VALU issue, which twice the waves per SIMD issue
// faster; the block maxima are recomputed there (six instructions per block) rather than held in registers.
// The codes of each column block leave after a barrier of their own, so their stores overlap the next block's
// arithmetic; the scales leave at the end.
template <bool RHT>
__device__ uint32_t tile_max_col4(const uint16_t* x, uint32_t cols, uint32_t nrb, const FastDiv& ns, uint32_t t,
                                  bool tiled, uint32_t sign_mask, uint2 (&v)[16]) {
    const Col4Pos p = col4_position(nrb, ns, t, !tiled);
    uint32_t m = 0;
    if (p.rb < nrb && p.c4 < cols) {
        load_col4_tile(x, cols, p, v);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float w[16];
            widen_col4_block<RHT>(v, j, sign_mask, w);
            const float bmax = absmax16(w);
            m = umax(m, as_u(RHT ? 0.25f * bmax : bmax) & 0x7FFFFFFFu);
        }
    }
    return m;
}

// The staged codes of column block j of every lane: output rows strip * 256 + 4 l + j for l < 64; threads 0..511,
// 8 consecutive threads per output row, write its 16 row-blocks (128 contiguous bytes).
__device__ __forceinline__ void col4_write_codes_block(const Col4Stash& st, const Col4Pos& p, uint32_t rows,
                                                       uint32_t cols, uint32_t nrb, uint32_t j,
                                                       uint8_t* __restrict__ codes) {
    if (threadIdx.x >= 512) return;
    const uint32_t nr = min((uint32_t)kColRB, nrb - p.group * kColRB);
    const uint32_t q = threadIdx.x & 7u, rb0 = p.group * kColRB + 2 * q;
    const uint32_t cl = 4 * (threadIdx.x >> 3) + j, c = p.strip * kStrip4 + cl;
    if (c >= cols || 2 * q >= nr) return;
    const uint4 a = col4_entry(st, 2 * q, cl);
    uint8_t* dst = codes + (size_t)c * (rows >> 1) + 8 * (size_t)rb0;
    if (2 * q + 1 < nr) {
        const uint4 b = col4_entry(st, 2 * q + 1, cl);
        if ((rows & 31u) == 0) {
            st_nt(dst, make_uint4(a.x, a.y, b.x, b.y));
        } else {
            st_nt(dst, make_uint2(a.x, a.y));
            st_nt(dst + 8, make_uint2(b.x, b.y));
        }
    } else {
        st_nt(dst, make_uint2(a.x, a.y));
    }
}

template <int MODE>
__global__ void __launch_bounds__(kColThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
k_amax_quant_colwise4(const uint16_t* __restrict__ x, uint32_t rows, uint32_t cols, uint32_t nrb, FastDiv ns,
                      uint32_t sign_mask, RngArgs rng, float* __restrict__ amax_out, uint8_t* __restrict__ codes,
                      uint8_t* __restrict__ scales, float* __restrict__ gout, Exchange ex, uint32_t tiled) {
    constexpr bool SR = MODE != kRN;
    constexpr bool RHT = MODE == kRHTSR;
    __shared__ Col4Stash st;
    __shared__ RTable tab;
    __shared__ uint32_t red[kColRB], missing[64], s_own;
    announce(ex);
    const Col4Pos pos = col4_position(nrb, ns, blockIdx.x, !tiled);
    const uint32_t wave = threadIdx.x >> 6;
    const bool active = pos.rb < nrb && pos.c4 < cols;
    uint2 v[16];
    uint32_t mbits = 0;
    if (active) {
        load_col4_tile(x, cols, pos, v);
        // the random words of the 4 blocks, generated while the loads are in flight (the vector unit is idle then)
        // and parked in LDS; generated later, between publishing and polling, they delayed the last workgroups'
        // publication and so every workgroup's wait
        if (SR) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const Rand4 r = block_rand_inv(rng, (pos.c4 + j) * nrb + pos.rb);
                st.e[wave][j * 64 + pos.lane] = make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]);
                __builtin_amdgcn_sched_barrier(0);   // one call at a time: the tile's registers are in flight
            }
        }
        if (RHT) flip_col4_tile(v, sign_mask);   // the random signs once, on the packed words
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float w[16];
            widen_col4_block<RHT>(v, j, 0u, w);
            const float bmax = absmax16(w);
            mbits = umax(mbits, as_u(RHT ? 0.25f * bmax : bmax) & 0x7FFFFFFFu);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // the tile stays in registers: keep the compiler from carrying widened values over the wait instead
#pragma unroll
    for (int k = 0; k < 16; ++k) asm volatile("" : "+v"(v[k].x), "+v"(v[k].y));
    uint32_t nmiss;
    uint32_t abits = exchange_max<RHT>(mbits, ex, red, missing, &s_own, tab, nmiss);
    if (nmiss) {
        // slow route: the maxima of the tiles whose slots were not seen, from the tensor, then the own tile again
        __shared__ uint32_t s_bits;
        uint32_t mm = 0;
        for (uint32_t t = 0; t < gridDim.x; ++t)
            if (slot_missing(missing, t)) mm = umax(mm, tile_max_col4<RHT>(x, cols, nrb, ns, t, tiled, sign_mask, v));
        mm = block_max<kColRB>(mm, red);
        if (threadIdx.x == 0) s_bits = umax(mm, abits);
        if (active) {
            load_col4_tile(x, cols, col4_at(pos.group, pos.strip), v);
            if (RHT) flip_col4_tile(v, sign_mask);
#pragma unroll
            for (int k = 0; k < 16; ++k) asm volatile("" : "+v"(v[k].x), "+v"(v[k].y));
        }
        __syncthreads();
        abits = __builtin_amdgcn_readfirstlane(s_bits);
        fill_rtable<RHT>(tab, global_scale(as_f(abits)));
    }
    const float amax = as_f(abits);
    const float g = global_scale(amax);
    const Divisor d6 = make_divisor_uniform(6.0f * g);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        amax_out[0] = amax;
        gout[0] = g;
    }
    uint32_t ln = threadIdx.x & 63u;
    asm volatile("" : "+v"(ln));   // formed after the wait, not held across it
    // the codes of each column block leave after a barrier, so their stores overlap the next block's arithmetic
    // (28.5 against 29.1 us at 8192 x 4096 RHT+SR with two groups of two blocks)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (active) {
            uint4& slot = st.e[wave][j * 64 + ln];
            const LdsRand inv{&slot};
            float w[16];
            widen_col4_block<RHT>(v, j, 0u, w);   // signs already applied
            uint32_t lo, hi, sb;
            quantize_block<SR, RHT>(w, d6, TableMul{tab}, inv, lo, hi, sb);
            slot = make_uint4(lo, hi, sb, 0u);
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        col4_write_codes_block(st, col4_at(pos.group, pos.strip), rows, cols, nrb, j, codes);
    }
    const Col4Pos wp = col4_at(pos.group, pos.strip);
    if (tiled) col4_write_scales_tiled(st, wp, cols, nrb, scales);
    else col4_write_scales_rows(st, wp, cols, nrb, scales);
    release_slot(ex, s_own);
}

// ------------------------------------------------------------------------------------------------------------
// 16x16 RN quantization, W and/or W^T from one read ([P2, intro: 2D weight scaling; results: both weight
// orientations]).  Same workgroup layout as the column-wise kernels (a step is one tile-row of 16 rows, lane = 8
// columns); lane pair (2m, 2m+1) holds the two halves of a 16x16 tile, whose amax is the max over the pair (both
// lanes of a pair always take the same steps).  W rows are written directly (consecutive lanes write consecutive
// 4-byte pieces of a row); W^T is staged in LDS like the column-wise codes.
// ------------------------------------------------------------------------------------------------------------
// Transposes an 8 x 8 matrix of nibbles held as 8 words (word k = row k, nibble c = column c): afterwards word c
// holds column c (nibble k = row k).  Three exchange stages between word pairs: 4 x 4 blocks (16-bit halves of words
// k, k + 4) and 2 x 2 blocks (bytes of words k, k + 2) by byte permutes, then single nibbles of words k, k + 1 by
// bit-field inserts.
__device__ __forceinline__ void transpose8x8_nibbles(uint32_t (&a)[8]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t x = a[k], y = a[k + 4];
        a[k] = __builtin_amdgcn_perm(y, x, 0x05040100u);       // x bytes 0, 1; y bytes 0, 1
        a[k + 4] = __builtin_amdgcn_perm(y, x, 0x07060302u);   // x bytes 2, 3; y bytes 2, 3
    }
#pragma unroll
    for (int k : {0, 1, 4, 5}) {
        const uint32_t x = a[k], y = a[k + 2];
        a[k] = __builtin_amdgcn_perm(y, x, 0x06020400u);       // x byte 0, y byte 0, x byte 2, y byte 2
        a[k + 2] = __builtin_amdgcn_perm(y, x, 0x07030501u);   // x byte 1, y byte 1, x byte 3, y byte 3
    }
    constexpr uint32_t lo = 0x0F0F0F0Fu;
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
        const uint32_t x = a[k], y = a[k + 1];
        a[k] = (x & lo) | ((y << 4) & ~lo);
        a[k + 1] = ((x >> 4) & lo) | (y & ~lo);
    }
}

template <bool WANT_W, bool WANT_WT, int RB>
__global__ void __launch_bounds__(64 * RB)
k_quant_16x16(const uint16_t* __restrict__ x, uint32_t rows, uint32_t cols, ColGrid cg,
              const float* __restrict__ amax, uint8_t* __restrict__ cw_codes, uint8_t* __restrict__ sw,
              float* __restrict__ gw, uint8_t* __restrict__ ct, uint8_t* __restrict__ st_scales,
              float* __restrict__ gt) {
    __shared__ ColStage<RB> st;
    __shared__ RTable tab;
    // Workgroups loop over the tiles (grid-stride); the next tile's loads are issued before the current tile's
    // W^T write-out, so reading overlaps writing, and the first tile's before the amax read and the table fill
    // (43.5 -> 41.7 us at 14336 x 4096).  Lanes of a pair own the two halves of one 16x16 tile, so both exist or
    // neither (cols is a multiple of 16).  Each wave writes its W codes and W scale rows; the W^T codes and scale rows
    // leave after the item's barrier.
    static_assert(WANT_WT, "W alone takes the band kernel");
    uint32_t tile = blockIdx.x;
    ColPos pos = col_position<RB>(cg, tile);
    bool have = tile < cg.ntiles && pos.rb < cg.nrb && pos.c8 < cols;
    uint4 v[16];
    if (have) load_col_tile(x, cols, pos, v);
    const float g = global_scale(amax[0]);
    const Divisor d6 = make_divisor_uniform(6.0f * g);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (WANT_W) gw[0] = g;
        if (WANT_WT) gt[0] = g;
    }
    fill_rtable<false>(tab, g);
    while (tile < cg.ntiles) {
    const uint32_t lane = pos.lane, h = lane & 1u, c8 = pos.c8, ti = pos.rb;
    if (have) {
        // Maximum magnitude of the lane's 128 inputs on the bf16 bit patterns (packed 16-bit integer maxima of
        // the magnitude bits: NaN > inf > finite, as for the binary32 values they widen to exactly).
        u16x2 mb = {0, 0};
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const uint32_t ws[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) mb = __builtin_elementwise_max(mb, __builtin_bit_cast(u16x2, ws[q] & 0x7FFF7FFFu));
        }
        float m = as_f((uint32_t)(mb.x > mb.y ? mb.x : mb.y) << 16);
        m = __builtin_elementwise_maximum(m, __shfl_xor(m, 1));
        const uint32_t sb = scale_code(m, d6);
        const float r = tab.r[sb];
        const bool fast = tab.rq[sb] == tab.rq[sb];   // see fast_multiplier
        // Every product is converted once: column pair (2p, 2p+1) gives byte p of every W row; the W^T codes are
        // the W codes transposed (two 8 x 8 nibble transposes), not a second conversion.
        uint32_t rowc[16];
        const uint32_t rbl = ti - pos.group * RB;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {   // rows 8 half .. 8 half + 7
                float qa[8], qb[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint4& row = v[8 * half + i];
                    const uint32_t word = p == 0 ? row.x : p == 1 ? row.y : p == 2 ? row.z : row.w;
                    qa[i] = bf16_lo(word, 0u) * r;
                    qb[i] = bf16_hi(word, 0u) * r;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    rowc[8 * half + i] = cvt_fp4_byte(p, p == 0 ? 0u : rowc[8 * half + i], qa[i], qb[i]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (!fast) [[unlikely]] {
            // NaN multiplier (NaN amax) or a degenerate scale: NaN products get code 0x7.  The tile is read again
            // so that the registers of the common path can be released as it goes.
            load_col_tile(x, cols, pos, v);
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const uint32_t ws[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
                float q[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) q[j] = ((j & 1) ? bf16_hi(ws[j >> 1], 0u) : bf16_lo(ws[j >> 1], 0u)) * r;
                rowc[k] = patch_nan8(rowc[k], q);
            }
        }
        {
            uint32_t t0[8], t1[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                t0[k] = rowc[k];
                t1[k] = rowc[8 + k];
            }
            transpose8x8_nibbles(t0);
            transpose8x8_nibbles(t1);
#pragma unroll
            for (int j = 0; j < 8; ++j) st.codes[stage_index<RB>(j, lane, rbl)] = make_uint2(t0[j], t1[j]);
        }
        if (WANT_W) {
#pragma unroll
            for (int k = 0; k < 16; ++k)
                st_nt(cw_codes + (size_t)(16 * ti + k) * (cols >> 1) + (c8 >> 1), rowc[k]);
        }
        if (h == 0) {
            st.tsw[rbl][lane >> 1] = (uint8_t)sb;
            st.tst[lane >> 1][rbl] = (uint8_t)sb;
        }
    }
    if (WANT_W && pos.rb < cg.nrb) write_w_scales<RB>(st, pos, cols, sw);
    const uint32_t next = tile + gridDim.x;
    const ColPos npos = col_position<RB>(cg, next);
    const bool nhave = next < cg.ntiles && npos.rb < cg.nrb && npos.c8 < cols;
    if (nhave) load_col_tile(x, cols, npos, v);
    if (WANT_WT) {
        __syncthreads();
        col_write_out<RB>(st, pos, rows, cols, cg.nrb, ct);
        write_wt_scales<RB>(st, pos, cols, cg.nrb, st_scales);
        __syncthreads();
    }
    tile = next;
    pos = npos;
    have = nhave;
    }
}

// ------------------------------------------------------------------------------------------------------------
// Four-over-six ([P3]): row-wise 1x16 RN; candidates T = 6 and T = 4; decode, squared errors, pinned tree sum
// (i, i+8), then strides 4, 2, 1; map-to-4 kept only if strictly lower.
// ------------------------------------------------------------------------------------------------------------
// Decode byte p of d (two codes) with the gfx950 FP4 -> f32 conversion.
__device__ __forceinline__ f32x2 cvt_fp4_pair(uint32_t d, int p) {
    switch (p) {
        case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
        case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
        case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
        default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
    }
}

// Decode 8 packed codes (element 2k in the low nibble of byte k) with the gfx950 FP4 -> f32 conversion.
__device__ __forceinline__ void unpack8(uint32_t d, float (&v)[8]) {
    const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
    const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
    const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
    const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
    v[0] = p0.x; v[1] = p0.y; v[2] = p1.x; v[3] = p1.y;
    v[4] = p2.x; v[5] = p2.y; v[6] = p3.x; v[7] = p3.y;
}

// One row-wise block's input words: 16 bf16 (two 16-byte words) or 16 binary32 (four), loaded from x viewed as
// 16-byte words, and widened to binary32 (exactly: a bf16 is the high half of its binary32).
template <bool F32>
struct BlockWords {
    uint4 w[F32 ? 4 : 2];
};

template <bool F32>
__device__ __forceinline__ BlockWords<F32> ld_block(const uint4* __restrict__ x, size_t n) {
    constexpr int K = F32 ? 4 : 2;
    BlockWords<F32> r;
#pragma unroll
    for (int k = 0; k < K; ++k) r.w[k] = ld16(x + K * n + k);
    return r;
}

template <bool F32>
__device__ __forceinline__ void widen_block(const BlockWords<F32>& r, float (&xv)[16]) {
    if constexpr (F32) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            xv[4 * k] = as_f(r.w[k].x);
            xv[4 * k + 1] = as_f(r.w[k].y);
            xv[4 * k + 2] = as_f(r.w[k].z);
            xv[4 * k + 3] = as_f(r.w[k].w);
        }
    } else {
        widen_row_block<false>(r.w[0], r.w[1], 0u, xv);
    }
}

// Error of one candidate from its 16 differences d (in place): ERR kErrMSE sums fl(d * d) and kErrMAE |d| by the
// width-16 tree (i with i + 8, then strides 4, 2, 1); kErrMaxAbs takes the largest |d| as an integer maximum of the
// magnitude bits, so a NaN difference makes the error NaN (NaN > inf > finite).
template <int ERR>
__device__ __forceinline__ float error16(float (&d)[16]) {
    if constexpr (ERR == kErrMaxAbs) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) m = umax(m, as_u(d[i]) & 0x7FFFFFFFu);
        return as_f(m);
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) d[i] = ERR == kErrMSE ? d[i] * d[i] : __builtin_fabsf(d[i]);
#pragma unroll
        for (int s = 8; s >= 1; s >>= 1)
#pragma unroll
            for (int i = 0; i < s; ++i) d[i] = d[i] + d[i + s];
        return d[0];
    }
}

// One block: both candidates, their decoded errors (ERR), and the choice.  xv are the 16 values, m their absmax,
// dv the divisors 6 g and 4 g, tab the multipliers of g.  A NaN or infinite g (a row whose amax is NaN or infinite)
// makes every multiplier NaN: both candidates give codes 0x7 and NaN errors (the map-to-6 one is kept), and its
// scale code is 0 where the quotient is 0 (bamax = 0; with an infinite g, any finite bamax), 0x7F (NaN) otherwise;
// that case is written directly.
template <int ERR>
__device__ __forceinline__ void quant_4o6_block(const float (&xv)[16], float m, float g, const Divisor (&dv)[2],
                                                const RTable& tab, uint32_t& lo_out, uint32_t& hi_out,
                                                uint32_t& sb_out) {
    if (!(__builtin_fabsf(g) < __builtin_inff())) [[unlikely]] {
        sb_out = (g != g) ? (m == 0.0f ? 0u : 0x7Fu) : (m < __builtin_inff() ? 0u : 0x7Fu);
        lo_out = hi_out = 0x77777777u;
        return;
    }
    uint32_t cand_lo[2], cand_hi[2], cand_sb[2];
    float err[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const uint32_t sb = scale_code(m, dv[c]);
        const float r = tab.r[sb];
        const bool fast = tab.rq[sb] == tab.rq[sb];   // see fast_multiplier
        float q[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) q[i] = xv[i] * r;
        const float(&q0)[8] = *reinterpret_cast<const float(*)[8]>(&q[0]);
        const float(&q1)[8] = *reinterpret_cast<const float(*)[8]>(&q[8]);
        uint32_t lo = pack8_rn(q0), hi = pack8_rn(q1);
        if (!fast) [[unlikely]] {
            lo = patch_nan8(lo, q0);
            hi = patch_nan8(hi, q1);
        }
        const float sbf = e4m3_decode(sb);
        float dq[16];
        unpack8(lo, *reinterpret_cast<float(*)[8]>(&dq[0]));
        unpack8(hi, *reinterpret_cast<float(*)[8]>(&dq[8]));
#pragma unroll
        for (int i = 0; i < 16; ++i) dq[i] = (dq[i] * sbf) * g - xv[i];
        cand_lo[c] = lo;
        cand_hi[c] = hi;
        cand_sb[c] = sb;
        err[c] = error16<ERR>(dq);
    }
    const int pick = (err[1] < err[0]) ? 1 : 0;
    lo_out = cand_lo[pick];
    hi_out = cand_hi[pick];
    sb_out = cand_sb[pick];
}

// Per-tensor g: grid-stride over blocks with the next block's loads in flight; the multipliers of the 128 scale
// codes are tabulated once per workgroup.
template <bool F32, int ERR>
__device__ __forceinline__ void quant_4o6_tensor_wg(const uint4* __restrict__ x, uint32_t total_blocks,
                                                    const float* __restrict__ amax, float gden,
                                                    uint2* __restrict__ codes, uint8_t* __restrict__ scales,
                                                    float* __restrict__ gout, uint32_t wg, uint32_t nwg, RTable& tab) {
    const float g = global_scale_den(amax[0], gden);
    if (wg == 0 && threadIdx.x == 0) gout[0] = g;
    const Divisor dv[2] = {make_divisor_uniform(6.0f * g), make_divisor_uniform(4.0f * g)};   // T = 6 and T = 4
    fill_rtable<false>(tab, g);
    const uint32_t stride = nwg * kThreads;
    uint32_t n = wg * kThreads + threadIdx.x;
    if (n >= total_blocks) return;
    BlockWords<F32> a = ld_block<F32>(x, n);
    for (; n < total_blocks; n += stride) {
        const uint32_t nn = n + stride;
        BlockWords<F32> a2 = a;
        if (nn < total_blocks) a2 = ld_block<F32>(x, nn);
        float xv[16];
        widen_block<F32>(a, xv);
        uint32_t lo, hi, sb;
        quant_4o6_block<ERR>(xv, absmax16(xv), g, dv, tab, lo, hi, sb);
        st_nt(codes + n, make_uint2(lo, hi));
        st_nt(scales + n, (uint8_t)sb);
        a = a2;
    }
}

template <bool F32, int ERR>
__global__ void __launch_bounds__(kThreads)
k_quant_4o6_tensor(const uint4* __restrict__ x, uint32_t total_blocks, const float* __restrict__ amax, float gden,
                   uint2* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gout) {
    __shared__ RTable tab;
    quant_4o6_tensor_wg<F32, ERR>(x, total_blocks, amax, gden, codes, scales, gout, blockIdx.x, gridDim.x, tab);
}

// Per-row g: a workgroup of NT threads walks whole rows (grid-stride over rows), lane t taking blocks t, t + NT, ...
// of each, with the next block's loads (in this row or the next) in flight.  g, its two divisors and the row's
// multiplier table are computed once per row: the table is double-buffered, so one barrier per row orders it (a
// thread writes the table of row i only after the barrier of row i - 1, which every thread passes only after its
// reads of row i - 2).
template <bool F32, int ERR, int NT = kThreads>
__device__ __forceinline__ void quant_4o6_rows_wg(const uint4* __restrict__ x, uint32_t rows, uint32_t bpr,
                                                  const float* __restrict__ amax, float gden,
                                                  uint2* __restrict__ codes, uint8_t* __restrict__ scales,
                                                  float* __restrict__ gout, uint32_t wg, uint32_t nwg,
                                                  RTable (&tabs)[2]) {
    const uint32_t t = threadIdx.x;
    BlockWords<F32> a{};
    uint32_t pr = wg, pb = t;   // the next block to load
    if (pr < rows && pb < bpr) a = ld_block<F32>(x, (size_t)pr * bpr + pb);
    pb += NT;
    if (pb >= bpr) {
        pr += nwg;
        pb = t;
    }
    for (uint32_t row = wg, parity = 0; row < rows; row += nwg, parity ^= 1u) {
        const float g = global_scale_den(amax[row], gden);
        if (t == 0) gout[row] = g;
        // a NaN or infinite g needs neither the table nor the divisors (every block of the row is written directly)
        const bool finite = __builtin_amdgcn_readfirstlane((uint32_t)(__builtin_fabsf(g) < __builtin_inff())) != 0;
        RTable& tab = tabs[parity];
        if (finite)
            for (uint32_t e = t; e < 128; e += NT) fill_rtable_entry<false>(tab, e, g);
        __syncthreads();
        Divisor dv[2] = {};
        if (finite) {
            dv[0] = make_divisor_uniform(6.0f * g);
            dv[1] = make_divisor_uniform(4.0f * g);
        }
        // (a thread with blocks in this row always has pb < bpr here)
        for (uint32_t blk = t; blk < bpr; blk += NT) {
            const BlockWords<F32> cur = a;
            if (pr < rows) a = ld_block<F32>(x, (size_t)pr * bpr + pb);
            pb += NT;
            if (pb >= bpr) {
                pr += nwg;
                pb = t;
            }
            float xv[16];
            widen_block<F32>(cur, xv);
            uint32_t lo, hi, sb;
            quant_4o6_block<ERR>(xv, absmax16(xv), g, dv, tab, lo, hi, sb);
            const size_t n = (size_t)row * bpr + blk;
            st_nt(codes + n, make_uint2(lo, hi));
            st_nt(scales + n, (uint8_t)sb);
        }
    }
}

// 128-thread workgroups, 16 per CU: each thread takes 4 blocks of a 512-block row, so the per-row table and barrier
// are shared by twice the blocks of a 256-thread workgroup (16384 x 8192 with the injected NaN/Inf: 74 -> 69 us;
// without: 79 -> 77 us; 64-thread workgroups and two blocks' loads in flight per lane measured no better)
constexpr int kThreads4o6Rows = 128;

template <bool F32, int ERR>
__global__ void __launch_bounds__(kThreads4o6Rows)
k_quant_4o6_rows(const uint4* __restrict__ x, uint32_t rows, uint32_t bpr, const float* __restrict__ amax,
                 float gden, uint2* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gout) {
    __shared__ RTable tabs[2];
    quant_4o6_rows_wg<F32, ERR, kThreads4o6Rows>(x, rows, bpr, amax, gden, codes, scales, gout, blockIdx.x,
                                                 gridDim.x, tabs);
}

// ------------------------------------------------------------------------------------------------------------
// Four-over-six with 16x16 tiles ([P3]: the reference quantizer takes 1x16 or 16x16 blocks), per-tensor g, codes
// packed along X's rows (W) and/or along its columns (W^T).  One lane per row of a tile: a 16-lane row of the wave
// holds one tile (lane i = tile row i), so a row's error sum stays in the lane and the tree over the 16 row sums,
// like the tile maximum, runs over DPP rotations within the 16-lane row.  A wave takes 4 tiles side by side; a
// workgroup 64 tiles: one band of 64 tile columns (W only), or 8 bands of 8 tile columns when W^T is written, so
// that every output row, of W and of W^T, receives 64 contiguous bytes of codes per item.
// ------------------------------------------------------------------------------------------------------------
constexpr uint32_t kTilesPerWave46 = 4;
constexpr uint32_t kTilesPerGroup46 = kTilesPerWave46 * kWavesPerGroup16;

// The value of lane (i + n) mod 16 of this lane's 16-lane row (DPP row rotation by n).
template <int N>
__device__ __forceinline__ uint32_t row_ror(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x120 + N, 0xF, 0xF, false);
}

template <int N>
__device__ __forceinline__ float row_ror_f(float v) {
    return as_f(row_ror<N>(as_u(v)));
}

// Per-element error term and the combination of two terms for the error mode: fl(d * d) and addition (kErrMSE),
// |d| and addition (kErrMAE), |d| and the integer maximum of the magnitude bits (kErrMaxAbs: NaN > inf > finite).
template <int ERR>
__device__ __forceinline__ float err_term(float d) { return ERR == kErrMSE ? d * d : __builtin_fabsf(d); }

template <int ERR>
__device__ __forceinline__ float err_join(float a, float b) {
    return ERR == kErrMaxAbs ? as_f(umax(as_u(a), as_u(b))) : a + b;
}

// Error of one candidate over the tile: this lane's row (the width-16 tree: i with i + 8, then 4, 2, 1), then the
// 16 row errors by the same tree (rows i and i + 8 first); for kErrMaxAbs the joins are maxima, whose order does not
// matter.  Lane i of the 16-lane row gets the combination over the rows rotated by i; lane 0's operand order is the
// pinned one.
template <int ERR>
__device__ __forceinline__ float tile_error(const float (&xv)[16], uint32_t lo, uint32_t hi, float sbf, float g) {
    // the first half's terms, then each term of the second half joined to its partner at once (the first level of
    // the tree) so that fewer values are live
    float e[8];
    unpack8(lo, e);
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = err_term<ERR>((e[i] * sbf) * g - xv[i]);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const f32x2 v = cvt_fp4_pair(hi, p);
        const float d0 = (v.x * sbf) * g - xv[8 + 2 * p];
        const float d1 = (v.y * sbf) * g - xv[9 + 2 * p];
        e[2 * p] = err_join<ERR>(e[2 * p], err_term<ERR>(d0));
        e[2 * p + 1] = err_join<ERR>(e[2 * p + 1], err_term<ERR>(d1));
    }
#pragma unroll
    for (int s2 = 4; s2 >= 1; s2 >>= 1)
#pragma unroll
        for (int i = 0; i < s2; ++i) e[i] = err_join<ERR>(e[i], e[i + s2]);
    float t = e[0];
    t = err_join<ERR>(t, row_ror_f<8>(t));   // lane i: row i and row i + 8 (lane 0: rows 0 and 8)
    t = err_join<ERR>(t, row_ror_f<4>(t));
    t = err_join<ERR>(t, row_ror_f<2>(t));
    t = err_join<ERR>(t, row_ror_f<1>(t));
    return t;
}

// Lane 0's value of this lane's 16-lane row (DPP row broadcast).
__device__ __forceinline__ uint32_t row_bcast0(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x150, 0xF, 0xF, false);
}

// A workgroup's outputs for one item: 64 tiles x 16 rows, tile-major (the lanes of a 16-lane row write consecutive
// slots), one pad slot per tile so that the row-major read-out spreads over the banks; two buffers, so that one
// barrier per item separates the writes of an item from the read-out of the item before it.
struct Stage46 {
    uint2 codes[2][kTilesPerGroup46][17];
    uint8_t scales[2][kTilesPerGroup46][17];
};
static_assert(kWavesPerGroup16 == 16 && kTilesPerGroup46 == 64, "a workgroup's 1024 threads write 64 tiles");

// One tile row: both candidates, the tile's errors and the choice (lane 0's, broadcast over the tile's lanes).
template <int ERR>
__device__ __forceinline__ void quant_4o6_tile_row(const float (&xv)[16], float g, bool gfinite,
                                                   const Divisor (&dv)[2], const RTable& tab, uint32_t& lo,
                                                   uint32_t& hi, uint32_t& sb) {
    // tile maximum: the row's (NaN-dominant), then over the 16 rows on the magnitude bits (NaN > inf > finite)
    uint32_t mb = as_u(absmax16(xv)) & 0x7FFFFFFFu;
    mb = umax(mb, row_ror<8>(mb));
    mb = umax(mb, row_ror<4>(mb));
    mb = umax(mb, row_ror<2>(mb));
    mb = umax(mb, row_ror<1>(mb));
    const float m = as_f(mb);
    if (!gfinite) {
        // every multiplier is NaN: codes 0x7, and the kept (map-to-6) scale is 0 where the quotient is 0
        sb = (g != g) ? (m == 0.0f ? 0u : 0x7Fu) : (m < __builtin_inff() ? 0u : 0x7Fu);
        lo = hi = 0x77777777u;
        return;
    }
    uint32_t cl[2], ch[2], cs[2];
    float err[2];
    constexpr int NC = ERR == kErrNone ? 1 : 2;   // kErrNone: map-to-6 alone
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        cs[c] = scale_code(m, dv[c]);
        const float rr = tab.r[cs[c]];
        float q[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) q[k] = xv[k] * rr;
        const float(&q0)[8] = *reinterpret_cast<const float(*)[8]>(&q[0]);
        const float(&q1)[8] = *reinterpret_cast<const float(*)[8]>(&q[8]);
        cl[c] = pack8_rn(q0);
        ch[c] = pack8_rn(q1);
        // a multiplier of 0 (g = 0) or NaN (NaN tile maximum) can make products NaN (inf * 0, x * NaN): code 0x7
        if (!(tab.rq[cs[c]] == tab.rq[cs[c]])) [[unlikely]] {
            cl[c] = patch_nan8(cl[c], q0);
            ch[c] = patch_nan8(ch[c], q1);
        }
        if (ERR != kErrNone) err[c] = tile_error<ERR>(xv, cl[c], ch[c], e4m3_decode(cs[c]), g);
    }
    if (ERR == kErrNone) {
        lo = cl[0];
        hi = ch[0];
        sb = cs[0];
        return;
    }
    // lane 0's comparison; ties and NaN keep map-to-6
    const bool four = row_bcast0(err[1] < err[0] ? 1u : 0u) != 0u;
    lo = four ? cl[1] : cl[0];
    hi = four ? ch[1] : ch[0];
    sb = four ? cs[1] : cs[0];
}

// The chunk of workgroup b among the grid's n: workgroups are dealt round-robin to the 8 XCDs, so with n a multiple
// of 8 the chunks b / 8 + (b % 8) n / 8 make each XCD's chunks consecutive.
__device__ __forceinline__ uint32_t xcd_chunk(uint32_t b, uint32_t n) {
    return (n & 7u) ? b : (b & 7u) * (n >> 3) + (b >> 3);
}

// The divisors 6 g and 4 g of a per-tensor g, formed unconditionally (unused when g is not finite) and moved to scalar
// registers: the compiler drops a readfirstlane of a value it knows to be uniform, and the division's vector result
// would then stay live across a kernel's item loop; passing it through an empty asm first hides that knowledge.
__device__ __forceinline__ void divisors_4o6(float g, Divisor (&dv)[2]) {
    dv[0] = make_divisor_uniform(6.0f * g);
    dv[1] = make_divisor_uniform(4.0f * g);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        asm volatile("" : "+v"(dv[c].d), "+v"(dv[c].y));
        dv[c].d = uniform_f(dv[c].d);
        dv[c].y = uniform_f(dv[c].y);
    }
}

// An opaque copy of the thread index: values derived from it where they are used are not kept in registers across
// a kernel's item loop (where they would not fit beside the tile and the next item's loads).
__device__ __forceinline__ uint32_t opaque_tid() {
    uint32_t t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// W only.  Items: one band (16 rows) by 64 tile columns, band-major; workgroup b takes items b, b + grid, ... (the
// whole grid works on neighbouring rows at any time) with the next item's loads in flight, and fills the multiplier
// table once.  Wave v holds tile columns 4 v .. 4 v + 3 of the item; W is written from LDS by rows (512 bytes of
// codes per row and item).
template <bool F32, int ERR>
__global__ void __launch_bounds__(kThreads16) __attribute__((amdgpu_waves_per_eu(8, 8)))
k_quant_4o6_16x16(const uint4* __restrict__ x, uint32_t ntc, uint32_t ntg, uint32_t items, float gden,
                  const float* __restrict__ amax, uint2* __restrict__ codes, uint8_t* __restrict__ scales,
                  float* __restrict__ gout) {
    __shared__ RTable tab;
    __shared__ Stage46 st;
    // this lane's 16 elements of the item (band rb, tile group tg) = block (16 rb + i) * ntc + tj of the row-wise view
    auto load = [&](uint32_t rb, uint32_t tg, BlockWords<F32>& a) {
        const uint32_t t = opaque_tid(), tj = tg * kTilesPerGroup46 + (t >> 4);
        if (tj < ntc) a = ld_block<F32>(x, (size_t)(16 * rb + (t & 15u)) * ntc + tj);
    };
    uint32_t w = blockIdx.x;
    uint32_t rb = __builtin_amdgcn_readfirstlane(w / ntg);   // (rb, tg) of the current item, in scalar registers
    uint32_t tg = __builtin_amdgcn_readfirstlane(w - rb * ntg);
    BlockWords<F32> a{};
    if (w < items) load(rb, tg, a);
    const float g = uniform_f(global_scale_den(amax[0], gden));
    if (blockIdx.x == 0 && threadIdx.x == 0) gout[0] = g;
    const bool gfinite = __builtin_fabsf(g) < __builtin_inff();
    Divisor dv[2];
    divisors_4o6(g, dv);
    fill_rtable<false>(tab, g);
    for (uint32_t buf = 0; w < items; w += gridDim.x, buf ^= 1u) {
        const uint32_t nw = w + gridDim.x;
        const uint32_t nrb = __builtin_amdgcn_readfirstlane(nw / ntg), ntgi = nw - nrb * ntg;
        const uint32_t t0 = tg * kTilesPerGroup46;   // first tile column of the item
        const bool active = t0 + (opaque_tid() >> 4) < ntc;
        float xv[16];
        widen_block<F32>(a, xv);
        // bf16: the next item's loads are in flight during this item's arithmetic; binary32 words would not fit in
        // the registers beside it, so they go out after it (overlapping the write-out)
        if (!F32 && nw < items) load(nrb, ntgi, a);
        uint32_t lo = 0, hi = 0, sb = 0;
        if (active) quant_4o6_tile_row<ERR>(xv, g, gfinite, dv, tab, lo, hi, sb);
        if (F32 && nw < items) load(nrb, ntgi, a);
        if (active) {
            const uint32_t t = opaque_tid(), slot = (t >> 4) * 17 + (t & 15u);
            (&st.codes[buf][0][0])[slot] = make_uint2(lo, hi);
            (&st.scales[buf][0][0])[slot] = (uint8_t)sb;
        }
        __syncthreads();
        // wave v takes output row v of the band, lane l tile l: 512 contiguous bytes of codes, 64 of scales
        const uint32_t t = opaque_tid(), wave = t >> 6, lane = t & 63u;
        if (t0 + lane < ntc) {
            const size_t o = (size_t)(16 * rb + wave) * ntc + t0 + lane;
            st_nt(codes + o, st.codes[buf][lane][wave]);
            st_nt(scales + o, st.scales[buf][lane][wave]);
        }
        rb = nrb;
        tg = ntgi;
    }
}

// A tile's codes transposed as a 16 x 16 matrix of nibbles across its 16 lanes: lane i holds row i (nibble k of
// (lo, hi) = element k) and gets column i (nibble k = element k of column i), the packing of a W^T row.  The usual
// recursive block transpose: 8 x 8 blocks swapped across the two words (partner lane i ^ 8), then in each word 4 x 4,
// 2 x 2 and 1 x 1 blocks (partners i ^ 4, i ^ 2, i ^ 1): each lane sends its word rotated so that the block its
// partner needs sits where the partner takes it, and keeps its own block by a bit-field insert.
__device__ __forceinline__ uint32_t dpp_xor8(uint32_t v) { return row_ror<8>(v); }
__device__ __forceinline__ uint32_t dpp_xor4(uint32_t v) {
    // lane i ^ 7 within the half row, then i ^ 3 within the quad
    const int h = __builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);
    return (uint32_t)__builtin_amdgcn_mov_dpp(h, 0x1B, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}

__device__ __forceinline__ void transpose16_nibbles(uint32_t& lo, uint32_t& hi) {
    const uint32_t i = __lane_id() & 15u;
    // 8 x 8 blocks: rows 0..7 give their elements 8..15 (hi) to rows 8..15, which give their elements 0..7 (lo)
    const uint32_t recv = dpp_xor8((i & 8u) ? lo : hi);
    if (i & 8u) lo = recv;
    else hi = recv;
    const uint32_t m4 = (i & 4u) ? 0xFFFF0000u : 0x0000FFFFu;
    const uint32_t m2 = (i & 2u) ? 0xFF00FF00u : 0x00FF00FFu;
    const uint32_t m1 = (i & 1u) ? 0xF0F0F0F0u : 0x0F0F0F0Fu;
    const uint32_t sh1 = (i & 1u) ? 28u : 4u;
    uint32_t* wp[2] = {&lo, &hi};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        uint32_t w = *wp[k];
        uint32_t r = dpp_xor4(__builtin_amdgcn_alignbit(w, w, 16));     // halves swapped
        w = (w & m4) | (r & ~m4);
        r = dpp_xor2(__builtin_amdgcn_perm(w, w, 0x02030001u));          // bytes swapped within each half
        w = (w & m2) | (r & ~m2);
        r = dpp_xor1(__builtin_amdgcn_alignbit(w, w, sh1));              // rotated by one nibble, either way
        w = (w & m1) | (r & ~m1);
        *wp[k] = w;
    }
}

// W^T (and W).  Items of 8 bands by 8 tile columns (128 x 128 elements of X): wave v holds band v / 2, tile columns
// 4 (v % 2) .. + 3 (lane 16 k + i: row i of tile k), and after quantizing transposes each tile's codes across its
// lanes (transpose16_nibbles), so that lane i also holds row i of the tile in W^T.  Both are staged in LDS,
// double-buffered (one barrier per item), and written by rows: every row of W and of W^T receives 64 contiguous
// bytes of codes (four threads, 16 bytes each) and 8 of scales per item, the scales as cached stores so that the
// pieces of neighbouring items meet in L2.  Items are numbered band-group-major; workgroup b takes per_wg
// consecutive ones (chunk xcd_chunk(b)) with the next item's loads in flight.
struct Stage16T {
    uint2 w[2][64][17];     // [buffer][tile 8 bl + c][row i]: W codes; the pad spreads the row read-out over banks
    uint2 t[2][64][17];     // [buffer][tile 8 c + bl][column j]: W^T codes
    uint8_t s[2][64];       // [buffer][8 bl + c]: tile scales
    uint8_t st[2][64];      // [buffer][8 c + bl]: the same, W^T order
};

template <bool F32, int ERR, bool W>
__global__ void __launch_bounds__(kThreads16) __attribute__((amdgpu_waves_per_eu(8, 8)))
k_quant_4o6_16x16t(const uint4* __restrict__ x, uint32_t ntc, uint32_t nbands, uint32_t ncg, uint32_t items,
                   uint32_t per_wg, float gden, const float* __restrict__ amax, uint2* __restrict__ codes_w,
                   uint8_t* __restrict__ scales_w, float* __restrict__ g_w, uint2* __restrict__ codes_wt,
                   uint8_t* __restrict__ scales_wt, float* __restrict__ g_wt) {
    __shared__ RTable tab;
    __shared__ Stage16T st;
    // this lane's 16 elements of the item (band group bg, column group cg)
    auto load = [&](uint32_t bg, uint32_t cg, BlockWords<F32>& a) {
        const uint32_t t = opaque_tid(), wave = t >> 6;
        const uint32_t rb = 8 * bg + (wave >> 1), tj = 8 * cg + 4 * (wave & 1u) + ((t >> 4) & 3u);
        if (rb < nbands && tj < ntc) a = ld_block<F32>(x, (size_t)(16 * rb + (t & 15u)) * ntc + tj);
    };
    const uint32_t w0 = xcd_chunk(blockIdx.x, gridDim.x) * per_wg;
    const uint32_t n = __builtin_amdgcn_readfirstlane(w0 < items ? min(per_wg, items - w0) : 0u);
    uint32_t bg = __builtin_amdgcn_readfirstlane(w0 / ncg);   // (bg, cg) of the current item
    uint32_t cg = __builtin_amdgcn_readfirstlane(w0 - bg * ncg);
    BlockWords<F32> a{};
    if (n) load(bg, cg, a);
    const float g = uniform_f(global_scale_den(amax[0], gden));
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (W) g_w[0] = g;
        g_wt[0] = g;
    }
    const bool gfinite = __builtin_fabsf(g) < __builtin_inff();
    Divisor dv[2];
    divisors_4o6(g, dv);
    fill_rtable<false>(tab, g);
    for (uint32_t k = 0, buf = 0; k < n; ++k, buf ^= 1u) {
        const uint32_t nbg = cg + 1 == ncg ? bg + 1 : bg, ncgi = cg + 1 == ncg ? 0u : cg + 1;
        {
            const uint32_t t = opaque_tid(), wave = t >> 6;
            const uint32_t bl = wave >> 1, c = 4 * (wave & 1u) + ((t >> 4) & 3u);
            const bool active = 8 * bg + bl < nbands && 8 * cg + c < ntc;
            float xv[16];
            widen_block<F32>(a, xv);
            // bf16: the next item's loads are in flight during this item's arithmetic; binary32 words would not fit
            // in the registers beside it, so they go out after it
            if (!F32 && k + 1 < n) load(nbg, ncgi, a);
            uint32_t lo = 0, hi = 0, sb = 0;
            if (active) quant_4o6_tile_row<ERR>(xv, g, gfinite, dv, tab, lo, hi, sb);
            if (F32 && k + 1 < n) load(nbg, ncgi, a);
            uint32_t tlo = lo, thi = hi;
            transpose16_nibbles(tlo, thi);   // a tile's 16 lanes are all active or all inactive
            if (active) {
                const uint32_t i = t & 15u;
                if (W) st.w[buf][8 * bl + c][i] = make_uint2(lo, hi);
                st.t[buf][8 * c + bl][i] = make_uint2(tlo, thi);
                if (i == 0) {
                    st.s[buf][8 * bl + c] = (uint8_t)sb;
                    st.st[buf][8 * c + bl] = (uint8_t)sb;
                }
            }
        }
        __syncthreads();
        // threads 0..511 write W, 512..1023 W^T: output row r of the item (0..127), tile pair q (16 bytes of codes)
        const uint32_t t = opaque_tid(), half = t >> 9, r = (t >> 2) & 127u, q = t & 3u;
        // W: row r = 16 bl + i, tile columns 8 cg + 2 q, + 1; W^T: row r = 16 c + j, bands 8 bg + 2 q, + 1
        const uint32_t blk = r >> 4, e = r & 15u;
        const uint32_t nrow = half ? ntc : nbands, ncol = half ? nbands : ntc;        // tiles down, tiles across
        const uint32_t rblk = half ? 8 * cg + blk : 8 * bg + blk;                     // the row's tile index down
        const uint32_t c0 = (half ? 8 * bg : 8 * cg) + 2 * q;                         // first tile across
        if ((half || W) && rblk < nrow && c0 < ncol) {
            const uint2(&sw)[64][17] = half ? st.t[buf] : st.w[buf];
            const uint2 a0 = sw[8 * blk + 2 * q][e], a1 = sw[8 * blk + 2 * q + 1][e];
            uint2* cdst = half ? codes_wt : codes_w;
            const size_t o = (size_t)(16 * rblk + e) * ncol + c0;
            if (c0 + 1 < ncol && (ncol & 1u) == 0) {
                st_nt(reinterpret_cast<uint4*>(cdst + o), make_uint4(a0.x, a0.y, a1.x, a1.y));
            } else {
                st_nt(cdst + o, a0);
                if (c0 + 1 < ncol) st_nt(cdst + o + 1, a1);
            }
            if (q == 0) {
                // 8 scale bytes of the row (fewer at the right edge)
                const uint8_t* ss = half ? &st.st[buf][8 * blk] : &st.s[buf][8 * blk];
                uint8_t* sdst = (half ? scales_wt : scales_w) + (o - 2 * q);
                const uint32_t nv = min(8u, ncol - (c0 - 2 * q));
                if (nv == 8 && (ncol & 7u) == 0) {
                    *reinterpret_cast<uint2*>(sdst) = *reinterpret_cast<const uint2*>(ss);
                } else {
                    for (uint32_t u = 0; u < nv; ++u) sdst[u] = ss[u];
                }
            }
        }
        bg = nbg;
        cg = ncgi;
    }
}

// ------------------------------------------------------------------------------------------------------------
// Tiled scale layout of the FP4 GEMM ([P2, approach]: 1x16 block scales in the SWIZZLE_32_4_4 layout): tiles of
// 128 rows x 4 scale columns, row-tile major, each a [32][4][4] byte array (byte 16 a + 4 b + c = row 32 b + a,
// column c of the tile), zero padding to whole tiles.  One lane per 16-byte row a of a tile: four 4-byte pieces of
// the rows a, a + 32, a + 64, a + 96.  A workgroup takes 8 consecutive tiles of one row tile.
// ------------------------------------------------------------------------------------------------------------
constexpr uint32_t kSwzTilesPerGroup = 8;

template <bool ALIGNED>
__global__ void __launch_bounds__(256)
k_swizzle_scales(const uint8_t* __restrict__ s, uint32_t rv, uint32_t nb, uint32_t bt, uint32_t groups_per_rt,
                 uint4* __restrict__ out) {
    const uint32_t rt = blockIdx.x / groups_per_rt;
    const uint32_t B = (blockIdx.x - rt * groups_per_rt) * kSwzTilesPerGroup + (threadIdx.x >> 5);
    if (B >= bt) return;
    const uint32_t a = threadIdx.x & 31u, k0 = 4 * B;
    uint32_t w[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t m = 128 * rt + 32 * b + a;
        w[b] = 0;
        if (m < rv) {
            const uint8_t* row = s + (size_t)m * nb + k0;
            if (ALIGNED) {   // nb % 4 == 0 and s 4-byte aligned: the 4 scales are one aligned word
                w[b] = *reinterpret_cast<const uint32_t*>(row);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (k0 + c < nb) w[b] |= (uint32_t)row[c] << (8 * c);
            }
        }
    }
    st_nt(out + ((size_t)rt * bt + B) * 32 + a, make_uint4(w[0], w[1], w[2], w[3]));
}

// ------------------------------------------------------------------------------------------------------------
// Standard NVFP4 decode ([P3]): y = fl(fl(val(code) * decode(sb)) * g); one 16-element block per lane.
// ------------------------------------------------------------------------------------------------------------
template <bool PER_ROW>
__global__ void __launch_bounds__(kThreads)
k_dequantize(const uint16_t* __restrict__ codes, const uint8_t* __restrict__ scales, const float* __restrict__ g,
             uint64_t total_quarters, FastDiv per_row, float4* __restrict__ y) {
    // one thread per 4 consecutive outputs (a quarter of a block: 2 code bytes), so each store instruction of a
    // wave covers 1 KiB of y contiguously
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    for (uint64_t q = (uint64_t)blockIdx.x * kThreads + threadIdx.x; q < total_quarters; q += stride) {
        const uint32_t n = (uint32_t)(q >> 2);
        const float gr = PER_ROW ? g[fdiv(n, per_row)] : g[0];
        const float sbf = e4m3_decode(scales[n]);
        const uint32_t c = codes[q];
        const f32x2 v01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
        const f32x2 v23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
        st_nt(y + q, make_float4((v01.x * sbf) * gr, (v01.y * sbf) * gr, (v23.x * sbf) * gr, (v23.y * sbf) * gr));
    }
}

// ------------------------------------------------------------------------------------------------------------
// Fused decode ([P3]: the optimized decode is named as future kernel work; [P1, random Hadamard transform]: blocks
// quantized after the rotation are brought back by its inverse).  d_i = fl(fl(val(code_i) * decode(sb)) * g) as in
// k_dequantize; with RHT the inverse transform: the butterfly with strides 1, 2, 4, 8 in binary32, one multiply by
// 0.25, then element i negated where bit i of the mask is set; written as float or as bf16 (round to nearest even,
// every NaN as 0x7FC0).
//   Two lanes per block: lane parity h holds elements 8 h .. 8 h + 7 (4 code bytes), so strides 1, 2 and 4 stay in
// the lane and stride 8 pairs the lane with its neighbour (one DPP exchange per value).  bf16 rows are then stored
// 16 bytes per lane, contiguous across the wave.
// ------------------------------------------------------------------------------------------------------------
// binary32 -> bf16 bits (in the high half of the result), round to nearest even on the 16 dropped bits; the
// increment carries into the exponent exactly as the rounded magnitude does (up to infinity).  NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t bf16_rne_hi(float f) {
    const uint32_t u = as_u(f);
    const uint32_t r = u + 0x7FFFu + ((u >> 16) & 1u);
    return (f != f) ? 0x7FC00000u : r;
}

template <bool RHT, bool BF16, bool PER_ROW>
__global__ void __launch_bounds__(kThreads)
k_dequantize_fused(const uint32_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                   const float* __restrict__ g, uint64_t total_halves, FastDiv per_row, uint32_t sign_mask,
                   void* __restrict__ y) {
    const uint32_t h = threadIdx.x & 1u;   // the grid stride is even, so a lane keeps its half
    float qm[8];                           // 0.25 with the lane's eight random signs
#pragma unroll
    for (int k = 0; k < 8; ++k) qm[k] = ((sign_mask >> (8 * h + k)) & 1u) ? -0.25f : 0.25f;
    const float other = h ? -1.0f : 1.0f;
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    for (uint64_t t = (uint64_t)blockIdx.x * kThreads + threadIdx.x; t < total_halves; t += stride) {
        const uint32_t n = (uint32_t)(t >> 1);
        const float gr = PER_ROW ? g[fdiv(n, per_row)] : g[0];
        const float sbf = e4m3_decode(scales[n]);
        float d[8];
        unpack8(codes[t], d);
#pragma unroll
        for (int k = 0; k < 8; ++k) d[k] = (d[k] * sbf) * gr;
        if (RHT) {
#pragma unroll
            for (int st = 1; st < 8; st <<= 1) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if ((i & st) == 0) {
                        const float a = d[i], b = d[i + st];
                        d[i] = a + b;
                        d[i + st] = a - b;
                    }
                }
            }
            // stride 8: the even lane forms w_k + w_(k+8) = own + other, the odd lane w_k - w_(k+8) = other - own;
            // fma(own, +-1, other) rounds that sum once, as the addition does
#pragma unroll
            for (int k = 0; k < 8; ++k) d[k] = __builtin_fmaf(d[k], other, pair_swap(d[k]));
#pragma unroll
            for (int k = 0; k < 8; ++k) d[k] = d[k] * qm[k];   // fl(-0.25 w) = -fl(0.25 w) exactly
        }
        if (BF16) {
            uint32_t r[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) r[k] = bf16_rne_hi(d[k]);
            const uint4 o = make_uint4(__builtin_amdgcn_perm(r[1], r[0], 0x07060302u),
                                       __builtin_amdgcn_perm(r[3], r[2], 0x07060302u),
                                       __builtin_amdgcn_perm(r[5], r[4], 0x07060302u),
                                       __builtin_amdgcn_perm(r[7], r[6], 0x07060302u));
            st_nt(reinterpret_cast<uint4*>(y) + t, o);
        } else {
            float4* yf = reinterpret_cast<float4*>(y) + 2 * t;
            st_nt(yf, make_float4(d[0], d[1], d[2], d[3]));
            st_nt(yf + 1, make_float4(d[4], d[5], d[6], d[7]));
        }
    }
}

// ------------------------------------------------------------------------------------------------------------
// amax kernels.  The maximum of magnitudes with NaN dominating (v_maximum3); reductions combine the binary32 bit
// patterns with an integer maximum, which orders NaN > inf > finite for magnitudes.
// ------------------------------------------------------------------------------------------------------------
__global__ void k_fill_zero(uint32_t* __restrict__ p, uint32_t n) {
    for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < n; i += gridDim.x * kThreads) p[i] = 0u;
}

// g = amax / gden for n entries (gden = 2688 = 6 * 448, or 6 B for a four-over-six bound B), used when the tensor
// to quantize is empty, so no block writes g.
__global__ void k_write_g(const float* __restrict__ amax, float* __restrict__ g, uint32_t n, float gden) {
    for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < n; i += gridDim.x * kThreads)
        g[i] = global_scale_den(amax[i], gden);
}

// Publishes a workgroup's partial maximum (magnitude bits) into a zeroed per-tensor amax.  Same-address atomics
// from every workgroup would serialise, so the current value is read first and the atomic is issued only when the
// partial is larger (the value only grows, so a stale read can only cause an extra atomic, never a missed one).
__device__ __forceinline__ void publish_max(uint32_t* amax_bits, uint32_t m) {
    const uint32_t cur = __hip_atomic_load(amax_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (m > cur) atomicMax(amax_bits, m);
}

// Magnitude bits of one row-wise block's maximum (after the transform when RHT).
template <bool RHT>
__device__ __forceinline__ uint32_t rowblock_absmax(const uint4& a, const uint4& b, uint32_t mask) {
    float w[16];
    widen_row_block<RHT>(a, b, mask, w);
    const float m = absmax16(w);
    return as_u(RHT ? 0.25f * m : m) & 0x7FFFFFFFu;
}

// The same on a block's words (bf16 with the optional transform, or binary32 without).
template <bool RHT, bool F32>
__device__ __forceinline__ uint32_t rowblock_absmax(const BlockWords<F32>& r, uint32_t mask) {
    if constexpr (F32) {
        float w[16];
        widen_block<true>(r, w);
        return as_u(absmax16(w)) & 0x7FFFFFFFu;
    } else {
        return rowblock_absmax<RHT>(r.w[0], r.w[1], mask);
    }
}

// Row-wise, per tensor: one 1024-thread workgroup per CU; a lane takes 8 blocks a round (base + 1024 j + t) with
// all 16 loads issued before the first is used; one atomic max per workgroup into a zeroed amax[0].
constexpr uint32_t kRowAmaxPerLane = 8;

// per_lane (1..8) blocks per lane and round: fewer let the workgroups of a grouped launch share small tensors.
template <bool RHT, bool F32 = false>
__device__ __forceinline__ void amax_rowwise_tensor_wg(const uint4* __restrict__ x, uint32_t total_blocks,
                                                       uint32_t sign_mask, uint32_t* amax_bits, uint32_t wg,
                                                       uint32_t nwg, uint32_t* red,
                                                       uint32_t per_lane = kRowAmaxPerLane) {
    const uint32_t per = per_lane * kColThreads;   // blocks per workgroup round
    uint32_t m = 0;
    for (uint32_t base = wg * per + threadIdx.x; base < total_blocks; base += nwg * per) {
        BlockWords<F32> a[kRowAmaxPerLane];
#pragma unroll
        for (uint32_t j = 0; j < kRowAmaxPerLane; ++j) {
            const uint32_t n = base + j * kColThreads;
            a[j] = BlockWords<F32>{};   // blocks past the end count as zeros
            if (j < per_lane && n < total_blocks) a[j] = ld_block<F32>(x, n);
        }
#pragma unroll
        for (uint32_t j = 0; j < kRowAmaxPerLane; ++j) m = umax(m, rowblock_absmax<RHT, F32>(a[j], sign_mask));
    }
    m = block_max<kColRB>(m, red);
    if (threadIdx.x == 0) publish_max(amax_bits, m);
}

template <bool RHT, bool F32>
__global__ void __launch_bounds__(kColThreads)
k_amax_rowwise_tensor(const uint4* __restrict__ x, uint32_t total_blocks, uint32_t sign_mask, uint32_t* amax_bits) {
    __shared__ uint32_t red[kColRB];
    amax_rowwise_tensor_wg<RHT, F32>(x, total_blocks, sign_mask, amax_bits, blockIdx.x, gridDim.x, red);
}

// Row-wise, per row: one workgroup per row (grid-stride over rows), direct store.
template <bool RHT, bool F32 = false>
__device__ __forceinline__ void amax_rowwise_rows_wg(const uint4* __restrict__ x, uint32_t rows,
                                                     uint32_t blocks_per_row, uint32_t sign_mask,
                                                     uint32_t* __restrict__ amax_bits, uint32_t wg, uint32_t nwg,
                                                     uint32_t* lds) {
    for (uint32_t r = wg; r < rows; r += nwg) {
        uint32_t m = 0;
        for (uint32_t b = threadIdx.x; b < blocks_per_row; b += kThreads) {
            const size_t n = (size_t)r * blocks_per_row + b;
            m = umax(m, rowblock_absmax<RHT, F32>(ld_block<F32>(x, n), sign_mask));
        }
        m = block_max(m, lds);
        if (threadIdx.x == 0) amax_bits[r] = m;
    }
}

template <bool RHT, bool F32>
__global__ void __launch_bounds__(kThreads)
k_amax_rowwise_rows(const uint4* __restrict__ x, uint32_t rows, uint32_t blocks_per_row, uint32_t sign_mask,
                    uint32_t* __restrict__ amax_bits) {
    __shared__ uint32_t lds[kWavesPerGroup];
    amax_rowwise_rows_wg<RHT, F32>(x, rows, blocks_per_row, sign_mask, amax_bits, blockIdx.x, gridDim.x, lds);
}

// Column-wise (V = X^T): a workgroup of 16 row-blocks x 512 columns, one row-block per wave, 8 columns per lane.  Per tensor: one
// publish per workgroup.  Per row
// of V (= per column of X): the waves' column maxima are combined in LDS, then one atomic per column.
template <bool RHT, bool PER_ROW>
__global__ void __launch_bounds__(kColThreads)
k_amax_colwise(const uint16_t* __restrict__ x, uint32_t cols, ColGrid cg, uint32_t sign_mask,
               uint32_t* __restrict__ amax_bits) {
    constexpr int kWaves = kColThreads / 64;
    __shared__ uint32_t colmax_lds[PER_ROW ? 512 * kWaves : kWaves];
    const ColPos pos = col_position(cg, blockIdx.x);
    const uint32_t wave = threadIdx.x >> 6;
    float cm[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (pos.rb < cg.nrb && pos.c8 < cols) {
        uint4 v[16];
        load_col_tile(x, cols, pos, v);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            float wp[2][16];
            widen_col_pair<RHT>(v, p, sign_mask, wp[0], wp[1]);
#pragma unroll
            for (int t = 0; t < 2; ++t) cm[2 * p + t] = absmax16(wp[t]);
        }
    }
    uint32_t cb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) cb[j] = as_u(RHT ? 0.25f * cm[j] : cm[j]) & 0x7FFFFFFFu;
    if (PER_ROW) {
#pragma unroll
        for (int j = 0; j < 8; ++j) colmax_lds[(8 * pos.lane + j) * kWaves + wave] = cb[j];
        __syncthreads();
        for (uint32_t cl = threadIdx.x; cl < 512; cl += kColThreads) {
            const uint32_t c = pos.strip * 512 + cl;
            uint32_t m = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) m = umax(m, colmax_lds[cl * kWaves + w]);
            if (c < cols) atomicMax(amax_bits + c, m);
        }
    } else {
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) m = umax(m, cb[j]);
        m = block_max<kWaves>(m, colmax_lds);
        if (threadIdx.x == 0) publish_max(amax_bits, m);
    }
}

// ------------------------------------------------------------------------------------------------------------
// Column-wise kernels for any column count (rows % 16 == 0 is all the method needs).  The tiled kernels above read
// 4 or 8 columns per load and so need every row to start on an 8- or 16-byte boundary; here a thread owns one
// column block (16 rows x 1 column) and the 64 lanes of a wave take 64 consecutive columns, so each of its 16 row
// loads still reads 128 contiguous bytes.  A workgroup covers 256 columns of up to kAnyRB row-blocks: workgroup b
// takes column chunk b % nchunks of row-block group b / nchunks.
// ------------------------------------------------------------------------------------------------------------
constexpr int kAnyThreads = 256;
constexpr uint32_t kAnyRB = 16;

// The 16 values of column c in row-block rb (sign-flipped and transformed with the RHT).
template <bool RHT>
__device__ __forceinline__ void load_col_block_any(const uint16_t* __restrict__ x, uint32_t cols, uint32_t rb,
                                                   uint32_t c, uint32_t mask, float (&w)[16]) {
    const uint16_t* p = x + (size_t)(16 * rb) * cols + c;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const uint32_t b = __builtin_nontemporal_load(p + (size_t)k * cols);
        w[k] = as_f((b << 16) ^ (RHT ? flip_bit(mask, k) : 0u));
    }
    if (RHT) fwht16(w);
}

// Column-wise quantization, any column count.  The tiled scale layout is padded to whole tiles (view rows up to a
// multiple of 128, scale columns up to a multiple of 4); the grid spans that padding and writes its bytes as zero.
template <int MODE, bool PER_ROW>
__global__ void __launch_bounds__(kAnyThreads)
k_quant_colwise_any(const uint16_t* __restrict__ x, uint32_t rows, uint32_t cols, uint32_t nchunks,
                    const float* __restrict__ amax, uint32_t sign_mask, RngArgs rng, uint8_t* __restrict__ codes,
                    uint8_t* __restrict__ scales, float* __restrict__ gout, uint32_t tiled) {
    constexpr bool SR = MODE != kRN;
    constexpr bool RHT = MODE == kRHTSR;
    __shared__ RTable tab;
    const uint32_t nrb = rows >> 4, grp = blockIdx.x / nchunks;
    const uint32_t c = (blockIdx.x - grp * nchunks) * kAnyThreads + threadIdx.x;
    Divisor d6{};
    if (!PER_ROW) {
        const float g = global_scale(amax[0]);
        d6 = make_divisor_uniform(6.0f * g);
        if (blockIdx.x == 0 && threadIdx.x == 0) gout[0] = g;
        fill_rtable<RHT>(tab, g);
    }
    const uint32_t bt = (nrb + 3) / 4, rb_end = tiled ? 4 * bt : nrb, c_end = tiled ? (cols + 127) & ~127u : cols;
    if (c >= c_end) return;
    float gr = 0.0f;
    if (PER_ROW && c < cols) {
        gr = global_scale(amax[c]);
        if (grp == 0) gout[c] = gr;
    }
    for (uint32_t rb = grp * kAnyRB; rb < min(rb_end, (grp + 1) * kAnyRB); ++rb) {
        const size_t so = tiled ? tiled_scale_offset(c, rb, bt) : (size_t)c * nrb + rb;
        if (c >= cols || rb >= nrb) {                    // padding of the tiled layout
            scales[so] = 0;
            continue;
        }
        float w[16];
        load_col_block_any<RHT>(x, cols, rb, c, sign_mask, w);
        Rand4 inv{{0, 0, 0, 0}};
        if (SR) inv = block_rand_inv(rng, c * nrb + rb);
        uint32_t lo, hi, sb;
        if (PER_ROW) quantize_block<SR, RHT>(w, make_divisor(6.0f * gr), RowMul<RHT>{gr}, inv, lo, hi, sb);
        else quantize_block<SR, RHT>(w, d6, TableMul{tab}, inv, lo, hi, sb);
        st_nt(reinterpret_cast<uint2*>(codes + (size_t)c * (rows >> 1) + 8 * (size_t)rb), make_uint2(lo, hi));
        scales[so] = (uint8_t)sb;
    }
}

// Column-wise amax, any column count: the maximum over the thread's blocks, then per column (PER_ROW: the view's
// rows are the columns) or per tensor.
template <bool RHT, bool PER_ROW>
__global__ void __launch_bounds__(kAnyThreads)
k_amax_colwise_any(const uint16_t* __restrict__ x, uint32_t rows, uint32_t cols, uint32_t nchunks, uint32_t sign_mask,
                   uint32_t* __restrict__ amax_bits) {
    __shared__ uint32_t red[kAnyThreads / 64];
    const uint32_t nrb = rows >> 4, grp = blockIdx.x / nchunks;
    const uint32_t c = (blockIdx.x - grp * nchunks) * kAnyThreads + threadIdx.x;
    uint32_t m = 0;
    if (c < cols) {
        for (uint32_t rb = grp * kAnyRB; rb < min(nrb, (grp + 1) * kAnyRB); ++rb) {
            float w[16];
            load_col_block_any<RHT>(x, cols, rb, c, sign_mask, w);
            const float a = absmax16(w);
            m = umax(m, as_u(RHT ? 0.25f * a : a) & 0x7FFFFFFFu);
        }
        if (PER_ROW) atomicMax(amax_bits + c, m);
    }
    if (!PER_ROW) {
        m = block_max<kAnyThreads / 64>(m, red);
        if (threadIdx.x == 0) publish_max(amax_bits, m);
    }
}

// ------------------------------------------------------------------------------------------------------------
// Single-read amax + row-wise 1x16 quantization (same exchange as the column-wise single-read kernel).  A
// workgroup owns bpl * 1024 consecutive blocks (bpl <= 8 per lane), lane t of the workgroup blocks base + 1024 j + t,
// so every load instruction of a wave covers 2 KiB of the tensor with its partner; the tile is held in registers
// across the wait and the codes and scales are stored straight from the lanes.
// ------------------------------------------------------------------------------------------------------------
constexpr uint32_t kRowFusedPerLane = 8;

// TILED: the workgroup takes item blockIdx.x of the tiled-scale mapping (128 rows x 64 blocks, 8 blocks per lane:
// block l of row 16 j + w for lane l of wave w) and writes its scales as 16 whole tiles at the end; otherwise lane t
// takes blocks blockIdx.x * bpl * 1024 + 1024 j + t.  rows, nb and items_per_band are used only when TILED.
// The blocks of row-wise single-read workgroup (tile) t: index and existence of the lane's j-th block.
struct RowFusedTile {
    uint32_t total_blocks, bpl, rows, nb, items_per_band;
    bool tiled;
    __device__ uint32_t index(uint32_t t, uint32_t j) const {
        if (tiled) {
            const RowTileItem it = row_tile_item(t, items_per_band);
            return (it.row0 + 16 * j + (threadIdx.x >> 6)) * nb + it.blk0 + (threadIdx.x & 63u);
        }
        return t * bpl * kColThreads + threadIdx.x + j * kColThreads;
    }
    __device__ bool valid(uint32_t t, uint32_t j) const {
        if (tiled) {
            const RowTileItem it = row_tile_item(t, items_per_band);
            return it.blk0 + (threadIdx.x & 63u) < nb && it.row0 + 16 * j + (threadIdx.x >> 6) < rows;
        }
        return j < bpl && index(t, j) < total_blocks;
    }
};

// TILED: the workgroup takes item blockIdx.x of the tiled-scale mapping (128 rows x 64 blocks, 8 blocks per lane:
// block l of row 16 j + w for lane l of wave w) and writes its scales as 16 whole tiles at the end; otherwise lane t
// takes blocks blockIdx.x * bpl * 1024 + 1024 j + t.  rows, nb and items_per_band are used only when TILED.
template <int MODE, bool TILED>
__global__ void __launch_bounds__(kColThreads)
k_amax_quant_rowwise(const uint4* __restrict__ x, uint32_t total_blocks, uint32_t bpl, uint32_t sign_mask,
                     RngArgs rng, float* __restrict__ amax_out, uint2* __restrict__ codes,
                     uint8_t* __restrict__ scales, float* __restrict__ gout, Exchange ex, uint32_t rows, uint32_t nb,
                     uint32_t items_per_band) {
    constexpr bool SR = MODE != kRN;
    constexpr bool RHT = MODE == kRHTSR;
    __shared__ ColStash st;
    __shared__ RTable tab;
    __shared__ uint32_t red[kColRB], missing[64], s_own;
    announce(ex);
    const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63u;
    const RowFusedTile tl{total_blocks, bpl, rows, nb, items_per_band, TILED};
    const RowTileItem it = TILED ? row_tile_item(blockIdx.x, items_per_band) : RowTileItem{0, 0};
    auto index = [&](uint32_t j) -> uint32_t { return tl.index(blockIdx.x, j); };
    auto valid = [&](uint32_t j) -> bool { return tl.valid(blockIdx.x, j); };
    uint4 a[kRowFusedPerLane], b[kRowFusedPerLane];
    float bm[kRowFusedPerLane];
    uint32_t mbits = 0;
#pragma unroll
    for (uint32_t j = 0; j < kRowFusedPerLane; ++j) {
        const uint32_t n = index(j);
        a[j] = b[j] = make_uint4(0, 0, 0, 0);
        if (valid(j)) {
            a[j] = ld16(x + 2 * (size_t)n);
            b[j] = ld16(x + 2 * (size_t)n + 1);
        }
    }
    // the random words, generated while the loads are in flight, parked in LDS
    if (SR) {
#pragma unroll
        for (uint32_t j = 0; j < kRowFusedPerLane; ++j) {
            const uint32_t n = index(j);
            if (valid(j)) {
                const Rand4 r = block_rand_inv(rng, n);
                st.e[wave][j * 64 + lane] = make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]);
            }
        }
    }
#pragma unroll
    for (uint32_t j = 0; j < kRowFusedPerLane; ++j) {
        float w[16];
        widen_row_block<RHT>(a[j], b[j], sign_mask, w);
        bm[j] = absmax16(w);   // 0 for the zero words of blocks outside the tensor
        mbits = umax(mbits, as_u(RHT ? 0.25f * bm[j] : bm[j]) & 0x7FFFFFFFu);
    }
#pragma unroll
    for (uint32_t j = 0; j < kRowFusedPerLane; ++j) {
        asm volatile("" : "+v"(a[j].x), "+v"(a[j].y), "+v"(a[j].z), "+v"(a[j].w));
        asm volatile("" : "+v"(b[j].x), "+v"(b[j].y), "+v"(b[j].z), "+v"(b[j].w));
    }
    uint32_t nmiss;
    uint32_t abits = exchange_max<RHT>(mbits, ex, red, missing, &s_own, tab, nmiss);
    if (nmiss) {
        // slow route: the maxima of the tiles whose slots were not seen, from the tensor (the own tile stays in
        // registers)
        __shared__ uint32_t s_bits;
        uint32_t m = 0;
        for (uint32_t t = 0; t < gridDim.x; ++t) {
            if (!slot_missing(missing, t)) continue;
            for (uint32_t j = 0; j < kRowFusedPerLane; ++j) {
                if (tl.valid(t, j)) {
                    const uint32_t n = tl.index(t, j);
                    m = umax(m, rowblock_absmax<RHT>(ld16(x + 2 * (size_t)n), ld16(x + 2 * (size_t)n + 1), sign_mask));
                }
            }
        }
        m = block_max<kColRB>(m, red);
        if (threadIdx.x == 0) s_bits = umax(m, abits);
        __syncthreads();
        abits = __builtin_amdgcn_readfirstlane(s_bits);
        fill_rtable<RHT>(tab, global_scale(as_f(abits)));
    }
    const float amax = as_f(abits);
    const float g = global_scale(amax);
    const Divisor d6 = make_divisor_uniform(6.0f * g);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        amax_out[0] = amax;
        gout[0] = g;
    }
#pragma unroll
    for (uint32_t j = 0; j < kRowFusedPerLane; ++j) {
        const uint32_t n = index(j);
        if (valid(j)) {
            Rand4 inv{{0, 0, 0, 0}};
            if (SR) {
                const uint4 r = st.e[wave][j * 64 + lane];
                inv = Rand4{{r.x, r.y, r.z, r.w}};
            }
            float w[16];
            widen_row_block<RHT>(a[j], b[j], sign_mask, w);
            uint32_t lo, hi, sb;
            quantize_block_m<SR, RHT>(w, bm[j], d6, TableMul{tab}, inv, lo, hi, sb);
            st_nt(codes + n, make_uint2(lo, hi));
            if (TILED) st.e[wave][j * 64 + lane].z = sb;   // the slot's random words are used up
            else st_nt(scales + n, (uint8_t)sb);
        }
    }
    if (TILED) {
        __syncthreads();
        // row r of the item is slice r / 16 of wave r % 16
        row_write_scales_tiled(it, rows, nb, scales, [&](uint32_t r, uint32_t c) {
            return (uint8_t)st.e[r & 15u][(r >> 4) * 64 + c].z;
        });
    }
    release_slot(ex, s_own);
}

// ------------------------------------------------------------------------------------------------------------
// Grouped launches ([P3]: grouped variants of the quantizer are named as future kernel work): up to kMaxGroup
// row-wise tensors of any shapes in one launch.  The descriptors travel as kernel arguments (nothing is allocated);
// the workgroups are split among the tensors in proportion to their blocks, each workgroup finds its tensor with a
// scalar search over the first-workgroup indices and then runs the single-tensor body on its share, so every result
// equals that of the per-tensor call.
// ------------------------------------------------------------------------------------------------------------
struct GroupItemK {
    const uint4* x;
    uint2* codes;
    uint8_t* scales;
    float* g;
    const float* amax;
    uint32_t rows, bpr, blocks;   // bpr = blocks per row
    FastDiv per_row;              // n / bpr
    uint32_t sign_mask;
    RngArgs rng;
    uint32_t wg0;                 // first workgroup of this tensor
};

struct GroupArgs {
    uint32_t count, total_wg;
    float gden;                   // four-over-six: 6 B for the bound B
    uint32_t per_lane = kRowAmaxPerLane;   // per-tensor amax: blocks per lane and round
    GroupItemK it[kMaxGroup];
};
static_assert(sizeof(GroupArgs) <= 4096, "grouped descriptors must fit the kernel-argument space");

// The tensor of this workgroup and the workgroup's index and count within it.
__device__ __forceinline__ uint32_t group_item(const GroupArgs& ga, uint32_t& wg, uint32_t& nwg) {
    uint32_t i = 0;
    for (uint32_t j = 1; j < ga.count; ++j)
        if (ga.it[j].wg0 <= blockIdx.x) i = j;
    const uint32_t end = i + 1 < ga.count ? ga.it[i + 1].wg0 : ga.total_wg;
    wg = blockIdx.x - ga.it[i].wg0;
    nwg = end - ga.it[i].wg0;
    return i;
}

template <int MODE, bool PER_ROW>
__global__ void __launch_bounds__(kThreads) k_quant_grouped(const GroupArgs ga) {
    __shared__ RTable tab;
    uint32_t wg, nwg;
    const GroupItemK& it = ga.it[group_item(ga, wg, nwg)];
    quant_rowwise_wg<MODE, PER_ROW>(it.x, it.blocks, it.per_row, it.amax, it.sign_mask, it.rng, it.codes, it.scales,
                                    it.g, wg, nwg, tab);
}

template <bool PER_ROW, int ERR>
__global__ void __launch_bounds__(kThreads) k_quant_4o6_grouped(const GroupArgs ga) {
    __shared__ RTable tabs[2];
    uint32_t wg, nwg;
    const GroupItemK& it = ga.it[group_item(ga, wg, nwg)];
    if (PER_ROW)
        quant_4o6_rows_wg<false, ERR>(it.x, it.rows, it.bpr, it.amax, ga.gden, it.codes, it.scales, it.g, wg, nwg,
                                      tabs);
    else
        quant_4o6_tensor_wg<false, ERR>(it.x, it.blocks, it.amax, ga.gden, it.codes, it.scales, it.g, wg, nwg,
                                        tabs[0]);
}

// Zeroes the per-tensor amax of every tensor (the grouped per-tensor amax publishes into zeroed values).
__global__ void k_zero_group_amax(const GroupArgs ga) {
    if (threadIdx.x < ga.count) *const_cast<float*>(ga.it[threadIdx.x].amax) = 0.0f;
}

template <bool RHT>
__global__ void __launch_bounds__(kColThreads) k_amax_grouped_tensor(const GroupArgs ga) {
    __shared__ uint32_t red[kColRB];
    uint32_t wg, nwg;
    const GroupItemK& it = ga.it[group_item(ga, wg, nwg)];
    amax_rowwise_tensor_wg<RHT>(it.x, it.blocks, it.sign_mask, reinterpret_cast<uint32_t*>(const_cast<float*>(it.amax)),
                                wg, nwg, red, ga.per_lane);
}

template <bool RHT>
__global__ void __launch_bounds__(kThreads) k_amax_grouped_rows(const GroupArgs ga) {
    __shared__ uint32_t lds[kWavesPerGroup];
    uint32_t wg, nwg;
    const GroupItemK& it = ga.it[group_item(ga, wg, nwg)];
    amax_rowwise_rows_wg<RHT>(it.x, it.rows, it.bpr, it.sign_mask, reinterpret_cast<uint32_t*>(const_cast<float*>(it.amax)),
                              wg, nwg, lds);
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

// Column-wise grid: one workgroup per (RB row-blocks) x (512-column strip), strip-fastest.
ColGrid col_grid(int64_t rows, int64_t cols, uint32_t& grid, uint32_t rb = kColRB) {
    ColGrid g;
    g.nrb = (uint32_t)(rows / 16);
    g.nstrips = (uint32_t)((cols + 511) / 512);
    g.ntiles = ((g.nrb + rb - 1) / rb) * g.nstrips;
    grid = g.ntiles;
    if (grid == 0) grid = 1;
    return g;
}

// Grid of the any-column-count kernels: 256-column chunks by groups of kAnyRB row-blocks, over the padded view of
// the tiled scale layout when `tiled`.
struct AnyGrid {
    uint32_t nchunks, grid;
};

AnyGrid any_grid(int64_t rows, int64_t cols, bool tiled) {
    const uint32_t nrb = (uint32_t)(rows / 16);
    const uint32_t rb_end = tiled ? (nrb + 3) / 4 * 4 : nrb;
    const uint32_t c_end = (uint32_t)(tiled ? (cols + 127) / 128 * 128 : cols);
    AnyGrid a;
    a.nchunks = (c_end + kAnyThreads - 1) / kAnyThreads;
    a.grid = a.nchunks * ((rb_end + kAnyRB - 1) / kAnyRB);
    if (a.grid == 0) a.grid = 1;
    return a;
}

// Grid of a tile-looping column kernel: at most `per_cu` workgroups per CU (all resident), and every workgroup the
// same number of tiles (448 tiles on 256 CUs: 224 workgroups of 2 tiles rather than two rounds with a partial
// second).
uint32_t looping_grid(uint32_t ntiles, uint32_t per_cu = 1) {
    const uint32_t slots = (uint32_t)cu_count() * per_cu;
    if (ntiles <= slots) return ntiles ? ntiles : 1;
    const uint32_t per = (ntiles + slots - 1) / slots;
    return (ntiles + per - 1) / per;
}

RngArgs rng_args(Philox p) {
    return RngArgs{(uint32_t)p.seed, (uint32_t)(p.seed >> 32), (uint32_t)p.offset, (uint32_t)(p.offset >> 32)};
}

hipError_t write_empty_g(const float* amax, float* g, uint32_t n, hipStream_t stream, float gden = 2688.0f) {
    if (n) k_write_g<<<grid_for(n, kThreads, 1), kThreads, 0, stream>>>(amax, g, n, gden);
    return hipGetLastError();
}


}  // namespace

// Row-wise amax kernels (bf16, or binary32 without the transform), into zeroed bits (per tensor) or bits[rows].
void launch_amax_rowwise(const void* x, int64_t rows, int64_t cols, bool per_row, bool use_rht, bool f32,
                         uint32_t sign_mask, uint32_t* bits, hipStream_t stream) {
    const uint32_t bpr = (uint32_t)(cols / 16);
    const uint32_t total = (uint32_t)(rows * bpr);
    const uint4* xv = reinterpret_cast<const uint4*>(x);
    if (per_row) {
        const uint32_t grid = (uint32_t)(rows < 65536 * 16 ? rows : 65536 * 16);
        if (f32) k_amax_rowwise_rows<false, true><<<grid, kThreads, 0, stream>>>(xv, (uint32_t)rows, bpr, 0u, bits);
        else if (use_rht)
            k_amax_rowwise_rows<true, false><<<grid, kThreads, 0, stream>>>(xv, (uint32_t)rows, bpr, sign_mask, bits);
        else k_amax_rowwise_rows<false, false><<<grid, kThreads, 0, stream>>>(xv, (uint32_t)rows, bpr, sign_mask, bits);
    } else {
        const uint32_t grid = grid_for(total, kColThreads * kRowAmaxPerLane, 1);
        if (f32) k_amax_rowwise_tensor<false, true><<<grid, kColThreads, 0, stream>>>(xv, total, 0u, bits);
        else if (use_rht) k_amax_rowwise_tensor<true, false><<<grid, kColThreads, 0, stream>>>(xv, total, sign_mask, bits);
        else k_amax_rowwise_tensor<false, false><<<grid, kColThreads, 0, stream>>>(xv, total, sign_mask, bits);
    }
}

hipError_t launch_amax_f32(const float* x, int64_t rows, int64_t cols, bool per_row, float* amax, hipStream_t stream) {
    uint32_t* bits = reinterpret_cast<uint32_t*>(amax);
    if (!per_row || rows == 0 || cols == 0) {
        const uint32_t n = per_row ? (uint32_t)rows : 1u;
        if (n) k_fill_zero<<<grid_for(n, kThreads, 1), kThreads, 0, stream>>>(bits, n);
    }
    if (rows == 0 || cols == 0) return hipGetLastError();
    launch_amax_rowwise(x, rows, cols, per_row, false, true, 0u, bits, stream);
    return hipGetLastError();
}

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
        launch_amax_rowwise(x, rows, cols, per_row, use_rht, false, sign_mask, bits, stream);
    } else if (cols % 8 != 0) {
        const AnyGrid a = any_grid(rows, cols, false);
        const uint32_t r = (uint32_t)rows, c = (uint32_t)cols;
#define NVFP4_ANY(R, P) k_amax_colwise_any<R, P><<<a.grid, kAnyThreads, 0, stream>>>(x, r, c, a.nchunks, sign_mask, bits)
        if (use_rht && per_row) NVFP4_ANY(true, true);
        else if (use_rht) NVFP4_ANY(true, false);
        else if (per_row) NVFP4_ANY(false, true);
        else NVFP4_ANY(false, false);
#undef NVFP4_ANY
    } else {
        uint32_t grid;
        const ColGrid w = col_grid(rows, cols, grid);
        const uint32_t c = (uint32_t)cols;
        if (use_rht && per_row) k_amax_colwise<true, true><<<grid, kColThreads, 0, stream>>>(x, c, w, sign_mask, bits);
        else if (use_rht) k_amax_colwise<true, false><<<grid, kColThreads, 0, stream>>>(x, c, w, sign_mask, bits);
        else if (per_row) k_amax_colwise<false, true><<<grid, kColThreads, 0, stream>>>(x, c, w, sign_mask, bits);
        else k_amax_colwise<false, false><<<grid, kColThreads, 0, stream>>>(x, c, w, sign_mask, bits);
    }
    return hipGetLastError();
}

hipError_t launch_quant_1x16(const uint16_t* x, int64_t rows, int64_t cols, bool colwise, bool per_row, Mode mode,
                             const float* amax, uint32_t sign_mask, Philox rng, uint8_t* codes, uint8_t* scales,
                             float* g, hipStream_t stream, bool tiled) {
    const RngArgs ra = rng_args(rng);
    const int64_t rv = colwise ? cols : rows;
    if (rows == 0 || cols == 0) return write_empty_g(amax, g, per_row ? (uint32_t)rv : 1u, stream);
    // tiled scales with padding (rows not a multiple of 128 or blocks per row not of 4) take the item kernel, which
    // writes the padding; without, the row-major kernel stores each scale byte at its tiled place
    const bool tiled_items = tiled && (rows % 128 != 0 || (cols / 16) % 4 != 0);
    if (!colwise && tiled_items) {
        const uint32_t nb = (uint32_t)(cols / 16), ipb = (nb + 63) / 64;
        const uint32_t items = (uint32_t)((rows + 127) / 128) * ipb;
        const uint32_t grid = std::min<uint32_t>(items, 3u * (uint32_t)cu_count());
        const uint4* xv = reinterpret_cast<const uint4*>(x);
        uint2* cv = reinterpret_cast<uint2*>(codes);
#define NVFP4_ROWT(M, P)                                                                                        \
    k_quant_rowwise_tiled<M, P><<<grid, kThreadsRT, 0, stream>>>(xv, (uint32_t)rows, nb, ipb, items, amax, sign_mask, \
                                                                ra, cv, scales, g)
        switch (mode) {
            case kRN: if (per_row) NVFP4_ROWT(kRN, true); else NVFP4_ROWT(kRN, false); break;
            case kSR: if (per_row) NVFP4_ROWT(kSR, true); else NVFP4_ROWT(kSR, false); break;
            case kRHTSR: if (per_row) NVFP4_ROWT(kRHTSR, true); else NVFP4_ROWT(kRHTSR, false); break;
        }
#undef NVFP4_ROWT
    } else if (!colwise) {
        const uint32_t bpr = (uint32_t)(cols / 16);
        const uint32_t total = (uint32_t)(rows * bpr);
        const FastDiv fd = make_fastdiv(bpr);
        const uint32_t grid = grid_for(total, kThreads, 8);
        const uint4* xv = reinterpret_cast<const uint4*>(x);
        uint2* cv = reinterpret_cast<uint2*>(codes);
        const uint32_t tbt = tiled ? bpr / 4 : 0u;
#define NVFP4_ROW(M, P) \
    k_quant_rowwise<M, P><<<grid, kThreads, 0, stream>>>(xv, total, fd, amax, sign_mask, ra, cv, scales, g, tbt)
        switch (mode) {
            case kRN: if (per_row) NVFP4_ROW(kRN, true); else NVFP4_ROW(kRN, false); break;
            case kSR: if (per_row) NVFP4_ROW(kSR, true); else NVFP4_ROW(kSR, false); break;
            case kRHTSR: if (per_row) NVFP4_ROW(kRHTSR, true); else NVFP4_ROW(kRHTSR, false); break;
        }
#undef NVFP4_ROW
    } else if (!per_row && cols % 4 == 0) {
        const uint32_t nrb = (uint32_t)(rows / 16), nstrips = (uint32_t)((cols + kStrip4 - 1) / kStrip4);
        const uint32_t grid = ((nrb + kColRB - 1) / kColRB) * nstrips;
        const FastDiv ns = make_fastdiv(nstrips);
#define NVFP4_COL4(M)                                                                                          \
    k_quant_colwise4<M><<<grid, kColThreads, 0, stream>>>(x, (uint32_t)rows, (uint32_t)cols, nrb, ns, amax,      \
                                                          sign_mask, ra, codes, scales, g, tiled ? 1u : 0u)
        switch (mode) {
            case kRN: NVFP4_COL4(kRN); break;
            case kSR: NVFP4_COL4(kSR); break;
            case kRHTSR: NVFP4_COL4(kRHTSR); break;
        }
#undef NVFP4_COL4
    } else if (cols % 8 != 0) {
        const AnyGrid a = any_grid(rows, cols, tiled);
#define NVFP4_ANY(M, P)                                                                                          \
    k_quant_colwise_any<M, P><<<a.grid, kAnyThreads, 0, stream>>>(x, (uint32_t)rows, (uint32_t)cols, a.nchunks, amax, \
                                                                  sign_mask, ra, codes, scales, g, tiled ? 1u : 0u)
        switch (mode) {
            case kRN: if (per_row) NVFP4_ANY(kRN, true); else NVFP4_ANY(kRN, false); break;
            case kSR: if (per_row) NVFP4_ANY(kSR, true); else NVFP4_ANY(kSR, false); break;
            case kRHTSR: if (per_row) NVFP4_ANY(kRHTSR, true); else NVFP4_ANY(kRHTSR, false); break;
        }
#undef NVFP4_ANY
    } else {
        uint32_t grid;
        const ColGrid w = col_grid(rows, cols, grid);
#define NVFP4_COL(M, P)                                                                                     \
    k_quant_colwise<M, P><<<grid, kColThreads, 0, stream>>>(x, (uint32_t)rows, (uint32_t)cols, w, amax,    \
                                                            sign_mask, ra, codes, scales, g, tiled ? 1u : 0u)
        switch (mode) {
            case kRN: if (per_row) NVFP4_COL(kRN, true); else NVFP4_COL(kRN, false); break;
            case kSR: if (per_row) NVFP4_COL(kSR, true); else NVFP4_COL(kSR, false); break;
            case kRHTSR: if (per_row) NVFP4_COL(kRHTSR, true); else NVFP4_COL(kRHTSR, false); break;
        }
#undef NVFP4_COL
    }
    return hipGetLastError();
}

// Device address of `scratch` (the single-read exchange slots) on the current device, looked up once per device with
// that device current; host code uses this address, never the array's name.
hipError_t scratch_on_device(uint64_t** out) {
    static std::atomic<uint64_t*> cached[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    uint64_t* p = cached[dev].load(std::memory_order_acquire);
    if (!p) {
        void* q = nullptr;
        e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        p = static_cast<uint64_t*>(q);
        cached[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

uint64_t ticks_from_env(const char* name, uint64_t dflt) {
    const char* e = getenv(name);
    if (!e || !*e) return dflt;
    return strtoull(e, nullptr, 10);
}

// The exchange of the next single-read launch: a fresh nonzero epoch and its slot region.  The wait bounds can be
// overridden (100 MHz ticks) by NVFP4_FUSED_WAIT_TICKS and NVFP4_FUSED_ARRIVE_TICKS, and NVFP4_FUSED_REGION puts
// every launch in one region: the tests use them to send workgroups down the slow route and to make concurrent
// launches share a region, and check that the results do not change.
hipError_t next_exchange(Exchange* ex) {
    uint64_t* base = nullptr;
    const hipError_t e = scratch_on_device(&base);
    if (e != hipSuccess) return e;
    static std::atomic<uint32_t> launches{0};
    uint32_t epoch = launches.fetch_add(1, std::memory_order_relaxed) + 1;
    if (epoch == 0) epoch = launches.fetch_add(1, std::memory_order_relaxed) + 1;   // after 2^32 launches
    const uint64_t fixed = ticks_from_env("NVFP4_FUSED_REGION", kSlotRegions);
    ex->region = base + (size_t)(fixed < kSlotRegions ? fixed : epoch % kSlotRegions) * kSlotsPerRegion;
    ex->epoch = epoch;
    ex->pad = 0;
    ex->wait_ticks = ticks_from_env("NVFP4_FUSED_WAIT_TICKS", kWaitTicks);
    ex->arrive_ticks = ticks_from_env("NVFP4_FUSED_ARRIVE_TICKS", kArriveTicks);
    return hipSuccess;
}

hipError_t launch_amax_quant(const uint16_t* x, int64_t rows, int64_t cols, bool colwise, Mode mode, uint32_t sign_mask,
                             Philox rng, float* amax, uint8_t* codes, uint8_t* scales, float* g, hipStream_t stream,
                             bool tiled) {
    if (rows > 0 && cols > 0 && colwise && cols % 4 == 0) {
        const uint32_t nrb = (uint32_t)(rows / 16), nstrips = (uint32_t)((cols + kStrip4 - 1) / kStrip4);
        const uint32_t grid = ((nrb + kColRB - 1) / kColRB) * nstrips;
        // two 1024-thread workgroups per CU (registers and LDS allow no third), all resident at once
        if (grid <= 2u * (uint32_t)cu_count() && grid <= kFusedMaxGrid) {
            uint32_t r = (uint32_t)rows, c = (uint32_t)cols, nr = nrb;
            FastDiv ns = make_fastdiv(nstrips);
            RngArgs ra = rng_args(rng);
            Exchange ex;
            const hipError_t e = next_exchange(&ex);
            if (e != hipSuccess) return e;
            uint32_t tl = tiled ? 1u : 0u;
            void* args[] = {(void*)&x, &r, &c, &nr, &ns, &sign_mask, &ra, (void*)&amax, (void*)&codes, (void*)&scales,
                            (void*)&g, &ex, &tl};
            const void* fn = mode == kRN ? (const void*)k_amax_quant_colwise4<kRN>
                             : mode == kSR ? (const void*)k_amax_quant_colwise4<kSR>
                                           : (const void*)k_amax_quant_colwise4<kRHTSR>;
            return hipLaunchKernel(fn, dim3(grid), dim3(kColThreads), args, 0, stream);
        }
    }
    // tiled scales: one item kernel (storing each scale byte at its tiled place from the row-major kernel measured
    // 25.2 against 22.9 us at 8192 x 4096 RN: every workgroup's scattered stores come at once, in phase 2)
    if (rows > 0 && cols > 0 && !colwise && tiled) {
        // one tiled-scale item (128 rows x 64 blocks) per workgroup, all resident
        const uint32_t nb = (uint32_t)(cols / 16), ipb = (nb + 63) / 64;
        const uint64_t items = (uint64_t)((rows + 127) / 128) * ipb;
        if (items <= (uint64_t)cu_count() && items <= kFusedMaxGrid) {
            const uint4* xv = reinterpret_cast<const uint4*>(x);
            uint2* cv = reinterpret_cast<uint2*>(codes);
            RngArgs ra = rng_args(rng);
            Exchange ex;
            const hipError_t e = next_exchange(&ex);
            if (e != hipSuccess) return e;
            uint32_t t = (uint32_t)(rows * nb), bp = kRowFusedPerLane, r = (uint32_t)rows, nbv = nb, ip = ipb;
            void* args[] = {(void*)&xv, &t, &bp, &sign_mask, &ra, (void*)&amax, (void*)&cv, (void*)&scales,
                            (void*)&g, &ex, &r, &nbv, &ip};
            const void* fn = mode == kRN ? (const void*)k_amax_quant_rowwise<kRN, true>
                             : mode == kSR ? (const void*)k_amax_quant_rowwise<kSR, true>
                                           : (const void*)k_amax_quant_rowwise<kRHTSR, true>;
            return hipLaunchKernel(fn, dim3((uint32_t)items), dim3(kColThreads), args, 0, stream);
        }
    } else if (rows > 0 && cols > 0 && !colwise) {
        const uint32_t total = (uint32_t)(rows * (cols / 16));
        const uint32_t cus = (uint32_t)cu_count();
        const uint32_t bpl = (uint32_t)(((uint64_t)total + (uint64_t)cus * kColThreads - 1) / ((uint64_t)cus * kColThreads));
        if (bpl <= kRowFusedPerLane) {
            const uint32_t per = bpl * kColThreads;
            const uint32_t grid = (total + per - 1) / per;   // <= CUs
            if (grid <= kFusedMaxGrid) {
                const uint4* xv = reinterpret_cast<const uint4*>(x);
                uint2* cv = reinterpret_cast<uint2*>(codes);
                RngArgs ra = rng_args(rng);
                Exchange ex;
                const hipError_t e = next_exchange(&ex);
                if (e != hipSuccess) return e;
                uint32_t t = total, bp = bpl, unused = 0;
                void* args[] = {(void*)&xv, &t, &bp, &sign_mask, &ra, (void*)&amax, (void*)&cv, (void*)&scales,
                                (void*)&g, &ex, &unused, &unused, &unused};
                const void* fn = mode == kRN ? (const void*)k_amax_quant_rowwise<kRN, false>
                                 : mode == kSR ? (const void*)k_amax_quant_rowwise<kSR, false>
                                               : (const void*)k_amax_quant_rowwise<kRHTSR, false>;
                return hipLaunchKernel(fn, dim3(grid), dim3(kColThreads), args, 0, stream);
            }
        }
    }
    // two passes over the tensor: amax, then quantization
    const hipError_t e = launch_amax(x, rows, cols, colwise, false, mode == kRHTSR, sign_mask, amax, stream);
    if (e != hipSuccess) return e;
    return launch_quant_1x16(x, rows, cols, colwise, false, mode, amax, sign_mask, rng, codes, scales, g, stream,
                             tiled);
}

hipError_t launch_quant_16x16(const uint16_t* x, int64_t rows, int64_t cols, const float* amax, uint8_t* codes_w,
                              uint8_t* scales_w, float* g_w, uint8_t* codes_wt, uint8_t* scales_wt, float* g_wt,
                              hipStream_t stream) {
    // an orientation is wanted when its g is given (an empty tensor's codes may be NULL)
    if (rows == 0 || cols == 0) {
        hipError_t e = hipSuccess;
        if (g_w) e = write_empty_g(amax, g_w, 1u, stream);
        if (e == hipSuccess && g_wt) e = write_empty_g(amax, g_wt, 1u, stream);
        return e;
    }
    // W alone: the four-over-six band kernel keeping the map-to-6 candidate alone, which is this quantization with
    // g = amax / 2688 (28.8 us against 33.2 us for the kernel below at 14336 x 4096)
    if (!g_wt)
        return launch_quant_4o6_16x16(x, rows, cols, kErrNone, 448, amax, codes_w, scales_w, g_w, codes_wt, scales_wt,
                                      g_wt, stream, false);
    // W^T (and W): tiles of 16 row-blocks, one 1024-thread workgroup per CU, each W^T output row receiving 128
    // contiguous bytes of codes per tile.  Measured at 14336 x 4096 and not kept: tiles of 8 row-blocks with two
    // workgroups per CU (58.5 against 47.6 us: 64-byte runs), of 14 row-blocks (512 tiles, two per CU: 65 against
    // 43.5 us: 112-byte runs that straddle 128-byte lines), and the four-over-six item kernel keeping map-to-6
    // (48.5 us: 256-byte load runs and 64-byte store runs).
    constexpr int kRB = kColRB;
    uint32_t grid;
    const ColGrid w = col_grid(rows, cols, grid, kRB);
    grid = looping_grid(w.ntiles, kColThreads / (64 * kRB));
#define NVFP4_2D(W, T)                                                                                          \
    k_quant_16x16<W, T, kRB><<<grid, 64 * kRB, 0, stream>>>(x, (uint32_t)rows, (uint32_t)cols, w, amax,       \
                                                              codes_w, scales_w, g_w, codes_wt, scales_wt, g_wt)
    if (g_w) NVFP4_2D(true, true);
    else NVFP4_2D(false, true);
#undef NVFP4_2D
    return hipGetLastError();
}

hipError_t launch_quant_4o6_16x16(const void* x, int64_t rows, int64_t cols, ErrMode err, int32_t bound,
                                  const float* amax, uint8_t* codes_w, uint8_t* scales_w, float* g_w,
                                  uint8_t* codes_wt, uint8_t* scales_wt, float* g_wt, hipStream_t stream, bool f32) {
    const float gden = (float)(6 * bound);
    // an orientation is wanted when its g is given (an empty tensor's codes may be NULL)
    if (rows == 0 || cols == 0) {
        hipError_t e = hipSuccess;
        if (g_w) e = write_empty_g(amax, g_w, 1u, stream, gden);
        if (e == hipSuccess && g_wt) e = write_empty_g(amax, g_wt, 1u, stream, gden);
        return e;
    }
    const uint32_t ntc = (uint32_t)(cols / 16), nbands = (uint32_t)(rows / 16);
    const uint4* xv = reinterpret_cast<const uint4*>(x);
    uint2* cw = reinterpret_cast<uint2*>(codes_w);
    uint2* ct = reinterpret_cast<uint2*>(codes_wt);
    // two 1024-thread workgroups per CU, each taking an equal run of consecutive items
    auto grid_of = [](uint32_t items, uint32_t& per) {
        const uint32_t slots = std::min<uint32_t>(items, 2u * (uint32_t)cu_count());
        per = (items + slots - 1) / slots;
        return (items + per - 1) / per;
    };
    if (!g_wt) {   // W only: items of one band by 64 tile columns, grid-stride
        const uint32_t ntg = (ntc + kTilesPerGroup46 - 1) / kTilesPerGroup46, items = nbands * ntg;
        const uint32_t grid = std::min<uint32_t>(items, 2u * (uint32_t)cu_count());
#define NVFP4_46W(F, E) \
    k_quant_4o6_16x16<F, E><<<grid, kThreads16, 0, stream>>>(xv, ntc, ntg, items, gden, amax, cw, scales_w, g_w)
#define NVFP4_46WE(F)                                      \
    do {                                                   \
        if (err == kErrMSE) NVFP4_46W(F, kErrMSE);         \
        else if (err == kErrMAE) NVFP4_46W(F, kErrMAE);    \
        else NVFP4_46W(F, kErrMaxAbs);                     \
    } while (0)
        if (err == kErrNone) NVFP4_46W(false, kErrNone);   // the 16x16 RN quantizer (bf16 only)
        else if (f32) NVFP4_46WE(true);
        else NVFP4_46WE(false);
#undef NVFP4_46WE
#undef NVFP4_46W
        return hipGetLastError();
    }
    // W^T (and W): items of 8 bands by 8 tile columns
    const uint32_t ncg = (ntc + 7) / 8, items = ((nbands + 7) / 8) * ncg;
    uint32_t per;
    const uint32_t grid = grid_of(items, per);
#define NVFP4_46T(F, E, W)                                                                                       \
    k_quant_4o6_16x16t<F, E, W><<<grid, kThreads16, 0, stream>>>(xv, ntc, nbands, ncg, items, per, gden, amax, cw, \
                                                                 scales_w, g_w, ct, scales_wt, g_wt)
#define NVFP4_46TO(F, E)                 \
    do {                                 \
        if (g_w) NVFP4_46T(F, E, true);  \
        else NVFP4_46T(F, E, false);     \
    } while (0)
#define NVFP4_46TE(F)                                      \
    do {                                                   \
        if (err == kErrMSE) NVFP4_46TO(F, kErrMSE);        \
        else if (err == kErrMAE) NVFP4_46TO(F, kErrMAE);   \
        else NVFP4_46TO(F, kErrMaxAbs);                    \
    } while (0)
    if (f32) NVFP4_46TE(true);
    else NVFP4_46TE(false);
#undef NVFP4_46TE
#undef NVFP4_46TO
#undef NVFP4_46T
    return hipGetLastError();
}

hipError_t launch_quant_4o6(const void* x, int64_t rows, int64_t cols, bool per_row, ErrMode err, int32_t bound,
                            const float* amax, uint8_t* codes, uint8_t* scales, float* g, hipStream_t stream,
                            bool f32) {
    const float gden = (float)(6 * bound);
    if (rows == 0 || cols == 0) return write_empty_g(amax, g, per_row ? (uint32_t)rows : 1u, stream, gden);
    const uint32_t bpr = (uint32_t)(cols / 16);
    const uint32_t total = (uint32_t)(rows * bpr);
    const uint4* xv = reinterpret_cast<const uint4*>(x);
    uint2* cv = reinterpret_cast<uint2*>(codes);
    const uint32_t r = (uint32_t)rows;
    const uint32_t grid_rows = (uint32_t)std::min<int64_t>(rows, (int64_t)cu_count() * 16);
    const uint32_t grid_tensor = grid_for(total, kThreads, 8);
#define NVFP4_46(F, E)                                                                                              \
    do {                                                                                                            \
        if (per_row) k_quant_4o6_rows<F, E><<<grid_rows, kThreads4o6Rows, 0, stream>>>(xv, r, bpr, amax, gden, cv, scales, g); \
        else k_quant_4o6_tensor<F, E><<<grid_tensor, kThreads, 0, stream>>>(xv, total, amax, gden, cv, scales, g);     \
    } while (0)
#define NVFP4_46F(F)                                   \
    do {                                               \
        if (err == kErrMSE) NVFP4_46(F, kErrMSE);      \
        else if (err == kErrMAE) NVFP4_46(F, kErrMAE); \
        else NVFP4_46(F, kErrMaxAbs);                  \
    } while (0)
    if (f32) NVFP4_46F(true);
    else NVFP4_46F(false);
#undef NVFP4_46F
#undef NVFP4_46
    return hipGetLastError();
}

hipError_t launch_swizzle_scales(const uint8_t* scales, int64_t rv, int64_t nb, uint8_t* out, hipStream_t stream) {
    if (rv == 0 || nb == 0) return hipSuccess;
    const uint32_t rt = (uint32_t)((rv + 127) / 128), bt = (uint32_t)((nb + 3) / 4);
    const uint32_t gpr = (bt + kSwzTilesPerGroup - 1) / kSwzTilesPerGroup;
    const uint32_t grid = rt * gpr;
    uint4* o = reinterpret_cast<uint4*>(out);
    if (nb % 4 == 0 && reinterpret_cast<uintptr_t>(scales) % 4 == 0)
        k_swizzle_scales<true><<<grid, 256, 0, stream>>>(scales, (uint32_t)rv, (uint32_t)nb, bt, gpr, o);
    else
        k_swizzle_scales<false><<<grid, 256, 0, stream>>>(scales, (uint32_t)rv, (uint32_t)nb, bt, gpr, o);
    return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* g, int64_t rv, int64_t cv,
                             bool per_row, float* y, hipStream_t stream) {
    if (rv == 0 || cv == 0) return hipSuccess;
    const uint32_t bpr = (uint32_t)(cv / 16);
    const uint64_t quarters = (uint64_t)rv * cv / 4;
    const FastDiv fd = make_fastdiv(bpr);
    const uint32_t grid = grid_for(quarters, kThreads * 4, 16);
    const uint16_t* c16 = reinterpret_cast<const uint16_t*>(codes);
    if (per_row)
        k_dequantize<true><<<grid, kThreads, 0, stream>>>(c16, scales, g, quarters, fd, reinterpret_cast<float4*>(y));
    else
        k_dequantize<false><<<grid, kThreads, 0, stream>>>(c16, scales, g, quarters, fd, reinterpret_cast<float4*>(y));
    return hipGetLastError();
}

// Kernel arguments of a grouped launch over the non-empty tensors; wgs(item) gives a tensor's workgroups.
template <typename F>
uint32_t build_group(const GroupTensor* items, int count, GroupArgs& ga, F wgs) {
    ga.count = 0;
    uint32_t total = 0;
    for (int i = 0; i < count; ++i) {
        const GroupTensor& t = items[i];
        if (t.rows == 0 || t.cols == 0) continue;
        GroupItemK& k = ga.it[ga.count++];
        k.x = reinterpret_cast<const uint4*>(t.x);
        k.codes = reinterpret_cast<uint2*>(t.codes);
        k.scales = t.scales;
        k.g = t.g;
        k.amax = t.amax;
        k.rows = (uint32_t)t.rows;
        k.bpr = (uint32_t)(t.cols / 16);
        k.blocks = k.rows * k.bpr;
        k.per_row = make_fastdiv(k.bpr);
        k.sign_mask = t.sign_mask;
        k.rng = rng_args(t.rng);
        k.wg0 = total;
        total += wgs(k);
    }
    ga.total_wg = total;
    return total;
}

uint32_t capped(uint64_t need, uint64_t cap) { return (uint32_t)(need == 0 ? 1 : need < cap ? need : cap); }

hipError_t launch_amax_grouped(const GroupTensor* items, int count, bool per_row, bool use_rht, hipStream_t stream) {
    const uint64_t cus = (uint64_t)cu_count();
    for (int i = 0; i < count; ++i) {   // empty tensors: amax 0 (per tensor, or per row for rows x 0)
        const GroupTensor& t = items[i];
        const uint32_t n = per_row ? (uint32_t)t.rows : 1u;
        if ((t.rows == 0 || t.cols == 0) && n)
            k_fill_zero<<<grid_for(n, kThreads, 1), kThreads, 0, stream>>>(reinterpret_cast<uint32_t*>(t.amax), n);
    }
    GroupArgs ga;
    if (per_row) {
        const uint32_t total = build_group(items, count, ga, [&](const GroupItemK& k) { return capped(k.rows, cus * 16); });
        if (ga.count) {
            if (use_rht) k_amax_grouped_rows<true><<<total, kThreads, 0, stream>>>(ga);
            else k_amax_grouped_rows<false><<<total, kThreads, 0, stream>>>(ga);
        }
    } else {
        // blocks per lane so that the launch has about one workgroup per CU in all (small tensors share the CUs
        // instead of taking one or two workgroups each): 32 tensors of 256 x 1024 take 8 workgroups each
        uint64_t all = 0;
        for (int i = 0; i < count; ++i) all += (uint64_t)items[i].rows * (uint64_t)(items[i].cols / 16);
        const uint64_t pl = std::min<uint64_t>(kRowAmaxPerLane,
                                               std::max<uint64_t>(1, (all + cus * kColThreads - 1) / (cus * kColThreads)));
        const uint64_t per = (uint64_t)kColThreads * pl;
        const uint32_t total = build_group(items, count, ga, [&](const GroupItemK& k) {
            return capped((k.blocks + per - 1) / per, cus);
        });
        ga.per_lane = (uint32_t)pl;
        if (ga.count) {
            k_zero_group_amax<<<1, 64, 0, stream>>>(ga);
            if (use_rht) k_amax_grouped_tensor<true><<<total, kColThreads, 0, stream>>>(ga);
            else k_amax_grouped_tensor<false><<<total, kColThreads, 0, stream>>>(ga);
        }
    }
    return hipGetLastError();
}

hipError_t launch_quant_grouped(const GroupTensor* items, int count, bool per_row, int method, ErrMode err,
                                int32_t bound, hipStream_t stream) {
    const uint64_t cus = (uint64_t)cu_count();
    const float gden = method == kFourOverSix ? (float)(6 * bound) : 2688.0f;
    for (int i = 0; i < count; ++i) {   // empty tensors: only g is written
        const GroupTensor& t = items[i];
        if (t.rows == 0 || t.cols == 0) {
            const hipError_t e = write_empty_g(t.amax, t.g, per_row ? (uint32_t)t.rows : 1u, stream, gden);
            if (e != hipSuccess) return e;
        }
    }
    GroupArgs ga;
    uint32_t total;
    if (method == kFourOverSix && per_row)
        total = build_group(items, count, ga, [&](const GroupItemK& k) { return capped(k.rows, cus * 8); });
    else
        total = build_group(items, count, ga, [&](const GroupItemK& k) {
            return capped((k.blocks + kThreads - 1) / kThreads, cus * 8);
        });
    if (ga.count == 0) return hipGetLastError();
    ga.gden = gden;
#define NVFP4_GQ(M, P) k_quant_grouped<M, P><<<total, kThreads, 0, stream>>>(ga)
#define NVFP4_G46(P)                                                                                         \
    do {                                                                                                     \
        if (err == kErrMSE) k_quant_4o6_grouped<P, kErrMSE><<<total, kThreads, 0, stream>>>(ga);             \
        else if (err == kErrMAE) k_quant_4o6_grouped<P, kErrMAE><<<total, kThreads, 0, stream>>>(ga);        \
        else k_quant_4o6_grouped<P, kErrMaxAbs><<<total, kThreads, 0, stream>>>(ga);                         \
    } while (0)
    switch (method) {
        case kRN: if (per_row) NVFP4_GQ(kRN, true); else NVFP4_GQ(kRN, false); break;
        case kSR: if (per_row) NVFP4_GQ(kSR, true); else NVFP4_GQ(kSR, false); break;
        case kRHTSR: if (per_row) NVFP4_GQ(kRHTSR, true); else NVFP4_GQ(kRHTSR, false); break;
        default:
            if (per_row) NVFP4_G46(true);
            else NVFP4_G46(false);
    }
#undef NVFP4_G46
#undef NVFP4_GQ
    return hipGetLastError();
}

hipError_t launch_dequantize_fused(const uint8_t* codes, const uint8_t* scales, const float* g, int64_t rv,
                                   int64_t cv, bool per_row, bool use_rht, uint32_t sign_mask, bool out_bf16, void* y,
                                   hipStream_t stream) {
    if (rv == 0 || cv == 0) return hipSuccess;
    const uint64_t halves = (uint64_t)rv * cv / 8;
    const FastDiv fd = make_fastdiv((uint32_t)(cv / 16));
    const uint32_t grid = grid_for(halves, kThreads * 4, 16);
    const uint32_t* c32 = reinterpret_cast<const uint32_t*>(codes);
#define NVFP4_DQ(R, B, P) \
    k_dequantize_fused<R, B, P><<<grid, kThreads, 0, stream>>>(c32, scales, g, halves, fd, sign_mask, y)
    const int sel = (use_rht ? 4 : 0) | (out_bf16 ? 2 : 0) | (per_row ? 1 : 0);
    switch (sel) {
        case 0: NVFP4_DQ(false, false, false); break;
        case 1: NVFP4_DQ(false, false, true); break;
        case 2: NVFP4_DQ(false, true, false); break;
        case 3: NVFP4_DQ(false, true, true); break;
        case 4: NVFP4_DQ(true, false, false); break;
        case 5: NVFP4_DQ(true, false, true); break;
        case 6: NVFP4_DQ(true, true, false); break;
        default: NVFP4_DQ(true, true, true); break;
    }
#undef NVFP4_DQ
    return hipGetLastError();
}

}  // namespace nvfp4
