// nvfp4_launch.h -- internal interface between the C-ABI shim (nvfp4_capi.hip) and the kernels
// (nvfp4_kernels.hip).  Arguments reaching these launchers have already been validated; each launcher only
// enqueues work on `stream` and returns the HIP error of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

enum Mode : int { kRN = 0, kSR = 1, kRHTSR = 2 };

// Four-over-six error measure of a candidate: sum of squared differences, sum of magnitudes, largest magnitude.
// kErrNone (internal) keeps the map-to-6 candidate alone: the standard NVFP4 quantization with g = amax / (6 B).
enum ErrMode : int { kErrMSE = 0, kErrMAE = 1, kErrMaxAbs = 2, kErrNone = 3 };

struct Philox {
    uint64_t seed;
    uint64_t offset;
};

// Grouped launches: at most this many tensors per launch (their descriptors travel as kernel arguments).
constexpr int kMaxGroup = 32;

// One row-wise tensor of a grouped launch (amax [1] or [rows]; codes/scales/g unused by the amax launch).
struct GroupTensor {
    const uint16_t* x;
    int64_t rows, cols;
    float* amax;
    uint8_t* codes;
    uint8_t* scales;
    float* g;
    uint32_t sign_mask;
    Philox rng;
};

// amax of V (row-wise: V = X, column-wise: V = X^T); per_row selects one value per row of V.
hipError_t launch_amax(const uint16_t* x, int64_t rows, int64_t cols, bool colwise, bool per_row, bool use_rht,
                       uint32_t sign_mask, float* amax, hipStream_t stream);

// 1x16 quantization of V (RN, SR or RHT+SR).  tiled (column-wise only): scales in the FP4 GEMM's tiled layout
// (128 x 4 tiles, [32][4][4] bytes each, zero padding) instead of [Rv, Cv/16].
hipError_t launch_quant_1x16(const uint16_t* x, int64_t rows, int64_t cols, bool colwise, bool per_row, Mode mode,
                             const float* amax, uint32_t sign_mask, Philox rng, uint8_t* codes, uint8_t* scales,
                             float* g, hipStream_t stream, bool tiled = false);

// amax and 1x16 quantization of V with a per-tensor g: one read of X when the tensor fits one workgroup per CU,
// else the two launches above.  tiled as for launch_quant_1x16.
hipError_t launch_amax_quant(const uint16_t* x, int64_t rows, int64_t cols, bool colwise, Mode mode, uint32_t sign_mask,
                             Philox rng, float* amax, uint8_t* codes, uint8_t* scales, float* g, hipStream_t stream,
                             bool tiled = false);

// 16x16 RN quantization; either output (g == nullptr) may be skipped.
hipError_t launch_quant_16x16(const uint16_t* x, int64_t rows, int64_t cols, const float* amax, uint8_t* codes_w,
                              uint8_t* scales_w, float* g_w, uint8_t* codes_wt, uint8_t* scales_wt, float* g_wt,
                              hipStream_t stream);

// Four-over-six with 16x16 tiles, per-tensor g = amax / (6 bound): W (codes packed along X's rows) and/or W^T
// (along X's columns), each tile's scale repeated per row; either output (g == nullptr) may be skipped.
hipError_t launch_quant_4o6_16x16(const void* x, int64_t rows, int64_t cols, ErrMode err, int32_t bound,
                                  const float* amax, uint8_t* codes_w, uint8_t* scales_w, float* g_w,
                                  uint8_t* codes_wt, uint8_t* scales_wt, float* g_wt, hipStream_t stream,
                                  bool f32 = false);

// Four-over-six, row-wise 1x16 RN, g = amax / (6 bound).
hipError_t launch_quant_4o6(const void* x, int64_t rows, int64_t cols, bool per_row, ErrMode err, int32_t bound,
                            const float* amax, uint8_t* codes, uint8_t* scales, float* g, hipStream_t stream,
                            bool f32 = false);

// Row-wise amax of a binary32 tensor (per tensor or per row), for the binary32 four-over-six input.
hipError_t launch_amax_f32(const float* x, int64_t rows, int64_t cols, bool per_row, float* amax, hipStream_t stream);

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* g, int64_t rv, int64_t cv,
                             bool per_row, float* y, hipStream_t stream);

// Grouped row-wise amax and quantization (method: kRN, kSR, kRHTSR, or kFourOverSix); each tensor's result equals
// that of the single-tensor launch.
constexpr int kFourOverSix = 3;
hipError_t launch_amax_grouped(const GroupTensor* items, int count, bool per_row, bool use_rht, hipStream_t stream);
hipError_t launch_quant_grouped(const GroupTensor* items, int count, bool per_row, int method, ErrMode err,
                                int32_t bound, hipStream_t stream);

// Decode with an optional inverse RHT; y is float or bf16 bits.
// Scale matrix [rv, nb] -> tiled layout of the FP4 GEMM (out: ceil(rv/128) * 128 * ceil(nb/4) * 4 bytes).
hipError_t launch_swizzle_scales(const uint8_t* scales, int64_t rv, int64_t nb, uint8_t* out, hipStream_t stream);

hipError_t launch_dequantize_fused(const uint8_t* codes, const uint8_t* scales, const float* g, int64_t rv,
                                   int64_t cv, bool per_row, bool use_rht, uint32_t sign_mask, bool out_bf16, void* y,
                                   hipStream_t stream);

}  // namespace nvfp4
