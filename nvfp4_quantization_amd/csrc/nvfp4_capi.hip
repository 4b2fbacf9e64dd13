// nvfp4_capi.hip -- the extern "C" entry points declared in include/nvfp4.h.
//
// Every entry point validates its arguments on the host first (no HIP call happens before validation passes, so
// invalid calls enqueue nothing and touch no device), then hands the work to the launchers in
// nvfp4_kernels.hip on the caller's stream.  There is no fallback path: an unsupported request is an error.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4.h"
#include "nvfp4_launch.h"

namespace {

// Kernels index 16-element blocks with 32-bit integers and add grid strides (< 2^22) to them: at most 2^35
// elements per tensor (64 GiB of bf16) keeps every block index and index + stride below 2^32.
constexpr int64_t kMaxElems = int64_t(1) << 35;
// Column-wise kernels address the rows of up to four row-blocks (64 rows, 128 * cols bytes) with 32-bit offsets from
// a buffer resource.
constexpr int64_t kMaxColwiseCols = int64_t(1) << 25;

#define NVFP4_TRY(expr)                  \
    do {                                 \
        const nvfp4_status st_ = (expr); \
        if (st_ != NVFP4_OK) return st_; \
    } while (0)

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

nvfp4_status check_sizes(int64_t rows, int64_t cols) {
    if (rows < 0 || cols < 0) return NVFP4_ERR_SHAPE;
    if (rows >= kMaxElems || cols >= kMaxElems) return NVFP4_ERR_SHAPE;
    if (rows != 0 && cols > (kMaxElems - 1) / rows) return NVFP4_ERR_SHAPE;
    return NVFP4_OK;
}

// Shape rules of a 1x16 quantization (and of the amax that feeds it).
nvfp4_status check_view(int64_t rows, int64_t cols, nvfp4_orient orient) {
    if (orient == NVFP4_ROWWISE) return (cols % 16) ? NVFP4_ERR_SHAPE : NVFP4_OK;
    if (orient == NVFP4_COLWISE) return (rows % 16 || cols >= kMaxColwiseCols) ? NVFP4_ERR_SHAPE : NVFP4_OK;
    return NVFP4_ERR_UNSUPPORTED;
}

// Four-over-six knobs: a known error measure and a bound B with 6 B exact and B within E4M3's range.
nvfp4_status check_knobs(nvfp4_4o6_error err_mode, int32_t bound) {
    if (err_mode != NVFP4_4O6_MSE && err_mode != NVFP4_4O6_MAE && err_mode != NVFP4_4O6_MAXABS)
        return NVFP4_ERR_UNSUPPORTED;
    return (bound >= 1 && bound <= 448) ? NVFP4_OK : NVFP4_ERR_UNSUPPORTED;
}

nvfp4::ErrMode err_of(nvfp4_4o6_error e) {
    return e == NVFP4_4O6_MSE ? nvfp4::kErrMSE : e == NVFP4_4O6_MAE ? nvfp4::kErrMAE : nvfp4::kErrMaxAbs;
}

nvfp4_status check_gmode(nvfp4_gmode gmode) {
    return (gmode == NVFP4_G_PER_TENSOR || gmode == NVFP4_G_PER_ROW) ? NVFP4_OK : NVFP4_ERR_UNSUPPORTED;
}

// A buffer of n elements: it may be NULL only when n == 0 (torch hands out NULL for empty tensors).
nvfp4_status check_buf(const void* p, int64_t n, uintptr_t align) {
    if (n > 0 && !p) return NVFP4_ERR_NULL;
    if (!aligned(p, align)) return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

// Output of a quantization of the view V = [rv, cv]; tiled_ok: the call can write the tiled scale layout.
nvfp4_status check_out(const nvfp4_out* out, int64_t rv, int64_t cv, nvfp4_gmode gmode, bool tiled_ok = false) {
    if (!out) return NVFP4_ERR_NULL;
    if (out->scale_layout != NVFP4_SCALES_ROWMAJOR && !(tiled_ok && out->scale_layout == NVFP4_SCALES_TILED))
        return NVFP4_ERR_UNSUPPORTED;
    NVFP4_TRY(check_buf(out->codes, rv * (cv / 2), 16));
    NVFP4_TRY(check_buf(out->scales, rv * (cv / 16), 16));
    return check_buf(out->g, gmode == NVFP4_G_PER_ROW ? rv : 1, 4);
}

nvfp4_status check_input(const uint16_t* x, int64_t rows, int64_t cols, const float* amax, int64_t n_amax) {
    NVFP4_TRY(check_buf(x, rows * cols, 16));
    return check_buf(amax, n_amax, 4);
}

int64_t view_rows(int64_t rows, int64_t cols, nvfp4_orient orient) {
    return orient == NVFP4_COLWISE ? cols : rows;
}

static_assert(NVFP4_MAX_GROUP == nvfp4::kMaxGroup, "grouped-call limit");
static_assert(sizeof(nvfp4_out) == 32 && sizeof(nvfp4_group_item) == 88, "the C layouts the binding mirrors");

nvfp4_status check_group(const nvfp4_group_item* items, int32_t count, nvfp4_gmode gmode, bool quantize,
                         nvfp4::GroupTensor* out) {
    if (count < 0 || count > NVFP4_MAX_GROUP) return NVFP4_ERR_SHAPE;
    if (count > 0 && !items) return NVFP4_ERR_NULL;
    NVFP4_TRY(check_gmode(gmode));
    for (int32_t i = 0; i < count; ++i) {
        const nvfp4_group_item& it = items[i];
        NVFP4_TRY(check_sizes(it.rows, it.cols));
        if (it.cols % 16) return NVFP4_ERR_SHAPE;
        NVFP4_TRY(check_input(it.x, it.rows, it.cols, it.amax, gmode == NVFP4_G_PER_ROW ? it.rows : 1));
        if (quantize) NVFP4_TRY(check_out(&it.out, it.rows, it.cols, gmode));
        out[i] = nvfp4::GroupTensor{it.x, it.rows, it.cols, it.amax, it.out.codes, it.out.scales, it.out.g,
                                    it.sign_mask, nvfp4::Philox{it.seed, it.offset}};
    }
    return NVFP4_OK;
}

nvfp4_status done(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP; }

nvfp4_status quantize_1x16(const uint16_t* x, int64_t rows, int64_t cols, nvfp4_orient orient, nvfp4_gmode gmode,
                           const float* amax, nvfp4::Mode mode, uint16_t sign_mask, uint64_t seed, uint64_t offset,
                           const nvfp4_out* out, void* stream) {
    NVFP4_TRY(check_sizes(rows, cols));
    NVFP4_TRY(check_gmode(gmode));
    NVFP4_TRY(check_view(rows, cols, orient));
    const int64_t rv = view_rows(rows, cols, orient), cv = orient == NVFP4_COLWISE ? rows : cols;
    NVFP4_TRY(check_input(x, rows, cols, amax, gmode == NVFP4_G_PER_ROW ? rv : 1));
    NVFP4_TRY(check_out(out, rv, cv, gmode, true));
    return done(nvfp4::launch_quant_1x16(x, rows, cols, orient == NVFP4_COLWISE, gmode == NVFP4_G_PER_ROW, mode,
                                         amax, sign_mask, nvfp4::Philox{seed, offset}, out->codes, out->scales,
                                         out->g, static_cast<hipStream_t>(stream),
                                         out->scale_layout == NVFP4_SCALES_TILED));
}

// Four-over-six with 16x16 tiles (bf16 or binary32 x): W to *row_out and/or W^T to *col_out.
nvfp4_status quantize_4o6_16x16(const void* x, bool f32, int64_t rows, int64_t cols, nvfp4_orient orient,
                                nvfp4_4o6_error err_mode, int32_t bound, const float* amax, const nvfp4_out* row_out,
                                const nvfp4_out* col_out, void* stream) {
    NVFP4_TRY(check_sizes(rows, cols));
    NVFP4_TRY(check_knobs(err_mode, bound));
    if (orient != NVFP4_ROWWISE && orient != NVFP4_COLWISE && orient != NVFP4_BOTH) return NVFP4_ERR_UNSUPPORTED;
    if (rows % 16 || cols % 16) return NVFP4_ERR_SHAPE;
    if (f32) {
        NVFP4_TRY(check_buf(x, rows * cols, 16));
        NVFP4_TRY(check_buf(amax, 1, 4));
    } else {
        NVFP4_TRY(check_input(static_cast<const uint16_t*>(x), rows, cols, amax, 1));
    }
    const bool want_w = orient == NVFP4_ROWWISE || orient == NVFP4_BOTH;
    const bool want_wt = orient == NVFP4_COLWISE || orient == NVFP4_BOTH;
    if (want_w) NVFP4_TRY(check_out(row_out, rows, cols, NVFP4_G_PER_TENSOR));
    if (want_wt) NVFP4_TRY(check_out(col_out, cols, rows, NVFP4_G_PER_TENSOR));
    return done(nvfp4::launch_quant_4o6_16x16(
        x, rows, cols, err_of(err_mode), bound, amax, want_w ? row_out->codes : nullptr,
        want_w ? row_out->scales : nullptr, want_w ? row_out->g : nullptr, want_wt ? col_out->codes : nullptr,
        want_wt ? col_out->scales : nullptr, want_wt ? col_out->g : nullptr, static_cast<hipStream_t>(stream), f32));
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_amax(const uint16_t* x, int64_t rows, int64_t cols, nvfp4_orient orient, nvfp4_gmode gmode,
                        int use_rht, uint16_t sign_mask, float* amax, void* stream) {
    NVFP4_TRY(check_sizes(rows, cols));
    NVFP4_TRY(check_gmode(gmode));
    NVFP4_TRY(check_view(rows, cols, orient));
    NVFP4_TRY(check_input(x, rows, cols, amax, gmode == NVFP4_G_PER_ROW ? view_rows(rows, cols, orient) : 1));
    return done(nvfp4::launch_amax(x, rows, cols, orient == NVFP4_COLWISE, gmode == NVFP4_G_PER_ROW, use_rht != 0,
                                   sign_mask, amax, static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_quantize_rn(const uint16_t* x, int64_t rows, int64_t cols, nvfp4_block block,
                               nvfp4_orient orient, nvfp4_gmode gmode, const float* amax, const nvfp4_out* row_out,
                               const nvfp4_out* col_out, void* stream) {
    if (block == NVFP4_BLOCK_1X16) {
        if (orient == NVFP4_ROWWISE)
            return quantize_1x16(x, rows, cols, orient, gmode, amax, nvfp4::kRN, 0, 0, 0, row_out, stream);
        if (orient == NVFP4_COLWISE)
            return quantize_1x16(x, rows, cols, orient, gmode, amax, nvfp4::kRN, 0, 0, 0, col_out, stream);
        return NVFP4_ERR_UNSUPPORTED;
    }
    if (block != NVFP4_BLOCK_16X16) return NVFP4_ERR_UNSUPPORTED;
    NVFP4_TRY(check_sizes(rows, cols));
    NVFP4_TRY(check_gmode(gmode));
    if (gmode != NVFP4_G_PER_TENSOR) return NVFP4_ERR_UNSUPPORTED;
    if (orient != NVFP4_ROWWISE && orient != NVFP4_COLWISE && orient != NVFP4_BOTH) return NVFP4_ERR_UNSUPPORTED;
    if (rows % 16 || cols % 16 || cols >= kMaxColwiseCols) return NVFP4_ERR_SHAPE;
    NVFP4_TRY(check_input(x, rows, cols, amax, 1));
    const bool want_w = orient == NVFP4_ROWWISE || orient == NVFP4_BOTH;
    const bool want_wt = orient == NVFP4_COLWISE || orient == NVFP4_BOTH;
    if (want_w) NVFP4_TRY(check_out(row_out, rows, cols, gmode));
    if (want_wt) NVFP4_TRY(check_out(col_out, cols, rows, gmode));
    return done(nvfp4::launch_quant_16x16(
        x, rows, cols, amax, want_w ? row_out->codes : nullptr, want_w ? row_out->scales : nullptr,
        want_w ? row_out->g : nullptr, want_wt ? col_out->codes : nullptr, want_wt ? col_out->scales : nullptr,
        want_wt ? col_out->g : nullptr, static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_quantize_sr(const uint16_t* x, int64_t rows, int64_t cols, nvfp4_orient orient,
                               nvfp4_gmode gmode, const float* amax, uint64_t seed, uint64_t offset,
                               const nvfp4_out* out, void* stream) {
    return quantize_1x16(x, rows, cols, orient, gmode, amax, nvfp4::kSR, 0, seed, offset, out, stream);
}

nvfp4_status nvfp4_quantize_rht_sr(const uint16_t* x, int64_t rows, int64_t cols, nvfp4_orient orient,
                                   nvfp4_gmode gmode, const float* amax, uint16_t sign_mask, uint64_t seed,
                                   uint64_t offset, const nvfp4_out* out, void* stream) {
    return quantize_1x16(x, rows, cols, orient, gmode, amax, nvfp4::kRHTSR, sign_mask, seed, offset, out, stream);
}

nvfp4_status nvfp4_amax_quantize(const uint16_t* x, int64_t rows, int64_t cols, nvfp4_orient orient,
                                 nvfp4_rounding rounding, uint16_t sign_mask, uint64_t seed, uint64_t offset,
                                 float* amax, const nvfp4_out* out, void* stream) {
    if (rounding != NVFP4_ROUND_RN && rounding != NVFP4_ROUND_SR && rounding != NVFP4_ROUND_RHT_SR)
        return NVFP4_ERR_UNSUPPORTED;
    NVFP4_TRY(check_sizes(rows, cols));
    NVFP4_TRY(check_view(rows, cols, orient));
    const int64_t rv = view_rows(rows, cols, orient), cv = orient == NVFP4_COLWISE ? rows : cols;
    NVFP4_TRY(check_input(x, rows, cols, amax, 1));
    NVFP4_TRY(check_out(out, rv, cv, NVFP4_G_PER_TENSOR, true));
    const nvfp4::Mode mode = rounding == NVFP4_ROUND_RN ? nvfp4::kRN : rounding == NVFP4_ROUND_SR ? nvfp4::kSR
                                                                                                  : nvfp4::kRHTSR;
    return done(nvfp4::launch_amax_quant(x, rows, cols, orient == NVFP4_COLWISE, mode, sign_mask,
                                         nvfp4::Philox{seed, offset}, amax, out->codes, out->scales, out->g,
                                         static_cast<hipStream_t>(stream), out->scale_layout == NVFP4_SCALES_TILED));
}

nvfp4_status nvfp4_quantize_4o6(const uint16_t* x, int64_t rows, int64_t cols, nvfp4_gmode gmode,
                                nvfp4_4o6_error err_mode, int32_t bound, const float* amax, const nvfp4_out* out,
                                void* stream) {
    NVFP4_TRY(check_sizes(rows, cols));
    NVFP4_TRY(check_gmode(gmode));
    NVFP4_TRY(check_knobs(err_mode, bound));
    if (cols % 16) return NVFP4_ERR_SHAPE;
    NVFP4_TRY(check_input(x, rows, cols, amax, gmode == NVFP4_G_PER_ROW ? rows : 1));
    NVFP4_TRY(check_out(out, rows, cols, gmode));
    return done(nvfp4::launch_quant_4o6(x, rows, cols, gmode == NVFP4_G_PER_ROW, err_of(err_mode), bound, amax,
                                        out->codes, out->scales, out->g, static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_quantize_4o6_16x16(const uint16_t* x, int64_t rows, int64_t cols, nvfp4_orient orient,
                                      nvfp4_4o6_error err_mode, int32_t bound, const float* amax,
                                      const nvfp4_out* row_out, const nvfp4_out* col_out, void* stream) {
    return quantize_4o6_16x16(x, false, rows, cols, orient, err_mode, bound, amax, row_out, col_out, stream);
}

nvfp4_status nvfp4_amax_f32(const float* x, int64_t rows, int64_t cols, nvfp4_gmode gmode, float* amax, void* stream) {
    NVFP4_TRY(check_sizes(rows, cols));
    NVFP4_TRY(check_gmode(gmode));
    if (cols % 16) return NVFP4_ERR_SHAPE;
    NVFP4_TRY(check_buf(x, rows * cols, 16));
    NVFP4_TRY(check_buf(amax, gmode == NVFP4_G_PER_ROW ? rows : 1, 4));
    return done(nvfp4::launch_amax_f32(x, rows, cols, gmode == NVFP4_G_PER_ROW, amax, static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_quantize_4o6_f32(const float* x, int64_t rows, int64_t cols, nvfp4_gmode gmode,
                                    nvfp4_4o6_error err_mode, int32_t bound, const float* amax,
                                    const nvfp4_out* out, void* stream) {
    NVFP4_TRY(check_sizes(rows, cols));
    NVFP4_TRY(check_gmode(gmode));
    NVFP4_TRY(check_knobs(err_mode, bound));
    if (cols % 16) return NVFP4_ERR_SHAPE;
    NVFP4_TRY(check_buf(x, rows * cols, 16));
    NVFP4_TRY(check_buf(amax, gmode == NVFP4_G_PER_ROW ? rows : 1, 4));
    NVFP4_TRY(check_out(out, rows, cols, gmode));
    return done(nvfp4::launch_quant_4o6(x, rows, cols, gmode == NVFP4_G_PER_ROW, err_of(err_mode), bound, amax,
                                        out->codes, out->scales, out->g, static_cast<hipStream_t>(stream), true));
}

nvfp4_status nvfp4_quantize_4o6_16x16_f32(const float* x, int64_t rows, int64_t cols, nvfp4_orient orient,
                                          nvfp4_4o6_error err_mode, int32_t bound, const float* amax,
                                          const nvfp4_out* row_out, const nvfp4_out* col_out, void* stream) {
    return quantize_4o6_16x16(x, true, rows, cols, orient, err_mode, bound, amax, row_out, col_out, stream);
}

nvfp4_status nvfp4_dequantize(const nvfp4_out* in, int64_t rv, int64_t cv, nvfp4_gmode gmode, float* y,
                              void* stream) {
    NVFP4_TRY(check_sizes(rv, cv));
    NVFP4_TRY(check_gmode(gmode));
    if (cv % 16) return NVFP4_ERR_SHAPE;
    NVFP4_TRY(check_out(in, rv, cv, gmode));
    NVFP4_TRY(check_buf(y, rv * cv, 16));
    return done(nvfp4::launch_dequantize(in->codes, in->scales, in->g, rv, cv, gmode == NVFP4_G_PER_ROW, y,
                                         static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_swizzle_scales(const uint8_t* scales, int64_t rv, int64_t nb, uint8_t* out, void* stream) {
    if (rv < 0 || nb < 0 || rv >= kMaxElems / 16 || nb >= kMaxElems / 16) return NVFP4_ERR_SHAPE;
    if (rv != 0 && nb > (kMaxElems / 16 - 1) / rv) return NVFP4_ERR_SHAPE;
    NVFP4_TRY(check_buf(scales, rv * nb, 1));
    NVFP4_TRY(check_buf(out, nvfp4_swizzled_scales_size(rv, nb), 16));
    return done(nvfp4::launch_swizzle_scales(scales, rv, nb, out, static_cast<hipStream_t>(stream)));
}

int64_t nvfp4_swizzled_scales_size(int64_t rv, int64_t nb) {
    if (rv < 0 || nb < 0) return 0;
    return (rv + 127) / 128 * 128 * ((nb + 3) / 4 * 4);
}

nvfp4_status nvfp4_amax_grouped(const nvfp4_group_item* items, int32_t count, nvfp4_gmode gmode, int use_rht,
                                void* stream) {
    nvfp4::GroupTensor t[NVFP4_MAX_GROUP];
    NVFP4_TRY(check_group(items, count, gmode, false, t));
    if (count == 0) return NVFP4_OK;
    return done(nvfp4::launch_amax_grouped(t, count, gmode == NVFP4_G_PER_ROW, use_rht != 0,
                                           static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_quantize_grouped(const nvfp4_group_item* items, int32_t count, nvfp4_gmode gmode,
                                    nvfp4_rounding rounding, nvfp4_4o6_error err_mode, int32_t bound,
                                    void* stream) {
    if (rounding != NVFP4_ROUND_RN && rounding != NVFP4_ROUND_SR && rounding != NVFP4_ROUND_RHT_SR &&
        rounding != NVFP4_ROUND_4O6)
        return NVFP4_ERR_UNSUPPORTED;
    if (rounding == NVFP4_ROUND_4O6) NVFP4_TRY(check_knobs(err_mode, bound));
    nvfp4::GroupTensor t[NVFP4_MAX_GROUP];
    NVFP4_TRY(check_group(items, count, gmode, true, t));
    if (count == 0) return NVFP4_OK;
    const int method = rounding == NVFP4_ROUND_RN ? nvfp4::kRN : rounding == NVFP4_ROUND_SR ? nvfp4::kSR
                       : rounding == NVFP4_ROUND_RHT_SR ? nvfp4::kRHTSR : nvfp4::kFourOverSix;
    return done(nvfp4::launch_quant_grouped(t, count, gmode == NVFP4_G_PER_ROW, method, err_of(err_mode), bound,
                                            static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_dequantize_fused(const nvfp4_out* in, int64_t rv, int64_t cv, nvfp4_gmode gmode, int use_rht,
                                    uint16_t sign_mask, int out_bf16, void* y, void* stream) {
    NVFP4_TRY(check_sizes(rv, cv));
    NVFP4_TRY(check_gmode(gmode));
    if (cv % 16) return NVFP4_ERR_SHAPE;
    NVFP4_TRY(check_out(in, rv, cv, gmode));
    NVFP4_TRY(check_buf(y, rv * cv, 16));
    return done(nvfp4::launch_dequantize_fused(in->codes, in->scales, in->g, rv, cv, gmode == NVFP4_G_PER_ROW,
                                               use_rht != 0, sign_mask, out_bf16 != 0, y,
                                               static_cast<hipStream_t>(stream)));
}

const char* nvfp4_status_str(nvfp4_status status) {
    switch (status) {
        case NVFP4_OK: return "NVFP4_OK";
        case NVFP4_ERR_NULL: return "NVFP4_ERR_NULL: a required pointer is NULL";
        case NVFP4_ERR_SHAPE: return "NVFP4_ERR_SHAPE: unsupported size";
        case NVFP4_ERR_ALIGN: return "NVFP4_ERR_ALIGN: misaligned pointer";
        case NVFP4_ERR_UNSUPPORTED: return "NVFP4_ERR_UNSUPPORTED: unsupported option or combination";
        case NVFP4_ERR_HIP: return "NVFP4_ERR_HIP: kernel launch failed";
    }
    return "unknown nvfp4_status";
}

}  // extern "C"
