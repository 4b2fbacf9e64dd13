"""MI355X-native (gfx950, HIP) NVFP4 training quantizer.

The compute lives in the HIP library built from ``csrc/`` (C ABI: ``include/nvfp4.h``); this package is its thin
Python binding (``binding``), the hipcc build step (``_build``) and the seeded synthetic inputs used by the tests
and the benchmark (``workloads``).
"""
from .binding import (  # noqa: F401
    BLOCK_1X16, BLOCK_16X16, BOTH, BOUND_HEADROOM, BOUND_STD, COLWISE, ERR_MAE, ERR_MAXABS, ERR_MSE, G_PER_ROW, G_PER_TENSOR, MAX_GROUP, ROUND_4O6, ROUND_RHT_SR, ROUND_RN,
    ROUND_SR, ROWWISE, SCALES_ROWMAJOR, SCALES_TILED, NVFP4Error, Quantized, alloc_out, nvfp4_amax, nvfp4_amax_grouped, nvfp4_amax_quantize,
    nvfp4_dequantize, nvfp4_dequantize_fused, nvfp4_amax_f32, nvfp4_quantize_4o6, nvfp4_quantize_4o6_16x16, nvfp4_quantize_4o6_16x16_f32, nvfp4_quantize_4o6_f32, nvfp4_quantize_grouped, nvfp4_quantize_rht_sr,
    nvfp4_quantize_rn, nvfp4_quantize_sr, nvfp4_swizzle_scales, nvfp4_swizzled_scales_size, view_shape,
)
