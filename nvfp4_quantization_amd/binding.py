"""Thin Python binding over the C ABI of ``include/nvfp4.h`` (ctypes).

Argument marshalling only: tensors must already live on the GPU; this module checks the dtype, the number of
elements and the contiguity of every tensor it hands to the library (a wrong-sized buffer would otherwise be read
or written past its end by the kernels), allocates missing outputs with torch (device memory is torch's job),
passes raw pointers and the current HIP stream, and turns a non-zero ``nvfp4_status`` into an exception.  Every
step of the method runs in the HIP library; there is no CPU path.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import NamedTuple, Optional

import torch

from ._build import LIB_PATH

ROWWISE, COLWISE, BOTH = 1, 2, 3
BLOCK_1X16, BLOCK_16X16 = 0, 1
G_PER_TENSOR, G_PER_ROW = 0, 1
ROUND_RN, ROUND_SR, ROUND_RHT_SR, ROUND_4O6 = 0, 1, 2, 3
MAX_GROUP = 32
SCALES_ROWMAJOR, SCALES_TILED = 0, 1
ERR_MSE, ERR_MAE, ERR_MAXABS = 0, 1, 2          # four-over-six error measures (nvfp4_4o6_error)
BOUND_STD, BOUND_HEADROOM = 448, 256           # four-over-six bounds: g = amax / (6 bound)

STATUS = {0: "NVFP4_OK", 1: "NVFP4_ERR_NULL", 2: "NVFP4_ERR_SHAPE", 3: "NVFP4_ERR_ALIGN",
          4: "NVFP4_ERR_UNSUPPORTED", 5: "NVFP4_ERR_HIP"}

# name -> (restype, argtypes); the same names and order as include/nvfp4.h
_P, _I64, _U64, _U16, _I, _I32 = C.c_void_p, C.c_int64, C.c_uint64, C.c_uint16, C.c_int, C.c_int32
SIGNATURES = {
    "nvfp4_amax": (_I, [_P, _I64, _I64, _I, _I, _I, _U16, _P, _P]),
    "nvfp4_quantize_rn": (_I, [_P, _I64, _I64, _I, _I, _I, _P, _P, _P, _P]),
    "nvfp4_quantize_sr": (_I, [_P, _I64, _I64, _I, _I, _P, _U64, _U64, _P, _P]),
    "nvfp4_quantize_rht_sr": (_I, [_P, _I64, _I64, _I, _I, _P, _U16, _U64, _U64, _P, _P]),
    "nvfp4_amax_quantize": (_I, [_P, _I64, _I64, _I, _I, _U16, _U64, _U64, _P, _P, _P]),
    "nvfp4_quantize_4o6": (_I, [_P, _I64, _I64, _I, _I, _I32, _P, _P, _P]),
    "nvfp4_quantize_4o6_16x16": (_I, [_P, _I64, _I64, _I, _I, _I32, _P, _P, _P, _P]),
    "nvfp4_quantize_4o6_f32": (_I, [_P, _I64, _I64, _I, _I, _I32, _P, _P, _P]),
    "nvfp4_quantize_4o6_16x16_f32": (_I, [_P, _I64, _I64, _I, _I, _I32, _P, _P, _P, _P]),
    "nvfp4_amax_f32": (_I, [_P, _I64, _I64, _I, _P, _P]),
    "nvfp4_dequantize": (_I, [_P, _I64, _I64, _I, _P, _P]),
    "nvfp4_dequantize_fused": (_I, [_P, _I64, _I64, _I, _I, _U16, _I, _P, _P]),
    "nvfp4_swizzle_scales": (_I, [_P, _I64, _I64, _P, _P]),
    "nvfp4_swizzled_scales_size": (_I64, [_I64, _I64]),
    "nvfp4_amax_grouped": (_I, [_P, C.c_int32, _I, _I, _P]),
    "nvfp4_quantize_grouped": (_I, [_P, _I32, _I, _I, _I, _I32, _P]),
    "nvfp4_status_str": (C.c_char_p, [_I]),
}


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}")
        self.status = status


class _Out(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("g", C.c_void_p), ("scale_layout", C.c_int32)]


class _GroupItem(C.Structure):
    _fields_ = [("x", C.c_void_p), ("rows", C.c_int64), ("cols", C.c_int64), ("amax", C.c_void_p), ("out", _Out),
                ("sign_mask", C.c_uint16), ("seed", C.c_uint64), ("offset", C.c_uint64)]


class Quantized(NamedTuple):
    codes: torch.Tensor   # [Rv, Cv/2] uint8
    scales: torch.Tensor  # [Rv, Cv/16] uint8 (E4M3 codes), or flat in the tiled layout (scale_layout SCALES_TILED)
    g: torch.Tensor       # [1] or [Rv] float32
    scale_layout: int = 0


_lib: Optional[C.CDLL] = None


def lib() -> C.CDLL:
    """Load the in-tree HIP library (it must have been built: ``python -m nvfp4_quantization_amd._build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"NVFP4 HIP library not built: {LIB_PATH} is missing "
                               "(run python -m nvfp4_quantization_amd._build)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int, where: str) -> None:
    if status != 0:
        raise NVFP4Error(status, where)


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _dev(t: torch.Tensor, what: str, dtypes=None, numel: Optional[int] = None, at_least: bool = False) -> int:
    """Device pointer of t after checking it: a tensor of one of dtypes, with exactly numel elements (at least numel
    with at_least), contiguous, on the GPU.  The checks that need no GPU come first."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{what} must have dtype {' or '.join(str(d) for d in dtypes)}, not {t.dtype}")
    if numel is not None and (t.numel() < numel if at_least else t.numel() != numel):
        raise ValueError(f"{what} must hold {'at least ' if at_least else ''}{numel} elements, not {t.numel()} "
                         f"(shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if not t.is_cuda:
        raise TypeError(f"{what} must be a GPU tensor")
    return t.data_ptr()


def _f32buf(t: torch.Tensor, what: str, n: int) -> int:
    return _dev(t, what, (torch.float32,), n)


def _bf16(x: torch.Tensor) -> int:
    if not isinstance(x, torch.Tensor) or x.dtype not in _BF16 or x.dim() != 2:
        raise TypeError("x must be a 2-D bf16 tensor (or its int16 bit patterns)")
    return _dev(x, "x")


def _stream(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def view_shape(rows: int, cols: int, orient: int) -> tuple[int, int]:
    return (rows, cols) if orient == ROWWISE else (cols, rows)


def alloc_out(rv: int, cv: int, gmode: int, device, scale_layout: int = SCALES_ROWMAJOR) -> Quantized:
    scales = (torch.empty((rv, cv // 16), dtype=torch.uint8, device=device) if scale_layout == SCALES_ROWMAJOR
              else torch.empty((nvfp4_swizzled_scales_size(rv, cv // 16),), dtype=torch.uint8, device=device))
    return Quantized(torch.empty((rv, cv // 2), dtype=torch.uint8, device=device), scales,
                     torch.empty((rv if gmode == G_PER_ROW else 1,), dtype=torch.float32, device=device), scale_layout)


def _out(o: Optional[Quantized], rv: int, cv: int, gmode: int):
    """The C struct of an output for the view [rv, cv], after checking every buffer's dtype and size."""
    if o is None:
        return None
    if o.scale_layout not in (SCALES_ROWMAJOR, SCALES_TILED):
        raise ValueError(f"unknown scale layout {o.scale_layout}")
    n_sc = rv * (cv // 16) if o.scale_layout == SCALES_ROWMAJOR else nvfp4_swizzled_scales_size(rv, cv // 16)
    return C.byref(_Out(_dev(o.codes, "codes", (torch.uint8,), rv * (cv // 2)),
                        _dev(o.scales, "scales", (torch.uint8,), n_sc),
                        _f32buf(o.g, "g", rv if gmode == G_PER_ROW else 1), o.scale_layout))


def _amax_n(rv: int, gmode: int) -> int:
    return rv if gmode == G_PER_ROW else 1


def nvfp4_amax(x: torch.Tensor, orient: int = ROWWISE, gmode: int = G_PER_TENSOR, use_rht: bool = False,
               sign_mask: int = 0, amax: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    rows, cols = x.shape
    rv, _ = view_shape(rows, cols, orient)
    if amax is None:
        amax = torch.empty((rv if gmode == G_PER_ROW else 1,), dtype=torch.float32, device=x.device)
    _check(lib().nvfp4_amax(_bf16(x), rows, cols, orient, gmode, int(bool(use_rht)), sign_mask & 0xFFFF,
                            _f32buf(amax, "amax", _amax_n(rv, gmode)), _stream(x.device, stream)), "nvfp4_amax")
    return amax


def nvfp4_quantize_rn(x: torch.Tensor, amax: torch.Tensor, block: int = BLOCK_1X16, orient: int = ROWWISE,
                      gmode: int = G_PER_TENSOR, row_out: Optional[Quantized] = None,
                      col_out: Optional[Quantized] = None, stream=None):
    """Returns (row_out, col_out); the orientation(s) not requested are None."""
    rows, cols = x.shape
    want_row = orient in (ROWWISE, BOTH)
    want_col = orient in (COLWISE, BOTH)
    if want_row and row_out is None:
        row_out = alloc_out(rows, cols, gmode, x.device)
    if want_col and col_out is None:
        col_out = alloc_out(cols, rows, gmode, x.device)
    n_amax = _amax_n(rows if orient == ROWWISE else cols, gmode)
    _check(lib().nvfp4_quantize_rn(_bf16(x), rows, cols, block, orient, gmode, _f32buf(amax, "amax", n_amax),
                                   _out(row_out if want_row else None, rows, cols, gmode),
                                   _out(col_out if want_col else None, cols, rows, gmode),
                                   _stream(x.device, stream)), "nvfp4_quantize_rn")
    return (row_out if want_row else None), (col_out if want_col else None)


def nvfp4_quantize_sr(x: torch.Tensor, amax: torch.Tensor, seed: int, offset: int, orient: int = ROWWISE,
                      gmode: int = G_PER_TENSOR, out: Optional[Quantized] = None, stream=None) -> Quantized:
    rows, cols = x.shape
    rv, cv = view_shape(rows, cols, orient)
    if out is None:
        out = alloc_out(rv, cv, gmode, x.device)
    _check(lib().nvfp4_quantize_sr(_bf16(x), rows, cols, orient, gmode, _f32buf(amax, "amax", _amax_n(rv, gmode)),
                                   seed, offset, _out(out, rv, cv, gmode), _stream(x.device, stream)),
           "nvfp4_quantize_sr")
    return out


def nvfp4_quantize_rht_sr(x: torch.Tensor, amax: torch.Tensor, sign_mask: int, seed: int, offset: int,
                          orient: int = ROWWISE, gmode: int = G_PER_TENSOR, out: Optional[Quantized] = None,
                          stream=None) -> Quantized:
    rows, cols = x.shape
    rv, cv = view_shape(rows, cols, orient)
    if out is None:
        out = alloc_out(rv, cv, gmode, x.device)
    _check(lib().nvfp4_quantize_rht_sr(_bf16(x), rows, cols, orient, gmode, _f32buf(amax, "amax", _amax_n(rv, gmode)),
                                       sign_mask & 0xFFFF, seed, offset, _out(out, rv, cv, gmode),
                                       _stream(x.device, stream)), "nvfp4_quantize_rht_sr")
    return out


def nvfp4_amax_quantize(x: torch.Tensor, orient: int, rounding: int, sign_mask: int = 0, seed: int = 0,
                        offset: int = 0, amax: Optional[torch.Tensor] = None, out: Optional[Quantized] = None,
                        stream=None) -> tuple[torch.Tensor, Quantized]:
    """amax and 1x16 quantization with a per-tensor g in one call; returns (amax, out)."""
    rows, cols = x.shape
    rv, cv = view_shape(rows, cols, orient)
    if amax is None:
        amax = torch.empty((1,), dtype=torch.float32, device=x.device)
    if out is None:
        out = alloc_out(rv, cv, G_PER_TENSOR, x.device)
    _check(lib().nvfp4_amax_quantize(_bf16(x), rows, cols, orient, rounding, sign_mask & 0xFFFF, seed, offset,
                                     _f32buf(amax, "amax", 1), _out(out, rv, cv, G_PER_TENSOR),
                                     _stream(x.device, stream)), "nvfp4_amax_quantize")
    return amax, out


def nvfp4_quantize_4o6(x: torch.Tensor, amax: torch.Tensor, gmode: int = G_PER_ROW,
                       out: Optional[Quantized] = None, stream=None, err_mode: int = ERR_MSE,
                       bound: int = BOUND_STD) -> Quantized:
    """Four-over-six, row-wise 1x16 (err_mode ERR_MSE, ERR_MAE or ERR_MAXABS; g = amax / (6 bound))."""
    rows, cols = x.shape
    if out is None:
        out = alloc_out(rows, cols, gmode, x.device)
    _check(lib().nvfp4_quantize_4o6(_bf16(x), rows, cols, gmode, err_mode, bound,
                                    _f32buf(amax, "amax", _amax_n(rows, gmode)), _out(out, rows, cols, gmode),
                                    _stream(x.device, stream)), "nvfp4_quantize_4o6")
    return out


def _f32(x: torch.Tensor) -> int:
    if not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or x.dim() != 2:
        raise TypeError("x must be a 2-D float32 tensor")
    return _dev(x, "x")


def nvfp4_amax_f32(x: torch.Tensor, gmode: int = G_PER_TENSOR, amax: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    rows, cols = x.shape
    if amax is None:
        amax = torch.empty((rows if gmode == G_PER_ROW else 1,), dtype=torch.float32, device=x.device)
    _check(lib().nvfp4_amax_f32(_f32(x), rows, cols, gmode, _f32buf(amax, "amax", _amax_n(rows, gmode)),
                                _stream(x.device, stream)), "nvfp4_amax_f32")
    return amax


def nvfp4_quantize_4o6_f32(x: torch.Tensor, amax: torch.Tensor, gmode: int = G_PER_ROW,
                           out: Optional[Quantized] = None, stream=None, err_mode: int = ERR_MSE,
                           bound: int = BOUND_STD) -> Quantized:
    """Four-over-six of a float32 tensor (row-wise 1x16)."""
    rows, cols = x.shape
    if out is None:
        out = alloc_out(rows, cols, gmode, x.device)
    _check(lib().nvfp4_quantize_4o6_f32(_f32(x), rows, cols, gmode, err_mode, bound,
                                        _f32buf(amax, "amax", _amax_n(rows, gmode)), _out(out, rows, cols, gmode),
                                        _stream(x.device, stream)), "nvfp4_quantize_4o6_f32")
    return out


def _quantize_4o6_16x16(fn, name, xp, rows, cols, device, amax, orient, err_mode, bound, row_out, col_out, stream):
    want_row, want_col = orient in (ROWWISE, BOTH), orient in (COLWISE, BOTH)
    if want_row and row_out is None:
        row_out = alloc_out(rows, cols, G_PER_TENSOR, device)
    if want_col and col_out is None:
        col_out = alloc_out(cols, rows, G_PER_TENSOR, device)
    _check(fn(xp, rows, cols, orient, err_mode, bound, _f32buf(amax, "amax", 1),
              _out(row_out if want_row else None, rows, cols, G_PER_TENSOR),
              _out(col_out if want_col else None, cols, rows, G_PER_TENSOR), _stream(device, stream)), name)
    return (row_out if want_row else None), (col_out if want_col else None)


def nvfp4_quantize_4o6_16x16(x: torch.Tensor, amax: torch.Tensor, orient: int = ROWWISE, err_mode: int = ERR_MSE,
                             bound: int = BOUND_STD, row_out: Optional[Quantized] = None,
                             col_out: Optional[Quantized] = None, stream=None):
    """Four-over-six with 16x16 tiles (per-tensor g): W (ROWWISE), W^T (COLWISE) or both from one read; returns
    (row_out, col_out), None for an orientation not asked for."""
    rows, cols = x.shape
    return _quantize_4o6_16x16(lib().nvfp4_quantize_4o6_16x16, "nvfp4_quantize_4o6_16x16", _bf16(x), rows, cols,
                               x.device, amax, orient, err_mode, bound, row_out, col_out, stream)


def nvfp4_quantize_4o6_16x16_f32(x: torch.Tensor, amax: torch.Tensor, orient: int = ROWWISE,
                                 err_mode: int = ERR_MSE, bound: int = BOUND_STD,
                                 row_out: Optional[Quantized] = None, col_out: Optional[Quantized] = None,
                                 stream=None):
    """nvfp4_quantize_4o6_16x16 of a float32 tensor."""
    rows, cols = x.shape
    return _quantize_4o6_16x16(lib().nvfp4_quantize_4o6_16x16_f32, "nvfp4_quantize_4o6_16x16_f32", _f32(x), rows,
                               cols, x.device, amax, orient, err_mode, bound, row_out, col_out, stream)


def nvfp4_swizzled_scales_size(rv: int, nb: int) -> int:
    return int(lib().nvfp4_swizzled_scales_size(rv, nb))


def nvfp4_swizzle_scales(scales: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The [rv, nb] uint8 scale matrix in the FP4 GEMM's tiled layout (flat uint8, zero-padded to 128 x 4 tiles)."""
    rv, nb = scales.shape
    if out is None:
        out = torch.empty(nvfp4_swizzled_scales_size(rv, nb), dtype=torch.uint8, device=scales.device)
    _check(lib().nvfp4_swizzle_scales(_dev(scales, "scales", (torch.uint8,)), rv, nb,
                                      _dev(out, "out", (torch.uint8,), nvfp4_swizzled_scales_size(rv, nb), True),
                                      _stream(scales.device, stream)), "nvfp4_swizzle_scales")
    return out


def _decode_in(codes: torch.Tensor, scales: torch.Tensor, g: torch.Tensor, gmode: int):
    if not isinstance(codes, torch.Tensor) or codes.dim() != 2:
        raise TypeError("codes must be a 2-D uint8 tensor [rv, cv/2]")
    rv, half = codes.shape
    cv = 2 * half
    return rv, cv, _out(Quantized(codes, scales, g), rv, cv, gmode)


def nvfp4_dequantize(codes: torch.Tensor, scales: torch.Tensor, g: torch.Tensor, gmode: int = G_PER_TENSOR,
                     y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode of a quantization's outputs (codes [rv, cv/2], row-major scales [rv, cv/16], g) to float32."""
    rv, cv, src = _decode_in(codes, scales, g, gmode)
    if y is None:
        y = torch.empty((rv, cv), dtype=torch.float32, device=codes.device)
    _check(lib().nvfp4_dequantize(src, rv, cv, gmode, _dev(y, "y", (torch.float32,), rv * cv),
                                  _stream(codes.device, stream)), "nvfp4_dequantize")
    return y


def nvfp4_dequantize_fused(codes: torch.Tensor, scales: torch.Tensor, g: torch.Tensor, gmode: int = G_PER_TENSOR,
                           use_rht: bool = False, sign_mask: int = 0, out_bf16: bool = False,
                           y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode, optionally through the inverse RHT; y is float32, or bfloat16 with out_bf16."""
    rv, cv, src = _decode_in(codes, scales, g, gmode)
    dtype = torch.bfloat16 if out_bf16 else torch.float32
    if y is None:
        y = torch.empty((rv, cv), dtype=dtype, device=codes.device)
    ydt = _BF16 if out_bf16 else (torch.float32,)
    _check(lib().nvfp4_dequantize_fused(src, rv, cv, gmode, int(bool(use_rht)), sign_mask & 0xFFFF,
                                        int(bool(out_bf16)), _dev(y, "y", ydt, rv * cv),
                                        _stream(codes.device, stream)), "nvfp4_dequantize_fused")
    return y


def _group(xs, amaxes, outs, sign_masks, seeds, offsets, gmode):
    n = len(xs)
    arr = (_GroupItem * max(n, 1))()
    for i, x in enumerate(xs):
        rows, cols = x.shape
        o = _out(outs[i], rows, cols, gmode) if outs is not None else None
        arr[i] = _GroupItem(_bf16(x), rows, cols, _f32buf(amaxes[i], "amax", _amax_n(rows, gmode)),
                            o._obj if o is not None else _Out(None, None, None, 0),
                            (sign_masks[i] if sign_masks is not None else 0) & 0xFFFF,
                            seeds[i] if seeds is not None else 0, offsets[i] if offsets is not None else 0)
    return arr


def nvfp4_amax_grouped(xs, gmode: int = G_PER_TENSOR, use_rht: bool = False, sign_masks=None, amaxes=None,
                       stream=None):
    """Row-wise amax of every tensor of xs in one launch; returns the list of amax tensors."""
    if amaxes is None:
        amaxes = [torch.empty((x.shape[0] if gmode == G_PER_ROW else 1,), dtype=torch.float32, device=x.device)
                  for x in xs]
    arr = _group(xs, amaxes, None, sign_masks, None, None, gmode)
    dev = xs[0].device if xs else torch.device("cuda")
    _check(lib().nvfp4_amax_grouped(arr, len(xs), gmode, int(bool(use_rht)), _stream(dev, stream)),
           "nvfp4_amax_grouped")
    return amaxes


def nvfp4_quantize_grouped(xs, amaxes, rounding: int, gmode: int = G_PER_TENSOR, sign_masks=None, seeds=None,
                           offsets=None, outs=None, stream=None, err_mode: int = ERR_MSE, bound: int = BOUND_STD):
    """Row-wise 1x16 quantization of every tensor of xs in one launch (RN, SR, RHT+SR or four-over-six); returns
    the list of Quantized outputs."""
    if outs is None:
        outs = [alloc_out(x.shape[0], x.shape[1], gmode, x.device) for x in xs]
    arr = _group(xs, amaxes, outs, sign_masks, seeds, offsets, gmode)
    dev = xs[0].device if xs else torch.device("cuda")
    _check(lib().nvfp4_quantize_grouped(arr, len(xs), gmode, rounding, err_mode, bound, _stream(dev, stream)),
           "nvfp4_quantize_grouped")
    return outs
