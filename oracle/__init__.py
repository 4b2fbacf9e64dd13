"""CPU oracle for the NVFP4 training quantizer (numpy front end over ``nvfp4_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg use
this package.  The product library (``nvfp4_quantization_amd``) never imports it, and this package imports
nothing from the product.

Every function takes and returns numpy arrays on the host.  bf16 tensors are passed as their ``uint16`` bit
patterns, row-major and contiguous.  The arithmetic, its readings of the pages and its citations live in
``nvfp4_oracle.c``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libnvfp4_oracle.so")

ROWWISE, COLWISE = 1, 2
G_PER_TENSOR, G_PER_ROW = 0, 1
MODE_RN, MODE_SR, MODE_RHT_SR = 0, 1, 2
ERR_MSE, ERR_MAE, ERR_MAXABS = 0, 1, 2        # four-over-six error modes (sum of squares, sum of magnitudes, max)

# gcc flags: one IEEE binary32 rounding per operation (no contraction, no fast-math), OpenMP over rows.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-Wall"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (the plain C compiler of the host)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        _lib = C.CDLL(build())
        _declare(_lib)
    return _lib


def _declare(L: C.CDLL) -> None:
    p, i64, u64, u16, u8, f32, i32 = C.c_void_p, C.c_int64, C.c_uint64, C.c_uint16, C.c_uint8, C.c_float, C.c_int
    L.nvo_num_threads.restype = i32
    L.nvo_set_num_threads.argtypes = [i32]
    L.nvo_bf16_to_f32.argtypes = [u16]
    L.nvo_bf16_to_f32.restype = f32
    L.nvo_e2m1_decode.argtypes = [u8]
    L.nvo_e2m1_decode.restype = f32
    L.nvo_e2m1_rn.argtypes = [f32]
    L.nvo_e2m1_rn.restype = u8
    L.nvo_e2m1_sr.argtypes = [f32, u8]
    L.nvo_e2m1_sr.restype = u8
    L.nvo_e2m1_rn_array.argtypes = [p, i64, p]
    L.nvo_e2m1_sr_array.argtypes = [p, p, i64, p]
    L.nvo_e4m3_encode_array.argtypes = [p, i64, p]
    L.nvo_e4m3_decode.argtypes = [u8]
    L.nvo_e4m3_decode.restype = f32
    L.nvo_e4m3_encode.argtypes = [f32]
    L.nvo_e4m3_encode.restype = u8
    L.nvo_philox4x32_10.argtypes = [p, p, p]
    L.nvo_block_random_bytes.argtypes = [u64, u64, u64, p]
    L.nvo_rht16.argtypes = [p, u16, p]
    L.nvo_global_scale.argtypes = [f32]
    L.nvo_global_scale.restype = f32
    L.nvo_block_scale.argtypes = [f32, f32, f32, p, p]
    L.nvo_amax.argtypes = [p, i64, i64, i32, i32, i32, u16, p]
    L.nvo_amax.restype = i32
    L.nvo_quantize_1x16.argtypes = [p, i64, i64, i32, i32, i32, p, u16, u64, u64, i64, i64, p, p, p]
    L.nvo_quantize_1x16.restype = i32
    L.nvo_quantize_16x16.argtypes = [p, i64, i64, p, i64, i64, p, p, p, p, p, p]
    L.nvo_quantize_16x16.restype = i32
    L.nvo_quantize_4o6.argtypes = [p, i64, i64, i32, i32, i32, p, i64, i64, p, p, p, p]
    L.nvo_quantize_4o6.restype = i32
    L.nvo_quantize_4o6_16x16.argtypes = [p, i64, i64, i32, i32, p, i64, i64, p, p, p, p, p, p, p]
    L.nvo_quantize_4o6_16x16.restype = i32
    L.nvo_dequantize.argtypes = [p, p, p, i64, i64, i32, p]
    L.nvo_dequantize.restype = i32
    L.nvo_rht16_inverse.argtypes = [p, u16, p]
    L.nvo_f32_to_bf16.argtypes = [f32]
    L.nvo_f32_to_bf16.restype = u16
    L.nvo_dequantize_fused.argtypes = [p, p, p, i64, i64, i32, i32, u16, i32, p]
    L.nvo_dequantize_fused.restype = i32
    L.nvo_quantize_4o6_f32.argtypes = [p, i64, i64, i32, i32, i32, p, i64, i64, p, p, p, p]
    L.nvo_quantize_4o6_f32.restype = i32
    L.nvo_quantize_4o6_16x16_f32.argtypes = [p, i64, i64, i32, i32, p, i64, i64, p, p, p, p, p, p, p]
    L.nvo_quantize_4o6_16x16_f32.restype = i32
    L.nvo_amax_f32.argtypes = [p, i64, i64, i32, p]
    L.nvo_amax_f32.restype = i32
    L.nvo_swizzle_scales.argtypes = [p, i64, i64, p]
    L.nvo_swizzle_scales.restype = i32


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _check(st: int, what: str) -> None:
    if st != 0:
        raise ValueError(f"oracle {what} returned status {st}")


def _bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("bf16 inputs are passed as uint16 bit patterns")
    return x


def view_shape(rows: int, cols: int, orient: int) -> tuple[int, int]:
    return (rows, cols) if orient == ROWWISE else (cols, rows)


# ---- scalar helpers (used by the oracle's own pins) -------------------------------------------------------
def set_num_threads(n: int) -> None:
    lib().nvo_set_num_threads(int(n))


def num_threads() -> int:
    return int(lib().nvo_num_threads())


def e2m1_rn(q: float) -> int:
    return int(lib().nvo_e2m1_rn(float(q)))


def e2m1_sr(q: float, rho: int) -> int:
    return int(lib().nvo_e2m1_sr(float(q), int(rho)))


def e2m1_decode(code: int) -> float:
    return float(lib().nvo_e2m1_decode(int(code)))


def e2m1_rn_array(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float32)
    out = np.zeros(q.shape, dtype=np.uint8)
    lib().nvo_e2m1_rn_array(_ptr(q), q.size, _ptr(out))
    return out


def e2m1_sr_array(q: np.ndarray, rho: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float32)
    rho = np.ascontiguousarray(rho, dtype=np.uint8)
    assert rho.shape == q.shape
    out = np.zeros(q.shape, dtype=np.uint8)
    lib().nvo_e2m1_sr_array(_ptr(q), _ptr(rho), q.size, _ptr(out))
    return out


def e4m3_encode_array(s: np.ndarray) -> np.ndarray:
    s = np.ascontiguousarray(s, dtype=np.float32)
    out = np.zeros(s.shape, dtype=np.uint8)
    lib().nvo_e4m3_encode_array(_ptr(s), s.size, _ptr(out))
    return out


def e4m3_encode(s: float) -> int:
    return int(lib().nvo_e4m3_encode(float(s)))


def e4m3_decode(code: int) -> float:
    return float(lib().nvo_e4m3_decode(int(code)))


def philox4x32_10(counter, key) -> list[int]:
    c = np.asarray(counter, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().nvo_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return [int(v) for v in out]


def block_random_bytes(seed: int, offset: int, block_index: int) -> np.ndarray:
    out = np.zeros(16, dtype=np.uint8)
    lib().nvo_block_random_bytes(seed, offset, block_index, _ptr(out))
    return out


def rht16(v: np.ndarray, sign_mask: int) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    assert v.shape == (16,)
    y = np.zeros(16, dtype=np.float32)
    lib().nvo_rht16(_ptr(v), int(sign_mask), _ptr(y))
    return y


def rht16_inverse(y: np.ndarray, sign_mask: int) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    assert y.shape == (16,)
    v = np.zeros(16, dtype=np.float32)
    lib().nvo_rht16_inverse(_ptr(y), int(sign_mask), _ptr(v))
    return v


def f32_to_bf16(x: float) -> int:
    return int(lib().nvo_f32_to_bf16(float(x)))


def global_scale(amax: float) -> np.float32:
    return np.float32(lib().nvo_global_scale(float(amax)))


def block_scale(bamax: float, g: float, T: float = 6.0) -> tuple[int, np.float32]:
    sb = np.zeros(1, dtype=np.uint8)
    r = np.zeros(1, dtype=np.float32)
    lib().nvo_block_scale(float(bamax), float(g), float(T), _ptr(sb), _ptr(r))
    return int(sb[0]), r[0]


# ---- tensor entry points ----------------------------------------------------------------------------------
def amax(x: np.ndarray, orient: int = ROWWISE, gmode: int = G_PER_TENSOR, use_rht: bool = False,
         sign_mask: int = 0) -> np.ndarray:
    x = _bits(x)
    rows, cols = x.shape
    rv, _ = view_shape(rows, cols, orient)
    out = np.zeros(rv if gmode == G_PER_ROW else 1, dtype=np.float32)
    _check(lib().nvo_amax(_ptr(x), rows, cols, orient, gmode, int(use_rht), int(sign_mask), _ptr(out)), "amax")
    return out


def quantize_1x16(x: np.ndarray, amax_arr: np.ndarray, mode: int, orient: int = ROWWISE,
                  gmode: int = G_PER_TENSOR, sign_mask: int = 0, seed: int = 0, offset: int = 0,
                  vrows: tuple[int, int] | None = None):
    """Returns (codes [Rv, Cv/2] u8, scales [Rv, Cv/16] u8, g f32).  With ``vrows=(a, b)`` only V rows a..b-1
    are computed (the other rows of the returned arrays stay zero)."""
    x = _bits(x)
    rows, cols = x.shape
    rv, cv = view_shape(rows, cols, orient)
    a, b = vrows if vrows is not None else (0, rv)
    amax_arr = np.ascontiguousarray(amax_arr, dtype=np.float32)
    codes = np.zeros((rv, cv // 2), dtype=np.uint8)
    scales = np.zeros((rv, cv // 16), dtype=np.uint8)
    g = np.zeros(rv if gmode == G_PER_ROW else 1, dtype=np.float32)
    _check(lib().nvo_quantize_1x16(_ptr(x), rows, cols, orient, gmode, mode, _ptr(amax_arr), int(sign_mask),
                                   seed, offset, a, b, _ptr(codes), _ptr(scales), _ptr(g)), "quantize_1x16")
    return codes, scales, g


def quantize_16x16(x: np.ndarray, amax_arr: np.ndarray, tile_rows: tuple[int, int] | None = None):
    """Returns ((codes_w, scales_w, g_w), (codes_wt, scales_wt, g_wt))."""
    x = _bits(x)
    rows, cols = x.shape
    a, b = tile_rows if tile_rows is not None else (0, rows // 16)
    amax_arr = np.ascontiguousarray(amax_arr, dtype=np.float32)
    cw = np.zeros((rows, cols // 2), dtype=np.uint8)
    sw = np.zeros((rows, cols // 16), dtype=np.uint8)
    gw = np.zeros(1, dtype=np.float32)
    ct = np.zeros((cols, rows // 2), dtype=np.uint8)
    stt = np.zeros((cols, rows // 16), dtype=np.uint8)
    gt = np.zeros(1, dtype=np.float32)
    _check(lib().nvo_quantize_16x16(_ptr(x), rows, cols, _ptr(amax_arr), a, b, _ptr(cw), _ptr(sw), _ptr(gw),
                                    _ptr(ct), _ptr(stt), _ptr(gt)), "quantize_16x16")
    return (cw, sw, gw), (ct, stt, gt)


def quantize_4o6(x: np.ndarray, amax_arr: np.ndarray, gmode: int = G_PER_ROW,
                 rows_range: tuple[int, int] | None = None, err_mode: int = ERR_MSE, bound: int = 448):
    """Returns (codes, scales, g, choice) where choice[r, b] = 1 if map-to-4 was kept; err_mode ERR_MSE, ERR_MAE or
    ERR_MAXABS; g = amax / (6 bound)."""
    x = _bits(x)
    rows, cols = x.shape
    a, b = rows_range if rows_range is not None else (0, rows)
    amax_arr = np.ascontiguousarray(amax_arr, dtype=np.float32)
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows, cols // 16), dtype=np.uint8)
    g = np.zeros(rows if gmode == G_PER_ROW else 1, dtype=np.float32)
    choice = np.zeros((rows, cols // 16), dtype=np.uint8)
    _check(lib().nvo_quantize_4o6(_ptr(x), rows, cols, gmode, err_mode, bound, _ptr(amax_arr), a, b, _ptr(codes),
                                  _ptr(scales), _ptr(g), _ptr(choice)), "quantize_4o6")
    return codes, scales, g, choice


def quantize_4o6_16x16(x: np.ndarray, amax_arr: np.ndarray, tile_rows: tuple[int, int] | None = None,
                       err_mode: int = ERR_MSE, bound: int = 448):
    """Four-over-six with 16x16 tiles (per-tensor g).  Returns ((codes_w, scales_w, g_w), (codes_wt, scales_wt,
    g_wt), choice) with choice[ti, tj] = 1 where map-to-4 was kept."""
    x = _bits(x)
    rows, cols = x.shape
    a, b = tile_rows if tile_rows is not None else (0, rows // 16)
    amax_arr = np.ascontiguousarray(amax_arr, dtype=np.float32)
    cw = np.zeros((rows, cols // 2), np.uint8)
    sw = np.zeros((rows, cols // 16), np.uint8)
    gw = np.zeros(1, np.float32)
    ct = np.zeros((cols, rows // 2), np.uint8)
    stt = np.zeros((cols, rows // 16), np.uint8)
    gt = np.zeros(1, np.float32)
    choice = np.zeros((rows // 16, cols // 16), np.uint8)
    _check(lib().nvo_quantize_4o6_16x16(_ptr(x), rows, cols, err_mode, bound, _ptr(amax_arr), a, b, _ptr(cw),
                                        _ptr(sw), _ptr(gw), _ptr(ct), _ptr(stt), _ptr(gt), _ptr(choice)),
           "quantize_4o6_16x16")
    return (cw, sw, gw), (ct, stt, gt), choice


def dequantize(codes: np.ndarray, scales: np.ndarray, g: np.ndarray, gmode: int = G_PER_TENSOR) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    g = np.ascontiguousarray(g, dtype=np.float32)
    rv, half = codes.shape
    y = np.zeros((rv, 2 * half), dtype=np.float32)
    _check(lib().nvo_dequantize(_ptr(codes), _ptr(scales), _ptr(g), rv, 2 * half, gmode, _ptr(y)), "dequantize")
    return y


def dequantize_fused(codes: np.ndarray, scales: np.ndarray, g: np.ndarray, gmode: int = G_PER_TENSOR,
                     use_rht: bool = False, sign_mask: int = 0, out_bf16: bool = False) -> np.ndarray:
    """Decode, optionally followed by the inverse RHT; float32 [rv, cv], or uint16 bf16 patterns with out_bf16."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    g = np.ascontiguousarray(g, dtype=np.float32)
    rv, cv = codes.shape[0], codes.shape[1] * 2
    y = np.zeros((rv, cv), dtype=np.uint16 if out_bf16 else np.float32)
    _check(lib().nvo_dequantize_fused(_ptr(codes), _ptr(scales), _ptr(g), rv, cv, gmode, int(use_rht),
                                      int(sign_mask), int(out_bf16), _ptr(y)), "dequantize_fused")
    return y


def swizzled_size(rv: int, nb: int) -> int:
    """Bytes of the tiled scale layout of an [rv, nb] scale matrix (whole 128 x 4 tiles)."""
    return (rv + 127) // 128 * 128 * ((nb + 3) // 4 * 4)


def swizzle_scales(scales: np.ndarray) -> np.ndarray:
    """The [rv, nb] E4M3 scale matrix in the tiled 128 x 4 (32 x 4 x 4) layout, zero-padded; flat uint8."""
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rv, nb = scales.shape
    out = np.empty(swizzled_size(rv, nb), dtype=np.uint8)
    _check(lib().nvo_swizzle_scales(_ptr(scales), rv, nb, _ptr(out)), "swizzle_scales")
    return out


def amax_f32(x: np.ndarray, gmode: int = G_PER_TENSOR) -> np.ndarray:
    """Row-wise amax of a float32 array (no transform): [1] or [rows]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    out = np.zeros(rows if gmode == G_PER_ROW else 1, dtype=np.float32)
    _check(lib().nvo_amax_f32(_ptr(x), rows, cols, gmode, _ptr(out)), "amax_f32")
    return out


def quantize_4o6_f32(x: np.ndarray, amax_arr: np.ndarray, gmode: int = G_PER_ROW, err_mode: int = ERR_MSE,
                     bound: int = 448):
    """Four-over-six of a float32 array; returns (codes, scales, g, choice) as quantize_4o6."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    amax_arr = np.ascontiguousarray(amax_arr, dtype=np.float32)
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows, cols // 16), dtype=np.uint8)
    g = np.zeros(rows if gmode == G_PER_ROW else 1, dtype=np.float32)
    choice = np.zeros((rows, cols // 16), dtype=np.uint8)
    _check(lib().nvo_quantize_4o6_f32(_ptr(x), rows, cols, gmode, err_mode, bound, _ptr(amax_arr), 0, rows,
                                      _ptr(codes), _ptr(scales), _ptr(g), _ptr(choice)), "quantize_4o6_f32")
    return codes, scales, g, choice


def quantize_4o6_16x16_f32(x: np.ndarray, amax_arr: np.ndarray, err_mode: int = ERR_MSE, bound: int = 448):
    """Four-over-six with 16x16 tiles of a float32 array; returns as quantize_4o6_16x16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    amax_arr = np.ascontiguousarray(amax_arr, dtype=np.float32)
    cw = np.zeros((rows, cols // 2), dtype=np.uint8)
    sw = np.zeros((rows, cols // 16), dtype=np.uint8)
    gw = np.zeros(1, dtype=np.float32)
    ct = np.zeros((cols, rows // 2), dtype=np.uint8)
    stt = np.zeros((cols, rows // 16), dtype=np.uint8)
    gt = np.zeros(1, dtype=np.float32)
    choice = np.zeros((rows // 16, cols // 16), dtype=np.uint8)
    _check(lib().nvo_quantize_4o6_16x16_f32(_ptr(x), rows, cols, err_mode, bound, _ptr(amax_arr), 0, rows // 16,
                                            _ptr(cw), _ptr(sw), _ptr(gw), _ptr(ct), _ptr(stt), _ptr(gt),
                                            _ptr(choice)),
           "quantize_4o6_16x16_f32")
    return (cw, sw, gw), (ct, stt, gt), choice
