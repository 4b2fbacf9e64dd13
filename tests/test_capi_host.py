"""C-ABI checks that need no GPU: the library loads, exports every function include/nvfp4.h declares, and every
invalid call is rejected on the host with the documented status before anything is enqueued.  The pointers below
are aligned placeholders that validation never dereferences (a valid call would launch kernels, so none is
made here)."""
import ctypes as C
import os
import re

import pytest

from nvfp4_quantization_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")

OK, NULL, SHAPE, ALIGN, UNSUP = 0, 1, 2, 3, 4
P = 0x10000          # 16-byte aligned placeholder
MIS = 0x10008        # 8-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("HIP library not built")
    return B.lib()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(["nvfp4_amax", "nvfp4_quantize_rn", "nvfp4_quantize_sr",
                                           "nvfp4_quantize_rht_sr", "nvfp4_amax_quantize", "nvfp4_quantize_4o6",
                                           "nvfp4_dequantize", "nvfp4_dequantize_fused", "nvfp4_amax_grouped",
                                           "nvfp4_quantize_grouped", "nvfp4_quantize_4o6_16x16", "nvfp4_swizzle_scales",
                                           "nvfp4_swizzled_scales_size", "nvfp4_quantize_4o6_f32",
                                           "nvfp4_amax_f32", "nvfp4_quantize_4o6_16x16_f32", "nvfp4_status_str"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(B.SIGNATURES) == set(declared_functions())


def test_bench_library_is_separate():
    """The benchmark's streaming and stream-hold kernels live in their own library, outside the C ABI."""
    from nvfp4_quantization_amd._build import BENCH_LIB_PATH
    if not os.path.exists(BENCH_LIB_PATH):
        pytest.skip("benchmark library not built")
    L = C.CDLL(BENCH_LIB_PATH)
    assert hasattr(L, "nvfp4_bench_stream") and hasattr(L, "nvfp4_bench_hold")
    L.nvfp4_bench_hold.restype = C.c_int
    L.nvfp4_bench_hold.argtypes = [C.c_int64, C.c_void_p]
    assert L.nvfp4_bench_hold(-1, None) != 0 and L.nvfp4_bench_hold(2_000_000, None) != 0   # rejected on the host
    assert not any(n.startswith("nvfp4_bench") for n in declared_functions())


def test_status_strings(lib):
    for code, name in B.STATUS.items():
        assert lib.nvfp4_status_str(code).decode().startswith(name)


def out(codes=P, scales=P, g=P, layout=0):
    return C.byref(B._Out(codes, scales, g, layout))


def test_amax_validation(lib):
    f = lib.nvfp4_amax
    assert f(None, 16, 16, 1, 0, 0, 0, P, None) == NULL
    assert f(P, 16, 16, 1, 0, 0, 0, None, None) == NULL
    assert f(P, -1, 16, 1, 0, 0, 0, P, None) == SHAPE
    assert f(P, 16, 24, 1, 0, 0, 0, P, None) == SHAPE          # row-wise: cols % 16
    assert f(P, 24, 16, 2, 0, 0, 0, P, None) == SHAPE          # column-wise: rows % 16
    assert f(MIS, 16, 16, 1, 0, 0, 0, P, None) == ALIGN
    assert f(P, 16, 16, 1, 0, 0, 0, P + 2, None) == ALIGN
    assert f(P, 16, 16, 3, 0, 0, 0, P, None) == UNSUP         # BOTH is not an amax view
    assert f(P, 16, 16, 1, 7, 0, 0, P, None) == UNSUP
    assert f(P, 1 << 20, 1 << 20, 1, 0, 0, 0, P, None) == SHAPE  # 2^40 elements
    assert f(P, 1 << 19, 1 << 16, 1, 0, 0, 0, P, None) == SHAPE  # 2^35 elements: block index + stride could wrap
    assert f(P, 16, 1 << 25, 2, 0, 0, 0, P, None) == SHAPE       # column-wise: cols < 2^25


def test_quantize_rn_validation(lib):
    f = lib.nvfp4_quantize_rn
    assert f(P, 16, 16, 0, 3, 0, P, out(), out(), None) == UNSUP      # 1x16 BOTH
    assert f(P, 16, 16, 1, 1, 1, P, out(), None, None) == UNSUP       # 16x16 per-row g
    assert f(P, 16, 24, 1, 1, 0, P, out(), None, None) == SHAPE       # 16x16 cols % 16
    assert f(P, 24, 16, 1, 2, 0, P, None, out(), None) == SHAPE       # 16x16 rows % 16
    assert f(P, 16, 1 << 25, 1, 2, 0, P, None, out(), None) == SHAPE  # 16x16 cols < 2^25
    assert f(P, 16, 16, 1, 3, 0, P, out(), None, None) == NULL        # BOTH needs both outputs
    assert f(P, 16, 16, 0, 1, 0, P, None, out(), None) == NULL        # row-wise needs row_out
    assert f(P, 16, 16, 0, 1, 0, P, out(g=None), None, None) == NULL
    assert f(P, 16, 16, 0, 1, 0, P, out(codes=MIS), None, None) == ALIGN
    assert f(P, 16, 16, 0, 1, 0, P, out(g=P + 1), None, None) == ALIGN
    assert f(P, 16, 16, 5, 1, 0, P, out(), None, None) == UNSUP       # unknown block
    assert f(P, 16, 16, 1, 4, 0, P, out(), out(), None) == UNSUP      # unknown orientation


def test_quantize_sr_and_rht_sr_validation(lib):
    for f, extra in ((lib.nvfp4_quantize_sr, ()), (lib.nvfp4_quantize_rht_sr, (0x1234,))):
        assert f(P, 16, 16, 3, 0, P, *extra, 1, 2, out(), None) == UNSUP   # BOTH
        assert f(P, 16, 24, 1, 0, P, *extra, 1, 2, out(), None) == SHAPE
        assert f(P, 16, 16, 1, 0, None, *extra, 1, 2, out(), None) == NULL
        assert f(P, 16, 16, 1, 0, P, *extra, 1, 2, None, None) == NULL
        assert f(P, 16, 16, 1, 2, P, *extra, 1, 2, out(), None) == UNSUP


def test_amax_quantize_validation(lib):
    f = lib.nvfp4_amax_quantize
    assert f(P, 16, 16, 2, 3, 0, 1, 2, P, out(), None) == UNSUP       # unknown rounding
    assert f(P, 16, 16, 3, 0, 0, 1, 2, P, out(), None) == UNSUP       # BOTH
    assert f(P, 24, 16, 2, 2, 0, 1, 2, P, out(), None) == SHAPE       # column-wise rows % 16
    assert f(P, 16, 24, 1, 0, 0, 1, 2, P, out(), None) == SHAPE       # row-wise cols % 16
    assert f(P, 16, 16, 2, 2, 0, 1, 2, None, out(), None) == NULL     # amax is an output here
    assert f(P, 16, 16, 2, 2, 0, 1, 2, P + 2, out(), None) == ALIGN
    assert f(P, 16, 16, 2, 2, 0, 1, 2, P, None, None) == NULL
    assert f(MIS, 16, 16, 2, 2, 0, 1, 2, P, out(), None) == ALIGN


def test_4o6_and_dequantize_validation(lib):
    q = lib.nvfp4_quantize_4o6
    assert q(P, 16, 24, 1, 0, 448, P, out(), None) == SHAPE
    assert q(P, 16, 16, 9, 0, 448, P, out(), None) == UNSUP
    assert q(P, 16, 16, 1, 0, 448, P, out(scales=None), None) == NULL
    assert q(P, 16, 16, 1, 3, 448, P, out(), None) == UNSUP          # unknown error mode
    assert q(P, 16, 16, 1, -1, 448, P, out(), None) == UNSUP
    assert q(P, 16, 16, 1, 2, 0, P, out(), None) == UNSUP            # bound outside 1..448
    assert q(P, 16, 16, 1, 2, 449, P, out(), None) == UNSUP
    d = lib.nvfp4_dequantize
    assert d(out(), 4, 24, 0, P, None) == SHAPE
    assert d(out(), 4, 32, 0, P + 4, None) == ALIGN                # y must be 16-byte aligned
    assert d(out(codes=None), 4, 32, 0, P, None) == NULL
    assert d(None, 4, 32, 0, P, None) == NULL
    assert d(out(), -4, 32, 0, P, None) == SHAPE
    assert d(out(layout=1), 4, 32, 0, P, None) == UNSUP            # tiled scales are not decoded


def test_dequantize_fused_validation(lib):
    d = lib.nvfp4_dequantize_fused
    #        in     rv  cv  gmode rht mask bf16 y  stream
    assert d(out(), 4, 24, 0, 1, 0x1234, 1, P, None) == SHAPE           # cv % 16
    assert d(out(), -1, 32, 0, 1, 0x1234, 1, P, None) == SHAPE
    assert d(out(), 1 << 20, 1 << 20, 0, 1, 0, 1, P, None) == SHAPE      # 2^40 elements
    assert d(out(), 4, 32, 2, 1, 0, 1, P, None) == UNSUP                 # unknown g mode
    assert d(None, 4, 32, 0, 1, 0, 1, P, None) == NULL
    assert d(out(codes=None), 4, 32, 0, 1, 0, 1, P, None) == NULL
    assert d(out(scales=None), 4, 32, 0, 1, 0, 1, P, None) == NULL
    assert d(out(g=None), 4, 32, 1, 1, 0, 1, P, None) == NULL
    assert d(out(), 4, 32, 0, 1, 0, 1, None, None) == NULL
    assert d(out(codes=MIS), 4, 32, 0, 1, 0, 1, P, None) == ALIGN
    assert d(out(g=P + 2), 4, 32, 0, 1, 0, 1, P, None) == ALIGN
    assert d(out(), 4, 32, 0, 1, 0, 0, P + 8, None) == ALIGN             # y must be 16-byte aligned
    assert d(out(codes=None, scales=None), 0, 32, 0, 1, 0, 1, None, None) == OK   # empty: nothing to decode


def test_grouped_validation(lib):
    def items(n, over=None):
        arr = (B._GroupItem * max(n, 1))()
        for i in range(n):
            f = dict(x=P, rows=32, cols=64, amax=P, out=B._Out(P, P, P), sign_mask=1, seed=2, offset=3)
            f.update((over or {}).get(i, {}))
            arr[i] = B._GroupItem(**f)
        return arr
    a, q = lib.nvfp4_amax_grouped, lib.nvfp4_quantize_grouped
    assert C.sizeof(B._GroupItem) == 88                                   # the C layout of nvfp4_group_item
    assert a(items(0), 0, 0, 1, None) == OK                               # nothing to do
    assert q(items(0), 0, 0, 2, 0, 448, None) == OK
    assert a(items(2), -1, 0, 1, None) == SHAPE
    assert a(items(33), 33, 0, 1, None) == SHAPE                          # more than NVFP4_MAX_GROUP
    assert a(None, 2, 0, 1, None) == NULL
    assert a(items(2), 2, 5, 1, None) == UNSUP                            # unknown g mode
    assert q(items(2), 2, 0, 9, 0, 448, None) == UNSUP                            # unknown rounding
    assert a(items(3, {2: dict(cols=24)}), 3, 0, 1, None) == SHAPE      # item 2: cols % 16
    assert a(items(3, {1: dict(x=MIS)}), 3, 0, 1, None) == ALIGN
    assert a(items(3, {1: dict(amax=None)}), 3, 0, 1, None) == NULL
    assert a(items(2, {0: dict(rows=-1)}), 2, 0, 1, None) == SHAPE
    assert q(items(2, {1: dict(out=B._Out(P, None, P))}), 2, 0, 0, 0, 448, None) == NULL
    assert q(items(2, {1: dict(out=B._Out(P, P, P + 2))}), 2, 1, 3, 0, 448, None) == ALIGN
    assert q(items(2, {0: dict(rows=1 << 20, cols=1 << 20)}), 2, 0, 1, 0, 448, None) == SHAPE
    # four-over-six is a grouped method only, with its knobs checked
    assert lib.nvfp4_amax_quantize(P, 16, 16, 1, 3, 0, 0, 0, P, out(), None) == UNSUP
    assert q(items(1), 1, 0, 3, 5, 448, None) == UNSUP
    assert q(items(1), 1, 0, 3, 0, 500, None) == UNSUP


def test_4o6_16x16_validation(lib):
    for f in (lib.nvfp4_quantize_4o6_16x16, lib.nvfp4_quantize_4o6_16x16_f32):
        assert f(P, 24, 16, 1, 0, 448, P, out(), None, None) == SHAPE          # rows % 16
        assert f(P, 16, 24, 1, 0, 448, P, out(), None, None) == SHAPE          # cols % 16
        assert f(P, -16, 16, 1, 0, 448, P, out(), None, None) == SHAPE
        assert f(None, 16, 16, 1, 0, 448, P, out(), None, None) == NULL
        assert f(P, 16, 16, 1, 0, 448, None, out(), None, None) == NULL
        assert f(P, 16, 16, 1, 0, 448, P, None, out(), None) == NULL           # W asked for, no row_out
        assert f(P, 16, 16, 2, 0, 448, P, out(), None, None) == NULL           # W^T asked for, no col_out
        assert f(P, 16, 16, 3, 0, 448, P, out(), None, None) == NULL           # both asked for
        assert f(P, 16, 16, 1, 0, 448, P, out(scales=None), None, None) == NULL
        assert f(P, 16, 16, 2, 0, 448, P, None, out(g=None), None) == NULL
        assert f(MIS, 16, 16, 1, 0, 448, P, out(), None, None) == ALIGN
        assert f(P, 16, 16, 1, 0, 448, P, out(g=P + 2), None, None) == ALIGN
        assert f(P, 16, 16, 2, 0, 448, P, None, out(codes=MIS), None) == ALIGN
        assert f(P, 16, 16, 4, 0, 448, P, out(), out(), None) == UNSUP         # unknown orientation
        assert f(P, 16, 16, 1, 7, 448, P, out(), None, None) == UNSUP          # unknown error mode
        assert f(P, 16, 16, 1, 0, 0, P, out(), None, None) == UNSUP            # bound outside 1..448


def test_swizzle_validation(lib):
    import oracle as O
    f = lib.nvfp4_swizzle_scales
    for rv, nb in [(0, 0), (1, 1), (128, 4), (129, 5), (300, 65), (8192, 256)]:
        assert lib.nvfp4_swizzled_scales_size(rv, nb) == O.swizzled_size(rv, nb)
    assert lib.nvfp4_swizzled_scales_size(-1, 4) == 0
    assert f(P, -1, 4, P, None) == SHAPE
    assert f(P, 4, -1, P, None) == SHAPE
    assert f(P, 1 << 16, 1 << 15, P, None) == SHAPE      # rv * nb >= 2^31
    assert f(None, 4, 4, P, None) == NULL
    assert f(P, 4, 4, None, None) == NULL
    assert f(P + 1, 4, 4, P + 4, None) == ALIGN           # out must be 16-byte aligned (scales need not be)
    assert f(None, 0, 4, None, None) == OK                # nothing to do: no pointer needed


def test_tiled_scale_layout_validation(lib):
    """The tiled scale layout is taken by the 1x16 calls only (checked before anything is enqueued)."""
    T = 1
    assert lib.nvfp4_quantize_rn(P, 16, 16, 1, 3, 0, P, out(), out(layout=T), None) == UNSUP  # 16x16
    assert lib.nvfp4_quantize_4o6(P, 16, 16, 0, 0, 448, P, out(layout=T), None) == UNSUP
    assert lib.nvfp4_quantize_4o6_16x16(P, 16, 16, 1, 0, 448, P, out(layout=T), None, None) == UNSUP
    assert lib.nvfp4_quantize_4o6_16x16(P, 16, 16, 2, 0, 448, P, None, out(layout=T), None) == UNSUP
    assert lib.nvfp4_quantize_sr(P, 16, 16, 2, 0, P, 0, 0, out(layout=7), None) == UNSUP   # unknown layout
    assert lib.nvfp4_quantize_sr(P, 16, 16, 2, 0, P, 0, 0, out(scales=None, layout=T), None) == NULL
    it = (B._GroupItem * 1)()
    it[0] = B._GroupItem(P, 16, 16, P, B._Out(P, P, P, T), 0, 0, 0)
    assert lib.nvfp4_quantize_grouped(it, 1, 0, 0, 0, 448, None) == UNSUP


def test_f32_input_validation(lib):
    q, a = lib.nvfp4_quantize_4o6_f32, lib.nvfp4_amax_f32
    assert q(P, 16, 24, 0, 0, 448, P, out(), None) == SHAPE          # cols % 16
    assert q(P, -1, 16, 0, 0, 448, P, out(), None) == SHAPE
    assert q(P, 16, 16, 5, 0, 448, P, out(), None) == UNSUP          # unknown g mode
    assert q(None, 16, 16, 0, 0, 448, P, out(), None) == NULL
    assert q(P, 16, 16, 0, 0, 448, None, out(), None) == NULL
    assert q(MIS, 16, 16, 0, 0, 448, P, out(), None) == ALIGN
    assert q(P, 16, 16, 0, 0, 448, P, out(layout=1), None) == UNSUP  # tiled scales: not for four-over-six
    assert q(P, 16, 16, 0, 9, 448, P, out(), None) == UNSUP          # unknown error mode
    assert q(P, 16, 16, 0, 1, 1000, P, out(), None) == UNSUP         # bound outside 1..448
    t = lib.nvfp4_quantize_4o6_16x16_f32
    assert t(P, 16, 16, 1, 0, 448, P, out(layout=1), None, None) == UNSUP
    assert a(P, 16, 24, 0, P, None) == SHAPE
    assert a(None, 16, 16, 0, P, None) == NULL
    assert a(P, 16, 16, 1, None, None) == NULL
    assert a(MIS, 16, 16, 0, P, None) == ALIGN
