"""GPU parity of the column-wise quantizers writing their scales straight into the FP4 GEMM's tiled layout.

Codes and g must equal the oracle's; the scales must equal the oracle's tiled layout of the oracle's scales
(oracle.swizzle_scales), byte for byte, padding included (the scale buffer is filled with 0xAB first).  Covers the
quantize kernel (amax given; per-tensor and per-row g), the single-read amax + quantize kernel (fast and slow
routes), the two-pass fallback, ragged row tiles (columns of X not a multiple of 128) and ragged scale-column tiles
(row-blocks not a multiple of 4 or 16), and the 8192 x 4096 weight-gradient workload.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import nvfp4_quantization_amd as Q
from nvfp4_quantization_amd import workloads as W

pytestmark = pytest.mark.gpu

ROUNDING = {"rn": (Q.ROUND_RN, O.MODE_RN), "sr": (Q.ROUND_SR, O.MODE_SR), "rht_sr": (Q.ROUND_RHT_SR, O.MODE_RHT_SR)}
SHAPES = [(512, 200), (48, 8), (80, 136), (1040, 72), (16, 520), (2048, 1024), (272, 1032), (48, 12), (64, 27),
          (144, 300), (272, 1001)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    Q.binding.lib()
    O.lib()


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def tiled_out(rows, cols, gmode):
    o = Q.alloc_out(cols, rows, gmode, "cuda", Q.SCALES_TILED)
    o.scales.fill_(0xAB)
    return o


def compare(x, o, a, mode, gmode, mask, seed, offset):
    torch.cuda.synchronize()
    oa = O.amax(x, O.COLWISE, gmode, mode == "rht_sr", mask)
    ga = a.cpu().numpy()
    assert (ga.view(np.uint32) == oa.view(np.uint32)).all() or (np.isnan(ga) == np.isnan(oa)).all()
    oc, os_, og = O.quantize_1x16(x, oa, ROUNDING[mode][1], O.COLWISE, gmode, mask, seed, offset)
    assert np.array_equal(o.codes.cpu().numpy(), oc), "codes"
    sw = O.swizzle_scales(os_)
    got = o.scales.cpu().numpy()
    bad = np.flatnonzero(got != sw)
    assert bad.size == 0, f"tiled scales: {bad.size} mismatches, first at {bad[:6].tolist()}"
    g = o.g.cpu().numpy()
    assert ((g.view(np.uint32) == og.view(np.uint32)) | (np.isnan(g) & np.isnan(og))).all()


@pytest.mark.parametrize("mode", ["rn", "sr", "rht_sr"])
@pytest.mark.parametrize("gmode", [0, 1])
@pytest.mark.parametrize("shape", SHAPES)
def test_quantize_colwise(mode, gmode, shape):
    say("tiled quantize", mode, "per-row" if gmode else "per-tensor", shape)
    mask, seed, offset = 0x3C5A, 0x77_0000_1234, 5
    x = W.outlier_columns(*shape, seed=(shape[0] * 11 + shape[1]) & 0xFFFF, n_cols=min(4, shape[1]))
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    a = Q.nvfp4_amax(xd, Q.COLWISE, gmode, use_rht=(mode == "rht_sr"), sign_mask=mask)
    o = tiled_out(*shape, gmode)
    if mode == "rn":
        Q.nvfp4_quantize_rn(xd, a, Q.BLOCK_1X16, Q.COLWISE, gmode, col_out=o)
    elif mode == "sr":
        Q.nvfp4_quantize_sr(xd, a, seed, offset, Q.COLWISE, gmode, out=o)
    else:
        Q.nvfp4_quantize_rht_sr(xd, a, mask, seed, offset, Q.COLWISE, gmode, out=o)
    compare(x, o, a, mode, gmode, mask, seed, offset)


def amax_quantize(x, mode, mask=0x5A3C, seed=0xDEAD_BEEF_0123, offset=3):
    say("tiled amax_quantize", mode, x.shape, offset)
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    o = tiled_out(*x.shape, 0)
    a, _ = Q.nvfp4_amax_quantize(xd, Q.COLWISE, ROUNDING[mode][0], mask, seed, offset, out=o)
    compare(x, o, a, mode, 0, mask, seed, offset)


@pytest.mark.parametrize("mode", ["rn", "sr", "rht_sr"])
@pytest.mark.parametrize("shape", SHAPES)
def test_amax_quantize_single_read(mode, shape):
    amax_quantize(W.lognormal_gradients(*shape, seed=(shape[0] * 5 + shape[1]) & 0xFFFF), mode)


@pytest.mark.parametrize("mode", ["rn", "rht_sr"])
def test_amax_quantize_slow_route(monkeypatch, mode):
    monkeypatch.setenv("NVFP4_FUSED_WAIT_TICKS", "0")
    x = W.lognormal_gradients(1040, 1032, seed=93)
    amax_quantize(x, mode, mask=W.sign_mask(4, 1), seed=4, offset=1)
    monkeypatch.delenv("NVFP4_FUSED_WAIT_TICKS")


def test_amax_quantize_two_pass():
    """More row groups than one workgroup per CU: amax, then the quantize kernel."""
    amax_quantize(W.lognormal_gradients(8208, 4104, seed=13), "rht_sr", mask=W.sign_mask(13, 0), seed=13, offset=0)


@pytest.mark.slow
def test_full_wgrad_colwise_single_read():
    x = W.make("wgrad_colwise_rht_sr_8192x4096")
    amax_quantize(x, "rht_sr", mask=W.sign_mask(2, 0), seed=2, offset=0)


# ---------------------------------------------------------------------------------------------------------------
# Row-wise: the single-read kernel and, where the tiled layout has padding, the quantizer take 128-row x 64-block
# items so that a workgroup owns whole tiles; without padding (rows a multiple of 128, blocks per row of 4) the
# quantizer stores each scale byte at its tiled place (128 x 1024, 256 x 4096, 384 x 512, 1024 x 8192).
# ---------------------------------------------------------------------------------------------------------------
ROW_SHAPES = [(300, 160), (1, 16), (128, 1024), (129, 1040), (1000, 4096), (256, 2064), (385, 3072), (256, 4096),
              (384, 512), (1024, 8192)]


def compare_rows(x, o, a, mode, gmode, mask, seed, offset):
    torch.cuda.synchronize()
    oa = O.amax(x, O.ROWWISE, gmode, mode == "rht_sr", mask)
    ga = a.cpu().numpy()
    assert ((ga.view(np.uint32) == oa.view(np.uint32)) | (np.isnan(ga) & np.isnan(oa))).all()
    oc, os_, og = O.quantize_1x16(x, oa, ROUNDING[mode][1], O.ROWWISE, gmode, mask, seed, offset)
    assert np.array_equal(o.codes.cpu().numpy(), oc), "codes"
    got, sw = o.scales.cpu().numpy(), O.swizzle_scales(os_)
    bad = np.flatnonzero(got != sw)
    assert bad.size == 0, f"tiled scales: {bad.size} mismatches, first at {bad[:6].tolist()}"
    g = o.g.cpu().numpy()
    assert ((g.view(np.uint32) == og.view(np.uint32)) | (np.isnan(g) & np.isnan(og))).all()


@pytest.mark.parametrize("mode", ["rn", "sr", "rht_sr"])
@pytest.mark.parametrize("gmode", [0, 1])
@pytest.mark.parametrize("shape", ROW_SHAPES)
def test_quantize_rowwise(mode, gmode, shape):
    say("tiled quantize row-wise", mode, "per-row" if gmode else "per-tensor", shape)
    mask, seed, offset = 0x9E37, 0x12_3456_789A, 2
    x = W.lognormal_gradients(*shape, seed=(shape[0] * 13 + shape[1]) & 0xFFFF)
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    a = Q.nvfp4_amax(xd, Q.ROWWISE, gmode, use_rht=(mode == "rht_sr"), sign_mask=mask)
    o = Q.alloc_out(*shape, gmode, "cuda", Q.SCALES_TILED)
    o.scales.fill_(0xAB)
    if mode == "rn":
        Q.nvfp4_quantize_rn(xd, a, Q.BLOCK_1X16, Q.ROWWISE, gmode, row_out=o)
    elif mode == "sr":
        Q.nvfp4_quantize_sr(xd, a, seed, offset, Q.ROWWISE, gmode, out=o)
    else:
        Q.nvfp4_quantize_rht_sr(xd, a, mask, seed, offset, Q.ROWWISE, gmode, out=o)
    compare_rows(x, o, a, mode, gmode, mask, seed, offset)


def amax_quantize_rows(x, mode, mask=0x1F2E, seed=0xABCDEF, offset=4):
    say("tiled amax_quantize row-wise", mode, x.shape, offset)
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    o = Q.alloc_out(*x.shape, 0, "cuda", Q.SCALES_TILED)
    o.scales.fill_(0xAB)
    a, _ = Q.nvfp4_amax_quantize(xd, Q.ROWWISE, ROUNDING[mode][0], mask, seed, offset, out=o)
    compare_rows(x, o, a, mode, 0, mask, seed, offset)


@pytest.mark.parametrize("mode", ["rn", "sr", "rht_sr"])
@pytest.mark.parametrize("shape", ROW_SHAPES)
def test_amax_quantize_rowwise_single_read(mode, shape):
    amax_quantize_rows(W.outlier_columns(*shape, seed=(shape[0] * 3 + shape[1]) & 0xFFFF, n_cols=3), mode)


@pytest.mark.parametrize("mode", ["rn", "rht_sr"])
def test_amax_quantize_rowwise_slow_route(monkeypatch, mode):
    monkeypatch.setenv("NVFP4_FUSED_WAIT_TICKS", "0")
    amax_quantize_rows(W.lognormal_gradients(1000, 4096, seed=95), mode, mask=W.sign_mask(6, 1), seed=6, offset=1)
    monkeypatch.delenv("NVFP4_FUSED_WAIT_TICKS")


def test_amax_quantize_rowwise_two_pass():
    """More 128 x 64-block items than CUs: amax, then the tiled quantize kernel."""
    amax_quantize_rows(W.lognormal_gradients(8320, 4096, seed=17), "rht_sr", mask=W.sign_mask(17, 0), seed=17, offset=0)


@pytest.mark.slow
def test_full_fprop_rowwise_single_read():
    """The 8192 x 4096 activations: 256 items, one per CU, on the single-read route."""
    amax_quantize_rows(W.make("fprop_rn_8192x4096"), "rn")
