"""Pins of the oracle's binary32-input four-over-six ([P3]: the reference quantizer takes bf16 or fp32 inputs).

The binary32 path must agree with the bf16 path wherever the input is representable in bf16 (the loader is the
only difference), choose the exact-rational argmin on inputs that are not (full 24-bit mantissas, so a dropped or
truncated low half would change the result), decode a block on the map-to-4 grid exactly, and take the amax as
the NaN-dominant maximum magnitude.
"""
from fractions import Fraction

import numpy as np
import torch

from conftest import read_golden
from nvfp4_quantization_amd import workloads as W

GRID = [float(v) for v in read_golden("e2m1_grid.txt")[0]]
SIGNED = np.array(GRID + [-v for v in GRID], dtype=np.float64)


def e4m3(sb):
    return float(torch.tensor([sb], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32)[0])


def nibbles(codes):
    out = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = codes & 0xF
    out[:, 1::2] = codes >> 4
    return out


def test_bf16_representable_inputs_match_the_bf16_path(oracle):
    xb = W.heavy_tail_rows(32, 512, seed=5, inject=True)           # bf16 patterns, with NaN / inf rows
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    for gmode in (0, 1):
        a_b, a_f = oracle.amax(xb, gmode=gmode), oracle.amax_f32(xf, gmode)
        assert np.array_equal(a_b.view(np.uint32), a_f.view(np.uint32))
        rb = oracle.quantize_4o6(xb, a_b, gmode=gmode)
        rf = oracle.quantize_4o6_f32(xf, a_f, gmode)
        for u, v in zip(rb, rf):
            assert np.array_equal(np.asarray(u).view(np.uint8), np.asarray(v).view(np.uint8))


def test_amax_f32_matches_numpy_and_nan_dominates(oracle):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 64)).astype(np.float32) * np.float32(1.000001)
    assert oracle.amax_f32(x, 0)[0] == np.abs(x).max()
    assert np.array_equal(oracle.amax_f32(x, 1), np.abs(x).max(axis=1))
    x[3, 5] = np.inf
    x[7, 9] = -np.nan
    a = oracle.amax_f32(x, 1)
    assert np.isinf(a[3]) and np.isnan(a[7]) and np.isnan(oracle.amax_f32(x, 0)[0])


def test_choice_is_exact_argmin_on_full_mantissas(oracle):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((16, 256)) * np.exp(rng.uniform(-3, 3, (16, 1)))).astype(np.float32)
    x[:, ::7] *= np.float32(3.3)                                    # uneven blocks so both choices occur
    assert (x.view(np.uint32) & 0xFFFF).any()                       # not bf16-representable
    a = oracle.amax_f32(x, 1)
    codes, scales, g, choice = oracle.quantize_4o6_f32(x, a, 1)
    nib = nibbles(codes)
    checked = 0
    for r in range(x.shape[0]):
        gf = Fraction(float(g[r]))
        for b in range(x.shape[1] // 16):
            blk = x[r, 16 * b:16 * b + 16]
            cand = []
            for T in (6.0, 4.0):
                sb, rr = oracle.block_scale(float(np.max(np.abs(blk))), float(g[r]), T)
                c = [oracle.e2m1_rn(np.float32(v) * rr) for v in blk]
                sbf = Fraction(e4m3(sb))
                cand.append((sum((Fraction(float(SIGNED[k])) * sbf * gf - Fraction(float(v))) ** 2
                                 for v, k in zip(blk, c)), sb, c))
            e6, e4 = cand[0][0], cand[1][0]
            if abs(e6 - e4) > Fraction(1, 10**4) * max(e6, e4):
                pick = 1 if e4 < e6 else 0
                assert choice[r, b] == pick
                assert scales[r, b] == cand[pick][1] and list(nib[r, 16 * b:16 * b + 16]) == cand[pick][2]
                checked += 1
    assert checked > 100 and choice.any() and not choice.all()


def test_block_on_map_to_4_grid_decodes_exactly(oracle):
    """g = 1 (amax 2688 passed in); E2M1 values times 1.5 have full binary32 meaning (no bf16 involved): map-to-4
    (scale 1.5) reproduces them exactly, map-to-6 (scale 1) cannot hold 4.5."""
    vals = np.array([4, 3, 2, 1.5, 1, 0.5, 0, -4, -3, -2, -1.5, -1, -0.5, 4, 3, 2], np.float64)
    x = np.array([1.5 * vals], np.float32)
    codes, scales, g, choice = oracle.quantize_4o6_f32(x, np.array([2688.0], np.float32), 0)
    assert choice[0, 0] == 1 and scales[0, 0] == oracle.e4m3_encode(1.5)
    np.testing.assert_array_equal(oracle.dequantize(codes, scales, g), x)


def test_16x16_tiles_match_the_bf16_path_on_bf16_inputs(oracle):
    xb = W.weight_outliers(64, 96, seed=8)
    xb[3, 5] = 0x7FC0                                               # a NaN tile
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    a = oracle.amax(xb)
    rb = oracle.quantize_4o6_16x16(xb, a)
    rf = oracle.quantize_4o6_16x16_f32(xf, a)
    for u, v in zip(rb[0] + rb[1] + (rb[2],), rf[0] + rf[1] + (rf[2],)):
        assert np.array_equal(np.asarray(u).view(np.uint8), np.asarray(v).view(np.uint8))


def test_16x16_tile_of_identical_rows_makes_the_1x16_choice(oracle):
    """A tile of 16 copies of one full-mantissa row: 16 times the block's error, so the 1x16 choice and codes."""
    rng = np.random.default_rng(21)
    for trial in range(20):
        row = (rng.standard_normal(16) * 2.0 ** rng.integers(-6, 6)).astype(np.float32)
        x = np.tile(row, (16, 1))
        a = np.array([2688.0], np.float32)
        (cw, sw, _), _, choice = oracle.quantize_4o6_16x16_f32(x, a)
        c1, s1, _, ch1 = oracle.quantize_4o6_f32(row[None, :], a, 0)
        assert choice[0, 0] == ch1[0, 0] and sw[0, 0] == s1[0, 0]
        assert all(np.array_equal(cw[i], c1[0]) for i in range(16))
