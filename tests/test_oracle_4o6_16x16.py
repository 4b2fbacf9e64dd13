"""Pins for the oracle's four-over-six with 16x16 tiles (CPU only).

The reading taken for the tile error (each row by the pinned width-16 tree, then the 16 row sums by the same tree)
is pinned by reduction to the 1x16 case: a tile whose 16 rows are the same block has exactly 16 times that block's
error in both candidates, so it must make the 1x16 choice and produce the 1x16 codes in every row.  The rest is
pinned to closed forms (a tile on the map-to-4 grid decodes exactly and picks 4; an exact tie keeps 6), to the
exact-rational argmin of the two candidates' errors, to the transpose relation of the two orientations, and to
the NaN rule.
"""
from fractions import Fraction

import numpy as np

from nvfp4_quantization_amd import workloads as W

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
SIGNED = GRID + [-v for v in GRID]


def bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def nibbles(codes):
    out = np.zeros((codes.shape[0], 2 * codes.shape[1]), np.uint8)
    out[:, 0::2] = codes & 0xF
    out[:, 1::2] = codes >> 4
    return out


def test_identical_rows_reduce_to_the_1x16_choice(oracle):
    blocks = W.heavy_tail_rows(24, 16, seed=61, inject=False)        # 24 blocks of 16
    amax = np.array([np.max(np.abs(f32(blocks)))], np.float32)
    x = np.zeros((16, 16 * 24), np.uint16)
    for t in range(24):
        x[:, 16 * t:16 * t + 16] = blocks[t]                         # tile t: block t in every row
    (cw, sw, gw), _, choice = oracle.quantize_4o6_16x16(x, amax)
    c1, s1, g1, ch1 = oracle.quantize_4o6(blocks, amax, gmode=0)
    assert gw[0] == g1[0]
    for t in range(24):
        assert choice[0, t] == ch1[t, 0]
        assert np.all(sw[:, t] == s1[t, 0])
        np.testing.assert_array_equal(cw[:, 8 * t:8 * t + 8], np.repeat(c1[t:t + 1], 16, axis=0))
    assert ch1.any() and not ch1.all()                               # both outcomes are exercised


def test_tile_on_map_to_4_grid_picks_4_and_decodes_exactly(oracle):
    """g = 1 (amax 2688 passed in); a tile of 4-grid values times 1.5 (s4 = 1.5 exactly) decodes exactly under
    map-to-4, while map-to-6 (s6 = 1) cannot represent 4.5."""
    rng = np.random.default_rng(62)
    vals = rng.choice([4, 3, 2, 1.5, 1, 0.5, 0, -4, -3, -2, -1.5, -1, -0.5], size=(16, 16)).astype(np.float64)
    vals[5, 9] = 4.0                                                 # tile max 6
    x = (1.5 * vals).astype(np.float32)
    (cw, sw, gw), (ct, st, gt), choice = oracle.quantize_4o6_16x16(bits(x), np.array([2688.0], np.float32))
    assert choice[0, 0] == 1 and np.all(sw == oracle.e4m3_encode(1.5)) and np.all(st == oracle.e4m3_encode(1.5))
    np.testing.assert_array_equal(oracle.dequantize(cw, sw, gw), x)
    np.testing.assert_array_equal(oracle.dequantize(ct, st, gt), x.T)


def test_exact_tie_keeps_6(oracle):
    x = np.where(np.arange(256).reshape(16, 16) % 3 == 0, 6.0, -6.0).astype(np.float32)
    (cw, sw, gw), _, choice = oracle.quantize_4o6_16x16(bits(x), np.array([2688.0], np.float32))
    assert choice[0, 0] == 0 and np.all(sw == 0x38)


def _exact_tile_error(v, codes, sb, g, oracle):
    sbf = Fraction(float(oracle.e4m3_decode(sb)))
    gf = Fraction(float(np.float32(g)))
    return sum((Fraction(SIGNED[c]) * sbf * gf - Fraction(float(a))) ** 2 for a, c in zip(v, codes))


def test_choice_is_exact_argmin_when_errors_are_well_separated(oracle):
    """The candidate with the smaller exact squared tile error (rational arithmetic on the decoded values, from
    the pinned block-scale and E2M1 step functions) is the one kept, except where the two exact errors are within
    1e-4 relative of each other."""
    # tiles alternate uniform values (map-to-4 usually wins) and Gaussian ones (map-to-6 usually wins), each scaled
    # by a power of two chosen per tile so that tile maxima span the tensor's range
    rng = np.random.default_rng(63)
    xf = np.zeros((4, 16, 6, 16), np.float32)
    for ti in range(4):
        for tj in range(6):
            t = rng.uniform(-1, 1, (16, 16)) if (ti + tj) % 2 else rng.normal(0, 1, (16, 16))
            xf[ti, :, tj, :] = t * 2.0 ** -((3 * ti + tj) % 7)
    x = bits(xf.reshape(64, 96))
    xf = f32(x).reshape(4, 16, 6, 16)
    x = bits(xf.reshape(64, 96))
    xf = f32(x)
    amax = oracle.amax(x)
    (cw, sw, gw), _, choice = oracle.quantize_4o6_16x16(x, amax)
    checked = 0
    for ti in range(4):
        for tj in range(6):
            v = xf[16 * ti:16 * ti + 16, 16 * tj:16 * tj + 16].ravel()
            cand = []
            for T in (6.0, 4.0):
                sb, r = oracle.block_scale(float(np.max(np.abs(v))), float(gw[0]), T)
                c = [oracle.e2m1_rn(np.float32(a) * r) for a in v]
                cand.append(_exact_tile_error(v, c, sb, gw[0], oracle))
            if abs(cand[0] - cand[1]) > Fraction(1, 10**4) * max(cand[0], cand[1]):
                assert choice[ti, tj] == (1 if cand[1] < cand[0] else 0), (ti, tj)
                checked += 1
            assert cand[choice[ti, tj]] <= cand[0] * (1 + Fraction(1, 10**4))
    assert checked >= 12 and choice.any() and not choice.all()


def test_wt_is_the_transpose_of_w(oracle):
    x = W.weight_outliers(48, 80, seed=64)
    (cw, sw, gw), (ct, st, gt), choice = oracle.quantize_4o6_16x16(x, oracle.amax(x))
    np.testing.assert_array_equal(nibbles(ct), nibbles(cw).T)
    np.testing.assert_array_equal(np.repeat(sw[::16], 16, axis=0), sw)
    np.testing.assert_array_equal(st, np.repeat(sw[::16], 1, axis=0).T.repeat(16, axis=0))
    assert gw[0] == gt[0]


def test_nan_tile(oracle):
    """A NaN in one tile (with a finite tensor amax given): that tile's scale is the NaN code 0x7F and its codes
    0x7 (every multiplier is NaN); map-to-6 is kept; the other tiles are as without the NaN."""
    x = W.weight_outliers(32, 32, seed=65)
    a = oracle.amax(x)
    clean = oracle.quantize_4o6_16x16(x, a)
    x2 = x.copy()
    x2[20, 3] = 0x7FC0
    (cw, sw, gw), _, choice = oracle.quantize_4o6_16x16(x2, a)
    assert np.all(sw[16:, 0] == 0x7F) and np.all(nibbles(cw)[16:, :16] == 0x7) and choice[1, 0] == 0
    np.testing.assert_array_equal(cw[:16], clean[0][0][:16])
    np.testing.assert_array_equal(cw[16:, 8:], clean[0][0][16:, 8:])
