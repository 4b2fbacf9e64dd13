"""Pins of the four-over-six error modes and bound (pytorch/ao #4852, PR body: the recipe's sweep varies "err_mode"
and "bound"; the page names both knobs without defining them).  The readings pinned here:

  * err_mode MSE: sum of fl(d * d); MAE: sum of |d|; MAXABS: the largest |d| (NaN if any d is NaN), where
    d = fl(xhat - x) per element, xhat the candidate's decoded value; map-to-4 is kept only if its error is strictly
    lower (ties and NaN keep map-to-6);
  * bound B: g = fl(A / (6 B)); B = 448 is the standard scale, B = 256 keeps every map-to-4 scale (at most 1.5 B =
    384) below E4M3's 448.

The blocks are built so that every decoded value and difference is a small integer (g = 1): each mode's error is
then an exact rational, the same in any summation order, and the argmin per mode is computed here with Fractions
from the definition (nearest E2M1 value, ties to the even code), not taken from the oracle.  The three blocks P, Q, R
give each mode a different choice vector, so a mode computed with another mode's measure fails.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

F = np.float32
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
MODES = (O.ERR_MSE, O.ERR_MAE, O.ERR_MAXABS)


def bf16_bits(v) -> np.ndarray:
    v = np.asarray(v, np.float32)
    b = v.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "values must be bf16-representable"
    return (b >> 16).astype(np.uint16)


def nearest_even(q: float) -> float:
    """E2M1 round to nearest, ties to the even code, saturating (non-negative q)."""
    d = np.abs(GRID - q)
    best = np.flatnonzero(d == d.min())
    return float(GRID[best[0] if len(best) == 1 else best[best % 2 == 0][0]])


def diffs(x, g: float, T: float, bamax: float) -> list:
    """Exact differences xhat - x of candidate T for non-negative x whose scale bamax / (T g) is E4M3-exact; the
    multiplier r = fl(1 / fl(s g)) and the products fl(x r) follow the method's binary32 steps."""
    s = F(F(bamax) / F(F(T) * F(g)))
    assert s in (F(4.0), F(6.0), F(256.0), F(384.0))
    r = F(F(1.0) / F(s * F(g)))
    out = []
    for xi in np.asarray(x, np.float64):
        xh = Fraction(nearest_even(float(F(F(xi) * r)))) * Fraction(float(s)) * Fraction(float(g))
        out.append(xh - Fraction(xi))
    return out


def exact_error(d: list, mode: int) -> Fraction:
    if mode == O.ERR_MSE:
        return sum(t * t for t in d)
    if mode == O.ERR_MAE:
        return sum(abs(t) for t in d)
    return max(abs(t) for t in d)


def expected_choice(x, mode, g=1.0, bamax=None) -> int:
    bamax = float(np.max(x)) if bamax is None else bamax
    e6 = exact_error(diffs(x, g, 6.0, bamax), mode)
    e4 = exact_error(diffs(x, g, 4.0, bamax), mode)
    return int(e4 < e6)


def block(*vals) -> np.ndarray:
    x = np.zeros(16, np.float32)
    x[:len(vals)] = vals
    return x


# (x, e6, e4) per element at block maximum 24, g = 1 (map-to-6 scale 4, map-to-4 scale 6):
#   3 -> (1, 0), 9 -> (1, 0), 15 -> (1, 3), 18 -> (2, 0), 16 -> (0, 2), 20 -> (4, 2); 24, 12, 6, 0 -> (0, 0)
P = block(24, 15, 3, 9, 3, 9)            # MSE 5 vs 9 -> 6;  MAE 5 vs 3 -> 4;  MAXABS 1 vs 3 -> 6
Q = block(24, 15, 18, 18, 18)            # MSE 13 vs 9 -> 4; MAE 7 vs 3 -> 4;  MAXABS 2 vs 3 -> 6
R = block(24, 20, 16, 16, 16, 16)        # MSE 16 vs 20 -> 6; MAE 4 vs 10 -> 6; MAXABS 4 vs 2 -> 4
TIE = block(24, 12, 6, 6, 12)            # exact on both grids: every mode ties
EXPECT = {O.ERR_MSE: [0, 1, 0], O.ERR_MAE: [1, 1, 0], O.ERR_MAXABS: [0, 0, 1]}
AMAX_G1 = np.array([2688.0], np.float32)   # bound 448: g = 2688 / 2688 = 1


def test_construction_separates_the_modes():
    for mode in MODES:
        assert [expected_choice(b, mode) for b in (P, Q, R)] == EXPECT[mode]
    assert len({tuple(v) for v in EXPECT.values()}) == 3
    for mode in MODES:
        assert expected_choice(TIE, mode) == 0


@pytest.mark.parametrize("mode", MODES)
def test_oracle_1x16_choice_per_mode(mode):
    x = np.stack([P, Q, R, TIE])
    for f32 in (False, True):
        if f32:
            codes, scales, g, choice = O.quantize_4o6_f32(x, AMAX_G1, O.G_PER_TENSOR, err_mode=mode)
        else:
            codes, scales, g, choice = O.quantize_4o6(bf16_bits(x), AMAX_G1, O.G_PER_TENSOR, err_mode=mode)
        assert g[0] == 1.0
        assert choice[:, 0].tolist() == EXPECT[mode] + [0]
        # the kept scale is the chosen candidate's: 24 / 4 = 6 for map-to-4, 24 / 6 = 4 for map-to-6
        assert [O.e4m3_decode(int(s)) for s in scales[:, 0]] == [6.0 if c else 4.0 for c in EXPECT[mode] + [0]]


def test_error_sums_are_exact_so_order_does_not_matter():
    """Every squared and absolute difference above is a small integer, so the binary32 tree sum is the exact sum:
    the choices pinned here do not depend on the summation order (that order is pinned separately)."""
    for b in (P, Q, R, TIE):
        for T in (6.0, 4.0):
            d = diffs(b, 1.0, T, 24.0)
            assert all(t.denominator == 1 and abs(t) <= 4 for t in d)


def test_nan_and_inf_keep_map_to_6_in_every_mode():
    x = np.stack([block(24, 15, np.nan), block(24, 20, np.inf)])
    for mode in MODES:
        _, _, _, choice = O.quantize_4o6(bf16_bits(x), AMAX_G1, O.G_PER_TENSOR, err_mode=mode)
        assert choice[:, 0].tolist() == [0, 0]


def tile_with_rows(rows_vals) -> np.ndarray:
    """A 16x16 tile: row i holds rows_vals[i] (placed in columns 0..), the rest zero."""
    t = np.zeros((16, 16), np.float32)
    for i, v in enumerate(rows_vals):
        t[i, :len(v)] = v
    return t


def test_oracle_16x16_modes_combine_rows():
    """Tile 0 is block P in one row; tile 1 spreads P's elements over six rows (one nonzero each, the tile maximum
    in row 0), so the tile error is the combination of row errors: a sum for MSE and MAE, a maximum for MAXABS.
    Tiles 2 and 3 do the same for R.  Either way the tile's choice is the block's."""
    spread_p = tile_with_rows([[24], [15], [3], [9], [3], [9]])
    spread_r = tile_with_rows([[24], [20], [16], [16], [16], [16]])
    x = np.concatenate([tile_with_rows([P]), spread_p, tile_with_rows([R]), spread_r], axis=1)
    for mode in MODES:
        exp = [EXPECT[mode][0], EXPECT[mode][0], EXPECT[mode][2], EXPECT[mode][2]]
        for t in range(4):
            tile = x[:, 16 * t:16 * t + 16]
            assert expected_choice(tile.ravel(), mode, bamax=24.0) == exp[t]
        for f32 in (False, True):
            if f32:
                (_, sw, gw), (_, st, _), choice = O.quantize_4o6_16x16_f32(x, AMAX_G1, err_mode=mode)
            else:
                (_, sw, gw), (_, st, _), choice = O.quantize_4o6_16x16(bf16_bits(x), AMAX_G1, err_mode=mode)
            assert gw[0] == 1.0 and choice[0].tolist() == exp, (mode, f32, choice)
            assert [O.e4m3_decode(int(sw[0, t])) for t in range(4)] == [6.0 if c else 4.0 for c in exp]


def test_bound_sets_g_in_closed_form():
    """g = A / (6 B): A = 6 B 2^k gives g = 2^k exactly, and the tensor maximum's map-to-6 scale is then B itself
    (E4M3 256 = 0x78, 448 = 0x7E); its map-to-4 scale is 1.5 B = 384 (0x7C) for B = 256 and saturates at 448 for
    B = 448."""
    for bound, k, sb6, sb4 in ((256, -3, 0x78, 0x7C), (256, 4, 0x78, 0x7C), (448, 0, 0x7E, 0x7E), (448, 5, 0x7E, 0x7E)):
        A = 6.0 * bound * 2.0 ** k
        x = block(A)[None, :]
        for mode in MODES:
            _, s, g, choice = O.quantize_4o6(bf16_bits(x), np.array([A], np.float32), O.G_PER_TENSOR, err_mode=mode,
                                             bound=bound)
            assert g[0] == 2.0 ** k
            # a lone maximum is exact on both grids (6 * B g = A, and 4 * 1.5 B g = A): a tie keeps map-to-6
            assert choice[0, 0] == 0 and s[0, 0] == sb6
        assert O.e4m3_encode(1.5 * bound) == sb4


def test_bound_changes_the_choice():
    """Block Q scaled by 64 (maximum 1536 = the tensor amax).  Bound 256: g = 1536 / 1536 = 1, scales 256 and 384,
    every difference a multiple of 64 of Q's, so MSE keeps map-to-4.  Bound 448: the map-to-4 scale 1536 / fl(4 g)
    (about 672) saturates to 448, the map-to-6 scale (about 448) rounds to 448 as well, so the two candidates are the
    same encoding, their errors tie, and map-to-6 is kept."""
    x = (Q * 64.0)[None, :]
    A = np.array([1536.0], np.float32)
    d6 = diffs(x[0], 1.0, 6.0, 1536.0)
    d4 = diffs(x[0], 1.0, 4.0, 1536.0)
    assert exact_error(d4, O.ERR_MSE) < exact_error(d6, O.ERR_MSE)
    _, s, g, choice = O.quantize_4o6(bf16_bits(x), A, O.G_PER_TENSOR, bound=256)
    assert g[0] == 1.0 and choice[0, 0] == 1 and s[0, 0] == 0x7C
    _, s, g, choice = O.quantize_4o6(bf16_bits(x), A, O.G_PER_TENSOR, bound=448)
    g448 = float(g[0])
    assert F(F(1536.0) / F(F(4.0) * F(g448))) > F(448.0)              # map-to-4 saturates
    assert abs(float(F(F(1536.0) / F(F(6.0) * F(g448)))) - 448.0) < 1e-3   # map-to-6 lands on 448
    assert choice[0, 0] == 0 and s[0, 0] == 0x7E


def test_bound_256_never_saturates_map_to_4():
    """With B = 256 the largest possible block scale of either candidate is 1.5 * 256 = 384 < 448 (on noisy data
    with per-tensor and per-row g); with B = 448 the block holding the maximum gets scale 448 whichever candidate
    is kept (map-to-6 lands on 448, map-to-4 saturates there)."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.standard_normal((64, 1)))).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)          # truncated to bf16
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    for gmode, amax in ((O.G_PER_TENSOR, np.abs(xf).max(keepdims=True).ravel()),
                        (O.G_PER_ROW, np.abs(xf).max(axis=1))):
        amax = amax.astype(np.float32)
        for mode in MODES:
            _, s, _, choice = O.quantize_4o6(xb, amax, gmode, err_mode=mode, bound=256)
            dec = np.vectorize(O.e4m3_decode)(s)
            assert dec.max() <= 384.0
            assert choice.any() and not choice.all()
            _, s, _, _ = O.quantize_4o6(xb, amax, gmode, err_mode=mode, bound=448)
            assert np.vectorize(O.e4m3_decode)(s).max() == 448.0


def test_knob_validation():
    x = bf16_bits(block(1.0)[None, :])
    with pytest.raises(Exception):
        O.quantize_4o6(x, AMAX_G1, O.G_PER_TENSOR, err_mode=3)
    for b in (0, 449):
        with pytest.raises(Exception):
            O.quantize_4o6(x, AMAX_G1, O.G_PER_TENSOR, bound=b)
