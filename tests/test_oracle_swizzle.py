"""Pins of the oracle's tiled scale layout (the FP4 GEMM's SWIZZLE_32_4_4 scale layout, [P2, approach]).

The pages name the layout only; the reading is spelled out by its name: tiles of 128 rows x 4 scale columns, each
stored as a [32][4][4] array (row 32 b + a of the tile, column c, at byte 16 a + 4 b + c), tiles row-tile major,
zero padding to whole tiles.  Pinned here by an independent array formulation (pad, split the row index as
(tile, b, a), permute the axes), by the name's factorisation on one tile, by bijectivity with zero padding, and
by the tile order on multi-tile shapes.
"""
import numpy as np
import pytest

import oracle as O

SHAPES = [(0, 0), (0, 5), (3, 0), (1, 1), (127, 3), (128, 4), (129, 5), (256, 8), (300, 65), (1000, 17)]


def labels(rv, nb):
    """Distinct-enough nonzero bytes: the value identifies (m, k) modulo 251."""
    m, k = np.meshgrid(np.arange(rv), np.arange(nb), indexing="ij")
    return ((m * 7 + k * 13) % 251 + 1).astype(np.uint8)


def by_axes(s):
    """The same layout by array operations: pad, view as (R, b, a, B, c), store as (R, B, a, b, c)."""
    rv, nb = s.shape
    rt, bt = -(-rv // 128), -(-nb // 4)
    p = np.zeros((rt * 128, bt * 4), np.uint8)
    p[:rv, :nb] = s
    return p.reshape(rt, 4, 32, bt, 4).transpose(0, 3, 2, 1, 4).reshape(-1)


@pytest.mark.parametrize("shape", SHAPES)
def test_matches_axis_permutation(shape):
    s = labels(*shape)
    out = O.swizzle_scales(s)
    assert out.size == O.swizzled_size(*shape)
    np.testing.assert_array_equal(out, by_axes(s))


def test_one_tile_is_the_named_32x4x4_array():
    s = np.random.default_rng(0).integers(0, 256, (128, 4), dtype=np.uint8)
    t = O.swizzle_scales(s).reshape(32, 4, 4)
    for a in range(32):
        for b in range(4):
            for c in range(4):
                assert t[a, b, c] == s[32 * b + a, c]


@pytest.mark.parametrize("shape", [(129, 5), (300, 65), (1000, 17)])
def test_bijective_with_zero_padding(shape):
    rv, nb = shape
    rng = np.random.default_rng(rv + nb)
    s = rng.integers(1, 256, shape, dtype=np.uint8)           # no zero in the input
    out = O.swizzle_scales(s)
    assert np.count_nonzero(out) == rv * nb                   # every scale lands once, padding is zero
    assert np.array_equal(np.sort(out[out != 0]), np.sort(s.reshape(-1)))
    # one input byte changed changes exactly one output byte, at a position no other input byte uses
    where = {}
    for m, k in {(0, 0), (rv - 1, nb - 1), (rv // 2, nb // 3), (127, 3), (128, 4), (31, 0), (32, 0)}:
        s2 = s.copy()
        s2[m, k] ^= 0xFF
        d = np.flatnonzero(O.swizzle_scales(s2) != out)
        assert d.size == 1
        where[(m, k)] = int(d[0])
    assert len(set(where.values())) == len(where)


def test_tile_order_is_row_tile_major():
    # scale (m, k) of tile (R, B) sits in the 512-byte tile R * ceil(nb/4) + B
    rv, nb = 384, 12
    for m, k in [(0, 0), (0, 4), (0, 8), (128, 0), (130, 5), (383, 11)]:
        s = np.zeros((rv, nb), np.uint8)
        s[m, k] = 0x5A
        pos = int(np.flatnonzero(O.swizzle_scales(s))[0])
        assert pos // 512 == (m // 128) * 3 + k // 4
        assert pos % 512 == 16 * (m % 32) + 4 * ((m % 128) // 32) + k % 4
