"""Pin of the four-over-six error-sum order (pytorch/ao #4852, PR body: the width-16 error reduction is a clamped
shuffle-down tree, and the kernel is bitwise identical to the reference because that order is fixed).

A block is built whose two candidates' squared errors hold the same values {1, 2^-24, 2^-24} at different positions,
so that their sums differ only by the order of the additions: 1 + 2^-24 is an exact tie that rounds back to 1, while
2^-24 + 2^-24 + 1 is exactly 1 + 2^-23.  The order decides which candidate is kept:

  * an independent model of the clamped shuffle-down tree (16 lanes; for off = 8, 4, 2, 1 every lane adds the value
    of lane i + off, or its own value where i + off falls outside the width; the result is lane 0) keeps map-to-6;
  * a left-to-right sum and a pairwise tree with strides 1, 2, 4, 8 both keep map-to-4.

The oracle must make the shuffle-down choice.  The per-element errors are derived here from the definition (nearest
E2M1 value with ties to the even code), not taken from the oracle.
"""
import numpy as np

import oracle as O

F = np.float32
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def bf16_bits(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, np.float32)
    b = v.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "values must be bf16-representable"
    return (b >> 16).astype(np.uint16)


def shuffle_down_sum(e) -> F:
    v = [F(t) for t in e]
    for off in (8, 4, 2, 1):
        v = [F(v[i] + (v[i + off] if i + off < 16 else v[i])) for i in range(16)]
    return v[0]


def sequential_sum(e) -> F:
    s = F(0)
    for t in e:
        s = F(s + F(t))
    return s


def stride_up_sum(e) -> F:
    v = [F(t) for t in e]
    for h in (1, 2, 4, 8):
        for i in range(0, 16, 2 * h):
            v[i] = F(v[i] + v[i + h])
    return v[0]


def nearest_even(q: float) -> float:
    """E2M1 round to nearest, ties to the even code, saturating (non-negative q only here)."""
    d = np.abs(GRID - q)
    best = np.flatnonzero(d == d.min())
    return float(GRID[best[0] if len(best) == 1 else best[best % 2 == 0][0]])


def candidate_errors(x: np.ndarray, g: float, T: float, bamax: float | None = None) -> list:
    """Squared errors fl(fl(xhat - x)^2) of candidate T for non-negative values whose scale (from bamax, the block
    or tile maximum) is exact here."""
    bamax = F(np.max(x) if bamax is None else bamax)
    s = F(bamax / F(F(T) * F(g)))
    assert s in (F(4.0), F(6.0))                       # E4M3-exact scales for this construction
    r = F(F(1.0) / F(s * F(g)))
    out = []
    for xi in x:
        q = F(F(xi) * r)
        xh = F(F(F(nearest_even(float(q))) * s) * F(g))
        d = F(xh - F(xi))
        out.append(F(d * d))
    return out


def discriminating_block() -> np.ndarray:
    x = np.zeros(16, np.float32)
    x[0] = x[4] = 2.0 ** -12     # both candidates round it to 0: error 2^-24 in both
    x[1] = 4.0                   # on the map-to-6 grid (scale 4), 1 away from map-to-4's 3
    x[8] = 3.0                   # on the map-to-4 grid (scale 6); map-to-6 rounds the tie 0.75 up to 4
    x[15] = 24.0                 # the block maximum, exact in both
    return x


def test_construction_discriminates_the_orders():
    x = discriminating_block()
    e6 = candidate_errors(x, 1.0, 6.0)
    e4 = candidate_errors(x, 1.0, 4.0)
    assert sorted(e6) == sorted(e4) and max(e6) == F(1.0) and F(2.0 ** -24) in e6
    keep4 = lambda s: s(e4) < s(e6)
    assert not keep4(shuffle_down_sum)                 # the pinned order keeps map-to-6 ...
    assert keep4(sequential_sum) and keep4(stride_up_sum)   # ... every other order tried keeps map-to-4
    assert shuffle_down_sum(e6) == F(1.0) and shuffle_down_sum(e4) == F(1.0 + 2.0 ** -23)


def test_oracle_1x16_keeps_the_shuffle_down_choice():
    x = discriminating_block()
    amax = np.array([2688.0], np.float32)             # g = 1
    codes, scales, g, choice = O.quantize_4o6(bf16_bits(x)[None, :], amax, O.G_PER_TENSOR)
    assert g[0] == 1.0 and choice[0, 0] == 0
    assert O.e4m3_decode(int(scales[0, 0])) == 4.0   # the map-to-6 scale
    codes32, scales32, _, choice32 = O.quantize_4o6_f32(x[None, :], amax, O.G_PER_TENSOR)
    assert choice32[0, 0] == 0 and np.array_equal(codes32, codes) and np.array_equal(scales32, scales)


def tiles_for_16x16() -> np.ndarray:
    """Two tiles side by side: tile 0 carries the block as its row 0 (all other rows zero apart from the tile
    maximum in row 15), so its error is that row's width-16 sum; tile 1 puts the same three errors in rows 0, 4, 8
    and 1 (one nonzero element each), so the order that matters is the one over the 16 row sums."""
    x = np.zeros((16, 32), np.float32)
    x[0, :16] = discriminating_block()
    x[0, 15] = 0.0
    x[15, 15] = 24.0
    x[0, 16 + 3] = x[4, 16 + 3] = 2.0 ** -12
    x[1, 16 + 5] = 4.0
    x[8, 16 + 7] = 3.0
    x[15, 16 + 15] = 24.0
    return x


def test_construction_of_row_sums_discriminates():
    tiles = tiles_for_16x16()
    for t, by_rows in ((0, False), (1, True)):
        x = tiles[:, 16 * t:16 * t + 16]
        rs = {T: [shuffle_down_sum(candidate_errors(x[i], 1.0, T, bamax=24.0)) for i in range(16)] for T in (6.0, 4.0)}
        if by_rows:                                    # single-term rows: the order over the row sums decides
            assert rs[6.0][8] == F(1.0) and rs[4.0][1] == F(1.0) and rs[6.0][0] == rs[4.0][4] == F(2.0 ** -24)
        keep4 = lambda s: s(rs[4.0]) < s(rs[6.0])
        assert keep4(sequential_sum) == by_rows and keep4(stride_up_sum) == by_rows
        assert not keep4(shuffle_down_sum)


def test_oracle_16x16_keeps_the_shuffle_down_choice():
    x = tiles_for_16x16()
    amax = np.array([2688.0], np.float32)
    (cw, sw, gw), (ct, st, gt), choice = O.quantize_4o6_16x16(bf16_bits(x), amax)
    assert gw[0] == 1.0 and choice.tolist() == [[0, 0]]
    assert O.e4m3_decode(int(sw[0, 0])) == 4.0 and O.e4m3_decode(int(sw[0, 1])) == 4.0
    (cw32, sw32, _), _, choice32 = O.quantize_4o6_16x16_f32(x, amax)
    assert choice32.tolist() == [[0, 0]] and np.array_equal(cw32, cw) and np.array_equal(sw32, sw)


def test_planted_sequential_order_would_fail():
    """The construction catches a plausible mistake: re-deciding with a left-to-right sum flips the choice, so an
    oracle that summed sequentially would disagree with the expected choice above."""
    x = discriminating_block()
    e6 = candidate_errors(x, 1.0, 6.0)
    e4 = candidate_errors(x, 1.0, 4.0)
    seq_choice = int(sequential_sum(e4) < sequential_sum(e6))
    _, _, _, choice = O.quantize_4o6(bf16_bits(x)[None, :], np.array([2688.0], np.float32), O.G_PER_TENSOR)
    assert seq_choice == 1 and choice[0, 0] != seq_choice
