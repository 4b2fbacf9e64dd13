"""Pins for the oracle's element and scale formats (CPU only).

E2M1 round-to-nearest is checked against an independent closed form (the midpoint thresholds of the printed grid)
over every bf16 pattern, the neighbourhood of every threshold and millions of random binary32 patterns.  E2M1
stochastic rounding is checked against exact rational arithmetic for every one of the 256 random bytes.  E4M3 is
checked against torch's float8_e4m3fn conversion (an independent library routine) on every code and on dense
sweeps of the finite range.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import read_golden

GRID = [Fraction(v) for v in read_golden("e2m1_grid.txt")[0]]


def test_grid_decode_matches_page(oracle):
    """Codes 0..7 decode to the printed magnitudes in order, 8..15 to their negatives."""
    for m, v in enumerate(GRID):
        assert oracle.e2m1_decode(m) == float(v)
        dec_neg = oracle.e2m1_decode(8 + m)
        assert dec_neg == -float(v) and np.signbit(np.float32(dec_neg))


def test_rn_examples_from_page(oracle):
    for q, expected in read_golden("rn_examples.txt"):
        code = oracle.e2m1_rn(float(q))
        assert oracle.e2m1_decode(code) == float(expected), (q, code)


def _rn_by_thresholds(q):
    """Independent closed form: nearest grid magnitude with ties to the even code.  The midpoints of the grid are
    0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5; at a midpoint the even code (0, 2, 4, 6) wins, so the comparison is <=
    towards an even code and < towards an odd one."""
    q = np.asarray(q, dtype=np.float32)
    with np.errstate(invalid="ignore"):
        t = np.abs(q.astype(np.float64))
    m = np.full(t.shape, 7, dtype=np.uint8)
    m[t <= 5.0] = 6
    m[t < 3.5] = 5
    m[t <= 2.5] = 4
    m[t < 1.75] = 3
    m[t <= 1.25] = 2
    m[t < 0.75] = 1
    m[t <= 0.25] = 0
    code = m | np.where(np.signbit(q), 8, 0).astype(np.uint8)
    code[np.isnan(q)] = 7
    return code


def _neighbourhood(values, radius):
    out = []
    for v in values:
        b = np.array([v], dtype=np.float32).view(np.uint32)[0]
        span = np.arange(-radius, radius + 1, dtype=np.int64) + int(b)
        span = span[(span >= 0) & (span < 2**32)]
        out.append(span.astype(np.uint32).view(np.float32))
    return np.concatenate(out)


def test_rn_exhaustive_bf16_and_threshold_neighbourhoods(oracle):
    every_bf16 = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    points = [0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0, np.inf]
    near = _neighbourhood(points, 3000)
    near = np.concatenate([near, -near])
    q = np.concatenate([every_bf16, near])
    np.testing.assert_array_equal(oracle.e2m1_rn_array(q), _rn_by_thresholds(q))


def test_rn_random_binary32_patterns(oracle):
    rng = np.random.default_rng(7)
    a = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    b = rng.uniform(-7.0, 7.0, size=2_000_000).astype(np.float32)
    q = np.concatenate([a, b])
    np.testing.assert_array_equal(oracle.e2m1_rn_array(q), _rn_by_thresholds(q))


def test_rn_special_values(oracle):
    assert oracle.e2m1_rn(float("nan")) == 0x7
    assert oracle.e2m1_rn(float("inf")) == 0x7
    assert oracle.e2m1_rn(float("-inf")) == 0xF
    assert oracle.e2m1_rn(-0.0) == 0x8
    assert oracle.e2m1_rn(1e30) == 0x7


def _sr_expected_up_count(t: float):
    """Exact rational P(up)*256 for the reading 'up iff rho < floor(256 (t - a) / (b - a))'."""
    tf = Fraction(float(np.float32(t)))
    lo = max(k for k, g in enumerate(GRID) if g <= tf)
    a, b = GRID[lo], GRID[lo + 1]
    f8 = int((256 * (tf - a) / (b - a)).__floor__())
    return lo, f8


def test_sr_every_random_byte_exact(oracle):
    rng = np.random.default_rng(11)
    vals = list(rng.uniform(0, 6, size=600).astype(np.float32))
    vals += [float(g) for g in GRID[:-1]]
    # values whose fraction sits just around a multiple of 1/256 of the grid step
    for lo in range(7):
        a, b = float(GRID[lo]), float(GRID[lo + 1])
        for k in (1, 37, 128, 255):
            v = np.float32(a + (b - a) * k / 256)
            vals += [v, np.nextafter(v, np.float32(0)), np.nextafter(v, np.float32(10))]
    vals = np.array(vals, dtype=np.float32)
    rho = np.tile(np.arange(256, dtype=np.uint8), len(vals))
    q = np.repeat(vals, 256)
    codes = oracle.e2m1_sr_array(q, rho).reshape(len(vals), 256)
    for i, v in enumerate(vals):
        lo, f8 = _sr_expected_up_count(v)
        expected = np.where(np.arange(256) < f8, lo + 1, lo)
        np.testing.assert_array_equal(codes[i], expected, err_msg=f"t={v!r}")
    # negative values: same magnitudes with the sign bit
    codes_neg = oracle.e2m1_sr_array(-q, rho).reshape(len(vals), 256)
    np.testing.assert_array_equal(codes_neg, codes | 8)


def test_sr_saturation_and_nan(oracle):
    for rho in (0, 128, 255):
        assert oracle.e2m1_sr(6.0, rho) == 7
        assert oracle.e2m1_sr(7.5, rho) == 7
        assert oracle.e2m1_sr(float("inf"), rho) == 7
        assert oracle.e2m1_sr(float("-inf"), rho) == 0xF
        assert oracle.e2m1_sr(float("nan"), rho) == 0x7
        assert oracle.e2m1_sr(-0.0, rho) == 0x8


def _torch_e4m3(v):
    return torch.tensor(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_every_code_vs_torch(oracle):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.tensor(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    ours = np.array([oracle.e4m3_decode(int(c)) for c in codes], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2
    np.testing.assert_array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert oracle.e4m3_decode(0x7E) == 448.0 and oracle.e4m3_decode(0x01) == 2.0**-9


def test_e4m3_encode_vs_torch_on_finite_range(oracle):
    finite = np.array([oracle.e4m3_decode(c) for c in range(0x7F)], dtype=np.float64)
    mids = (finite[:-1] + finite[1:]) / 2
    mids32 = mids.astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids)     # midpoints are exact in binary32
    up = np.nextafter(mids32, np.float32(np.inf))
    down = np.nextafter(mids32, np.float32(0))
    rng = np.random.default_rng(3)
    logu = np.exp2(rng.uniform(-16, np.log2(464.0), size=1_000_000)).astype(np.float32)
    unif = rng.uniform(0, 464, size=500_000).astype(np.float32)
    sub = rng.uniform(0, 2.0**-6, size=200_000).astype(np.float32)
    v = np.concatenate([finite.astype(np.float32), mids32, up, down, logu, unif, sub,
                        np.array([0.0, 448.0, 460.0, 464.0, 2.0**-10, 1.5 * 2.0**-9], np.float32)])
    v = v[v <= 464.0]
    np.testing.assert_array_equal(oracle.e4m3_encode_array(v), _torch_e4m3(v))


def test_e4m3_encode_saturates_and_nan(oracle):
    # Reading: "satfinite" -- beyond 448 (torch turns values above 464 into NaN) the scale clamps to 448.
    for v in (464.5, 500.0, 1e6, 3.0e38, float("inf")):
        assert oracle.e4m3_encode(v) == 0x7E
    assert oracle.e4m3_encode(float("nan")) == 0x7F
    for v in (-0.0, -1.0, -float("inf")):
        assert oracle.e4m3_encode(v) == 0x00


def test_e4m3_power_of_two_ladder(oracle):
    """448 * 2^-k: normal codes ((15-k) << 3) | 6 down to k = 14, then the subnormals 7, 3.5 -> 4 (tie to
    even), 1.75 -> 2, 0.875 -> 1, 0.4375 -> 0 (all in units of 2^-9)."""
    expected = {k: ((15 - k) << 3) | 6 for k in range(15)}
    expected.update({15: 0x07, 16: 0x04, 17: 0x02, 18: 0x01, 19: 0x00, 20: 0x00})
    for k, code in expected.items():
        assert oracle.e4m3_encode(448.0 * 2.0**-k) == code, k
