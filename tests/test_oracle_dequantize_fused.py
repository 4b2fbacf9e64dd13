"""Pins for the oracle's fused decode: the inverse RHT, the binary32 -> bf16 rounding and their composition with
the standard decode (CPU only).

The inverse transform is pinned to the Sylvester matrix written out from its definition (unit vectors give its
columns exactly), to exact round trips with the forward transform on inputs where no step rounds, and to the
binary64 product within the butterfly's error bound.  The bf16 rounding is pinned to torch's conversion (a
library routine) on stratified binary32 patterns.  The composition is pinned to the standard decode, to the
inverse transform applied block by block, and to the orthogonality of the transform: decoding a tensor that was
quantized with the rotation, through the inverse rotation, loses exactly as much as the rotated tensor lost.
"""
import numpy as np
import pytest
import torch

from nvfp4_quantization_amd import workloads as W


def _sylvester16():
    return np.array([[(-1) ** bin(i & j).count("1") for j in range(16)] for i in range(16)], dtype=np.float64)


def _signs(mask):
    return np.array([-1.0 if (mask >> i) & 1 else 1.0 for i in range(16)])


def torch_bf16(x):
    """torch's binary32 -> bf16 conversion (round to nearest even), with every NaN written as 0x7FC0."""
    x = np.asarray(x, dtype=np.float32)
    out = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    out[np.isnan(x)] = 0x7FC0
    return out


# ------------------------------------------------------------------------------------------ inverse RHT
def test_inverse_of_unit_vectors_is_signed_quarter_hadamard_column(oracle):
    """M^-1 = diag(s) H / 4: the image of e_j is column j of H / 4 with row i negated where bit i of the mask
    is set."""
    H = _sylvester16()
    for mask in (0, 0x0001, 0x8000, 0xA5C3, 0xFFFF):
        for j in range(16):
            e = np.zeros(16, np.float32)
            e[j] = 1.0
            want = (_signs(mask) * H[:, j] / 4).astype(np.float32)
            np.testing.assert_array_equal(oracle.rht16_inverse(e, mask), want)


def test_inverse_undoes_forward_exactly_when_nothing_rounds(oracle):
    """Integers of magnitude <= 1024: every sum of the forward and inverse butterflies is an exact multiple of
    1/4 below 2^15, so inverse(forward(v)) = v bit for bit, for every sign mask tried (a mask applied at the
    wrong end or with the wrong bit order fails this)."""
    rng = np.random.default_rng(21)
    for trial in range(400):
        v = rng.integers(-1024, 1025, size=16).astype(np.float32)
        mask = int(rng.integers(0, 1 << 16)) if trial else 0x0001
        np.testing.assert_array_equal(oracle.rht16_inverse(oracle.rht16(v, mask), mask), v)
    # a mismatched mask does not invert
    v = np.arange(1, 17, dtype=np.float32)
    assert not np.array_equal(oracle.rht16_inverse(oracle.rht16(v, 0x0003), 0x0001), v)


def test_inverse_matches_dense_definition_within_rounding(oracle):
    """diag(s) H y / 4 in binary64 against the binary32 evaluation: four roundings in the butterfly,
    |z32 - z64| <= 4 * 2^-24 * (1/4) * sum|y| (times a hair)."""
    H = _sylvester16()
    rng = np.random.default_rng(22)
    for trial in range(2000):
        y = (rng.standard_normal(16) * np.exp(3 * rng.standard_normal(16))).astype(np.float32)
        mask = int(rng.integers(0, 1 << 16))
        exact = _signs(mask) * (H @ y.astype(np.float64)) / 4
        got = oracle.rht16_inverse(y, mask).astype(np.float64)
        bound = 4 * 2.0**-24 * np.abs(y.astype(np.float64)).sum() / 4 * 1.0001
        assert np.all(np.abs(got - exact) <= bound), trial


def test_inverse_propagates_nan_and_inf(oracle):
    y = np.ones(16, np.float32)
    y[3] = np.nan
    assert np.all(np.isnan(oracle.rht16_inverse(y, 0x00FF)))
    y[3] = np.inf
    assert np.all(np.isinf(oracle.rht16_inverse(y, 0)))


# ------------------------------------------------------------------------------------------ bf16 rounding
def _stratified_patterns(rng):
    """Every sign and exponent, with the dropped 16 bits at and around the rounding boundaries, over random kept
    mantissas; plus uniformly random patterns."""
    low = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], dtype=np.uint32)
    hi = np.arange(512, dtype=np.uint32) << 23                       # sign and exponent
    kept = rng.integers(0, 1 << 7, size=64, dtype=np.uint32) << 16    # random kept mantissa bits
    kept = np.concatenate([kept, np.array([0, 1 << 16, 0x7F << 16], dtype=np.uint32)])
    pats = (hi[:, None, None] | kept[None, :, None] | low[None, None, :]).ravel()
    return np.concatenate([pats, rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)])


def test_bf16_rounding_matches_torch(oracle):
    """Non-NaN patterns against torch.  (torch's own NaN results differ between its scalar path, 0x7FC0, and its
    vectorised CPU path, 0xFFFF; the oracle's NaN rule is checked on its own below.)"""
    rng = np.random.default_rng(23)
    pats = _stratified_patterns(rng)
    x = pats.view(np.float32)
    got = np.array([oracle.f32_to_bf16(v) for v in x], dtype=np.uint16)
    nan = np.isnan(x)
    assert np.all(got[nan] == 0x7FC0)
    want = torch_bf16(x[~nan])
    got, pats = got[~nan], pats[~nan]
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(pats[i]), hex(got[i]), hex(want[i])) for i in bad[:8]]


def test_bf16_rounding_special_values(oracle):
    assert oracle.f32_to_bf16(0.0) == 0x0000 and oracle.f32_to_bf16(-0.0) == 0x8000
    assert oracle.f32_to_bf16(np.inf) == 0x7F80 and oracle.f32_to_bf16(-np.inf) == 0xFF80
    assert oracle.f32_to_bf16(np.nan) == 0x7FC0
    assert oracle.f32_to_bf16(np.array([0xFFC00001], np.uint32).view(np.float32)[0]) == 0x7FC0
    assert oracle.f32_to_bf16(1.0 + 2.0**-8) == 0x3F80        # tie, kept pattern even: stays
    assert oracle.f32_to_bf16(1.0 + 3 * 2.0**-8) == 0x3F82    # tie, kept pattern odd: rounds up
    fmax = np.finfo(np.float32).max
    assert oracle.f32_to_bf16(fmax) == 0x7F80                 # beyond the largest bf16 plus half an ulp


# ------------------------------------------------------------------------------------------ fused decode
def _quantized(oracle, rows=64, cols=256, seed=24, mode=None, mask=0):
    x = W.lognormal_gradients(rows, cols, seed=seed)
    mode = oracle.MODE_RN if mode is None else mode
    a = oracle.amax(x, use_rht=mode == oracle.MODE_RHT_SR, sign_mask=mask)
    codes, scales, g = oracle.quantize_1x16(x, a, mode, sign_mask=mask, seed=5, offset=1)
    return x, codes, scales, g


def test_fused_without_rht_equals_standard_decode(oracle):
    _, codes, scales, g = _quantized(oracle)
    y = oracle.dequantize(codes, scales, g)
    z = oracle.dequantize_fused(codes, scales, g)
    np.testing.assert_array_equal(z.view(np.uint32), y.view(np.uint32))


@pytest.mark.parametrize("use_rht", [False, True])
def test_fused_bf16_output_is_torch_rounding_of_float_output(oracle, use_rht):
    _, codes, scales, g = _quantized(oracle, mode=oracle.MODE_RHT_SR, mask=0x6A91)
    z32 = oracle.dequantize_fused(codes, scales, g, use_rht=use_rht, sign_mask=0x6A91)
    z16 = oracle.dequantize_fused(codes, scales, g, use_rht=use_rht, sign_mask=0x6A91, out_bf16=True)
    np.testing.assert_array_equal(z16, torch_bf16(z32))


def test_fused_rht_is_blockwise_inverse_of_decode(oracle):
    _, codes, scales, g = _quantized(oracle, rows=8, cols=64, mode=oracle.MODE_RHT_SR, mask=0x1357)
    y = oracle.dequantize(codes, scales, g)
    z = oracle.dequantize_fused(codes, scales, g, use_rht=True, sign_mask=0x1357)
    for r in range(y.shape[0]):
        for b in range(y.shape[1] // 16):
            want = oracle.rht16_inverse(y[r, 16 * b:16 * b + 16], 0x1357)
            np.testing.assert_array_equal(z[r, 16 * b:16 * b + 16].view(np.uint32), want.view(np.uint32))


def test_fused_rht_error_equals_rotated_error(oracle):
    """The transform is orthonormal, so per block ||x - xhat||_2 = ||rht(x) - dequant(q)||_2, where xhat is the
    fused decode with the inverse transform (up to binary32 rounding of the two butterflies)."""
    mask = 0xC3A5
    x, codes, scales, g = _quantized(oracle, rows=32, cols=128, mode=oracle.MODE_RHT_SR, mask=mask)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    y = oracle.dequantize(codes, scales, g).astype(np.float64)
    z = oracle.dequantize_fused(codes, scales, g, use_rht=True, sign_mask=mask).astype(np.float64)
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // 16):
            sl = slice(16 * b, 16 * b + 16)
            ry = oracle.rht16(x[r, sl].astype(np.uint32).__lshift__(16).view(np.float32), mask).astype(np.float64)
            e_rot = np.linalg.norm(ry - y[r, sl])
            e_back = np.linalg.norm(xf[r, sl] - z[r, sl])
            scale = np.abs(xf[r, sl]).sum() + np.abs(y[r, sl]).sum()
            assert abs(e_rot - e_back) <= 1e-6 * scale, (r, b, e_rot, e_back)
    # a wrong mask on the way back loses far more
    zw = oracle.dequantize_fused(codes, scales, g, use_rht=True, sign_mask=mask ^ 0x0F0F).astype(np.float64)
    assert np.linalg.norm(xf - zw) > 3 * np.linalg.norm(xf - z)


def test_fused_per_row_g_and_nan(oracle):
    x = W.activation_outliers(16, 64, seed=25)
    x[3, 7] = 0x7FC0                                       # a NaN: row 3 decodes to NaN everywhere
    a = oracle.amax(x, gmode=oracle.G_PER_ROW)
    codes, scales, g = oracle.quantize_1x16(x, a, oracle.MODE_RN, gmode=oracle.G_PER_ROW)
    y = oracle.dequantize(codes, scales, g, gmode=oracle.G_PER_ROW)
    z = oracle.dequantize_fused(codes, scales, g, gmode=oracle.G_PER_ROW, out_bf16=True)
    np.testing.assert_array_equal(z, torch_bf16(y))
    assert np.all(z[3] == 0x7FC0) and not np.any(z[np.arange(16) != 3] == 0x7FC0)
