"""GPU parity of the fused decode (nvfp4_dequantize_fused) against the CPU oracle.

Every input comes from the oracle's own quantization of a seeded workload, or from seeded random bytes; both sides
decode the same arrays.  Bar: float output bit-exact (NaN equal to NaN), bf16 output bit-exact.  Shapes span
several workgroups and ragged tails; the full-size case decodes the 8192x4096 weight-gradient quantization
(column-wise RHT + SR) back through the inverse transform, in the launch configuration the benchmark times.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import nvfp4_quantization_amd as Q
from nvfp4_quantization_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    Q.binding.lib()          # fails loudly if the HIP library is missing
    O.lib()


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def d(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_decode(codes, scales, g, gmode, use_rht, mask, out_bf16):
    y = Q.nvfp4_dequantize_fused(d(codes), d(scales), d(g), gmode, use_rht, mask, out_bf16)
    torch.cuda.synchronize()
    y = y.cpu()
    return y.view(torch.int16).numpy().view(np.uint16) if out_bf16 else y.numpy()


def compare(codes, scales, g, gmode, use_rht, mask, out_bf16):
    got = gpu_decode(codes, scales, g, gmode, use_rht, mask, out_bf16)
    want = O.dequantize_fused(codes, scales, g, gmode, use_rht, mask, out_bf16)
    assert got.shape == want.shape
    if out_bf16:
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{len(bad)} bf16 mismatches, first {bad[:4].tolist()}: " \
                              f"{got[tuple(bad[0])]:#06x} vs {want[tuple(bad[0])]:#06x}"
    else:
        both_nan = np.isnan(got) & np.isnan(want)
        bad = np.argwhere((got.view(np.uint32) != want.view(np.uint32)) & ~both_nan)
        assert bad.size == 0, f"{len(bad)} float mismatches, first {bad[:4].tolist()}"
    return got


def oracle_quantized(x, mode, orient, gmode, mask, seed=11, offset=3):
    a = O.amax(x, orient, gmode, mode == O.MODE_RHT_SR, mask)
    return O.quantize_1x16(x, a, mode, orient, gmode, mask, seed, offset)


SHAPES = [(64, 256), (37, 160), (1, 16), (300, 48), (129, 4096)]


@pytest.mark.parametrize("out_bf16", [True, False])
@pytest.mark.parametrize("gmode", [0, 1])
@pytest.mark.parametrize("shape", SHAPES)
def test_rht_sr_round_trip_rowwise(shape, gmode, out_bf16):
    mask = W.sign_mask(shape[0], shape[1])
    say("fused decode, row-wise RHT+SR", shape, "per-row" if gmode else "per-tensor", "bf16" if out_bf16 else "f32")
    x = W.lognormal_gradients(*shape, seed=shape[0] * 17 + shape[1])
    codes, scales, g = oracle_quantized(x, O.MODE_RHT_SR, O.ROWWISE, gmode, mask)
    compare(codes, scales, g, gmode, True, mask, out_bf16)


@pytest.mark.parametrize("out_bf16", [True, False])
@pytest.mark.parametrize("shape", [(512, 200), (48, 8), (1040, 72)])
def test_rht_sr_round_trip_colwise(shape, out_bf16):
    mask = W.sign_mask(shape[1], shape[0])
    say("fused decode, column-wise RHT+SR", shape, "bf16" if out_bf16 else "f32")
    x = W.outlier_columns(*shape, seed=shape[0] + 3 * shape[1], n_cols=min(4, shape[1]))
    codes, scales, g = oracle_quantized(x, O.MODE_RHT_SR, O.COLWISE, 0, mask)
    compare(codes, scales, g, 0, True, mask, out_bf16)


@pytest.mark.parametrize("out_bf16", [True, False])
@pytest.mark.parametrize("gmode", [0, 1])
def test_plain_decode_of_rn_and_4o6(gmode, out_bf16):
    say("fused decode without RHT", gmode, out_bf16)
    x = W.activation_outliers(96, 512, seed=31)
    codes, scales, g = oracle_quantized(x, O.MODE_RN, O.ROWWISE, gmode, 0)
    compare(codes, scales, g, gmode, False, 0, out_bf16)
    x = W.heavy_tail_rows(64, 256, seed=32, frac_special=2e-3)
    a = O.amax(x, O.ROWWISE, gmode)
    codes, scales, g, _ = O.quantize_4o6(x, a, gmode)
    got = compare(codes, scales, g, gmode, False, 0, out_bf16)
    if out_bf16:   # rows holding an injected NaN or infinity decode to the canonical NaN everywhere
        assert np.any(np.all(got == 0x7FC0, axis=1))


@pytest.mark.parametrize("out_bf16", [True, False])
@pytest.mark.parametrize("use_rht", [False, True])
@pytest.mark.parametrize("gmode", [0, 1])
def test_arbitrary_bytes_and_special_scales(gmode, use_rht, out_bf16):
    """Every E4M3 scale code (sign bit and NaN patterns included), random code bytes, and global scales that are
    zero, tiny, huge, infinite or NaN."""
    say("fused decode, arbitrary bytes", gmode, use_rht, out_bf16)
    rng = np.random.default_rng(1000 + 4 * gmode + 2 * use_rht + out_bf16)
    rv = 96
    codes = rng.integers(0, 256, size=(rv, 64), dtype=np.uint8)
    scales = np.resize(np.arange(256, dtype=np.uint8), (rv, 8))
    if gmode:
        g = rng.uniform(0.25, 4.0, size=rv).astype(np.float32)
        g[:8] = [0.0, -0.0, 1e-38, 3e38, np.inf, -np.inf, np.nan, 2.0 ** -140]
    else:
        g = np.array([0.37], np.float32)
    compare(codes, scales, g, gmode, use_rht, 0xB4E1, out_bf16)


def test_bf16_ties_and_overflow():
    """Decoded sums that land exactly halfway between two bf16 values round to the even one; values past the
    largest bf16 go to infinity.  g = 2^-7 with scale 1.0 makes every decoded value a multiple of 2^-8, so the
    inverse transform's quarter-sums hit ties of the 8-bit bf16 significand often."""
    rng = np.random.default_rng(77)
    codes = rng.integers(0, 256, size=(256, 64), dtype=np.uint8)
    scales = np.full((256, 8), 0x38, np.uint8)                 # E4M3 1.0
    scales[::7] = 0x7E                                         # 448
    g = np.array([2.0 ** -7], np.float32)
    for use_rht in (False, True):
        compare(codes, scales, g, 0, use_rht, 0x0F0F, True)
    compare(codes, np.full((256, 8), 0x7E, np.uint8), np.array([3.3e38], np.float32), 0, False, 0, True)


def test_empty():
    y = Q.nvfp4_dequantize_fused(torch.empty((0, 8), dtype=torch.uint8, device="cuda"),
                                 torch.empty((0, 1), dtype=torch.uint8, device="cuda"),
                                 torch.ones((1,), device="cuda"), 0, True, 0x1, True)
    torch.cuda.synchronize()
    assert y.shape == (0, 16) and y.dtype == torch.bfloat16


@pytest.mark.slow
def test_full_wgrad_decode_through_inverse_rht():
    """The 8192x4096 weight-gradient workload, quantized column-wise with RHT + SR by the oracle, decoded through
    the inverse transform to bf16 (and to float) in full."""
    x = W.make("wgrad_colwise_rht_sr_8192x4096")
    mask = W.sign_mask(2, 0)
    say("full wgrad decode", x.shape, hex(mask))
    codes, scales, g = oracle_quantized(x, O.MODE_RHT_SR, O.COLWISE, 0, mask, seed=2, offset=0)
    compare(codes, scales, g, 0, True, mask, True)
    compare(codes, scales, g, 0, True, mask, False)
