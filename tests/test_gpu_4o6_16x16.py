"""GPU parity of four-over-six with 16x16 tiles (nvfp4_quantize_4o6_16x16) against the CPU oracle.

Codes, scales and g must equal the oracle's W and W^T outputs bit for bit, in each orientation alone and both from
one read, under every error mode and several bounds.  Inputs mix tiles where map-to-4 wins and tiles where map-to-6
wins, ragged tile counts per workgroup, special values (NaN, infinities, zeros) and the full 14336x4096 weight
workload of the 16x16 pass.
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


def bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def mixed_tiles(rows, cols, seed):
    """Tiles alternating uniform values (map-to-4 usually wins) and Gaussian ones, scaled by per-tile powers of 2."""
    rng = np.random.default_rng(seed)
    x = np.zeros((rows, cols), np.float32)
    for ti in range(rows // 16):
        for tj in range(cols // 16):
            t = rng.uniform(-1, 1, (16, 16)) if (ti + tj) % 2 else rng.normal(0, 1, (16, 16))
            x[16 * ti:16 * ti + 16, 16 * tj:16 * tj + 16] = t * 2.0 ** -((3 * ti + tj) % 7)
    return bits(x)


def same(out, codes, scales, g, what):
    c, s_, gg = out.codes.cpu().numpy(), out.scales.cpu().numpy(), out.g.cpu().numpy()
    bad = np.argwhere(c != codes)
    assert bad.size == 0, f"{what}: {len(bad)} code byte mismatches, first {bad[:4].tolist()}"
    bad = np.argwhere(s_ != scales)
    assert bad.size == 0, f"{what}: {len(bad)} scale mismatches, first {bad[:4].tolist()}"
    assert gg.view(np.uint32)[0] == g.view(np.uint32)[0] or (np.isnan(gg[0]) and np.isnan(g[0])), what


def check(x, amax=None, expect_both=False, orient=Q.BOTH, err_mode=Q.ERR_MSE, bound=Q.BOUND_STD):
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    a = Q.nvfp4_amax(xd, Q.ROWWISE, Q.G_PER_TENSOR) if amax is None else torch.from_numpy(amax).cuda()
    row, col = Q.nvfp4_quantize_4o6_16x16(xd, a, orient, err_mode, bound)
    torch.cuda.synchronize()
    oa = O.amax(x) if amax is None else amax
    np.testing.assert_array_equal(a.cpu().numpy().view(np.uint32), oa.view(np.uint32))
    (cw, sw, gw), (ct, st, gt), choice = O.quantize_4o6_16x16(x, oa, err_mode=err_mode, bound=bound)
    assert (row is not None) == (orient != Q.COLWISE) and (col is not None) == (orient != Q.ROWWISE)
    if row is not None:
        same(row, cw, sw, gw, "W")
    if col is not None:
        same(col, ct, st, gt, "W^T")
    if expect_both:
        assert choice.any() and not choice.all()
    return choice


@pytest.mark.parametrize("orient", [Q.ROWWISE, Q.COLWISE, Q.BOTH])
@pytest.mark.parametrize("shape", [(16, 16), (32, 64), (48, 1040), (256, 4096), (80, 2064), (1040, 48)])
def test_mixed_tiles(shape, orient):
    say("4o6 16x16 mixed", shape, orient)
    check(mixed_tiles(*shape, seed=shape[0] + shape[1]), expect_both=shape[0] * shape[1] >= 2048, orient=orient)


@pytest.mark.parametrize("bound", [Q.BOUND_STD, Q.BOUND_HEADROOM, 37])
@pytest.mark.parametrize("err_mode", [Q.ERR_MSE, Q.ERR_MAE, Q.ERR_MAXABS])
def test_error_modes_and_bounds(err_mode, bound):
    """Every error measure and bound, both orientations; the modes must actually disagree on some tiles here."""
    x = mixed_tiles(96, 1040, seed=11)
    say("4o6 16x16 knobs", err_mode, bound)
    choice = check(x, expect_both=True, err_mode=err_mode, bound=bound)
    other = O.quantize_4o6_16x16(x, O.amax(x), err_mode=(err_mode + 1) % 3, bound=bound)[2]
    assert (choice != other).any()


@pytest.mark.parametrize("shape", [(64, 128), (144, 4096)])
def test_weight_distribution(shape):
    say("4o6 16x16 weight", shape)
    check(W.weight_outliers(*shape, seed=shape[0] * 3 + shape[1]))


def test_special_values():
    say("4o6 16x16 special values")
    x = mixed_tiles(64, 96, seed=5)
    x[3, 7] = 0x7FC0                 # NaN in tile (0, 0)
    x[20, 40] = 0x7F80               # +inf in tile (1, 2)
    x[40, 70] = 0xFF80               # -inf in tile (2, 4)
    x[48:64, 80:96] = 0              # an all-zero tile
    x[32:48, 16:32] = 0x8000         # a tile of negative zeros
    for amax in (np.array([3.5], np.float32), np.array([0.0], np.float32), np.array([np.inf], np.float32),
                 np.array([np.nan], np.float32), np.array([1e-30], np.float32)):
        for err_mode in (Q.ERR_MSE, Q.ERR_MAE, Q.ERR_MAXABS):
            check(x, amax, err_mode=err_mode, bound=Q.BOUND_HEADROOM if err_mode else Q.BOUND_STD)
    check(x)                          # the tensor's own amax (NaN)


def test_empty():
    xd = torch.empty((0, 32), dtype=torch.int16, device="cuda")
    a = torch.tensor([7.0], device="cuda")
    row, col = Q.nvfp4_quantize_4o6_16x16(xd, a, Q.BOTH)
    torch.cuda.synchronize()
    assert row.codes.shape == (0, 16) and row.g.cpu().numpy()[0] == O.global_scale(7.0)
    assert col.codes.shape == (32, 0) and col.g.cpu().numpy()[0] == O.global_scale(7.0)
    # g = amax / (6 bound) for another bound, also when nothing is quantized
    row, col = Q.nvfp4_quantize_4o6_16x16(xd, a, Q.BOTH, Q.ERR_MAE, Q.BOUND_HEADROOM)
    torch.cuda.synchronize()
    g256 = O.quantize_4o6_16x16(np.zeros((16, 32), np.uint16), np.array([7.0], np.float32),
                                bound=Q.BOUND_HEADROOM)[0][2][0]
    assert row.g.cpu().numpy()[0] == g256 and col.g.cpu().numpy()[0] == g256


@pytest.mark.slow
def test_full_weight_14336x4096():
    """W and W^T from one read, in the launch configuration the benchmark times."""
    x = W.make("weight_16x16_14336x4096")
    say("4o6 16x16 full weight", x.shape)
    check(x, orient=Q.BOTH)
