"""GPU parity of the binary32-input four-over-six (nvfp4_amax_f32, nvfp4_quantize_4o6_f32) against the CPU oracle.

Inputs have full 24-bit mantissas (not bf16-representable), per-row and per-tensor g, ragged block counts per
workgroup, NaN / inf rows, zeros and subnormals, and the 16384 x 8192 four-over-six shape.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import nvfp4_quantization_amd as Q

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    Q.binding.lib()
    O.lib()


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def make(rows, cols, seed, special=False):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-4, 4, (rows, 1)))).astype(np.float32)
    x[:, ::5] *= np.float32(2.7)
    if special and rows >= 8:
        x[1, 3] = np.nan
        x[2, 7] = np.inf
        x[3, :] = 0.0
        x[4, :16] = np.float32(1e-42)           # subnormal block
        x[5, 20] = -np.inf
    return x


def check(x, gmode):
    xd = torch.from_numpy(x).cuda()
    a = Q.nvfp4_amax_f32(xd, gmode)
    out = Q.nvfp4_quantize_4o6_f32(xd, a, gmode)
    torch.cuda.synchronize()
    oa = O.amax_f32(x, gmode)
    ga = a.cpu().numpy()
    assert ((ga.view(np.uint32) == oa.view(np.uint32)) | (np.isnan(ga) & np.isnan(oa))).all(), "amax"
    oc, os_, og, _ = O.quantize_4o6_f32(x, oa, gmode)
    bad = np.argwhere(out.codes.cpu().numpy() != oc)
    assert bad.size == 0, f"codes: {len(bad)} mismatches, first {bad[:4].tolist()}"
    assert np.array_equal(out.scales.cpu().numpy(), os_), "scales"
    g = out.g.cpu().numpy()
    assert ((g.view(np.uint32) == og.view(np.uint32)) | (np.isnan(g) & np.isnan(og))).all(), "g"


@pytest.mark.parametrize("gmode", [0, 1])
@pytest.mark.parametrize("shape", [(1, 16), (37, 160), (256, 1024), (300, 4112), (1025, 512)])
def test_4o6_f32(gmode, shape):
    say("4o6 f32", gmode, shape)
    check(make(*shape, seed=shape[0] + 7 * shape[1], special=True), gmode)


def test_4o6_f32_empty():
    out = Q.nvfp4_quantize_4o6_f32(torch.empty((0, 32), device="cuda"), torch.tensor([3.0], device="cuda"), 0)
    torch.cuda.synchronize()
    assert out.g.cpu().numpy()[0] == O.global_scale(3.0)


@pytest.mark.slow
def test_4o6_f32_16384x8192():
    x = make(16384, 8192, seed=4)
    say("4o6 f32 full", x.shape)
    check(x, 1)


def check_16x16(x, amax=None, orient=Q.BOTH, err_mode=Q.ERR_MSE, bound=Q.BOUND_STD):
    xd = torch.from_numpy(x).cuda()
    a = Q.nvfp4_amax_f32(xd, 0) if amax is None else torch.from_numpy(amax).cuda()
    row, col = Q.nvfp4_quantize_4o6_16x16_f32(xd, a, orient, err_mode, bound)
    torch.cuda.synchronize()
    oa = O.amax_f32(x, 0) if amax is None else amax
    (cw, sw, gw), (ct, st, gt), _ = O.quantize_4o6_16x16_f32(x, oa, err_mode=err_mode, bound=bound)
    for out, codes, scales, gg, what in ((row, cw, sw, gw, "W"), (col, ct, st, gt, "W^T")):
        if out is None:
            continue
        bad = np.argwhere(out.codes.cpu().numpy() != codes)
        assert bad.size == 0, f"{what} codes: {len(bad)} mismatches, first {bad[:4].tolist()}"
        assert np.array_equal(out.scales.cpu().numpy(), scales), what + " scales"
        g = out.g.cpu().numpy()
        assert g.view(np.uint32)[0] == gg.view(np.uint32)[0] or (np.isnan(g[0]) and np.isnan(gg[0]))


@pytest.mark.parametrize("shape", [(16, 16), (48, 1040), (256, 4096), (80, 2064)])
def test_4o6_16x16_f32(shape):
    say("4o6 16x16 f32", shape)
    check_16x16(make(*shape, seed=3 * shape[0] + shape[1], special=False))


def test_4o6_16x16_f32_special_values():
    say("4o6 16x16 f32 special values")
    x = make(64, 96, seed=9, special=True)
    for amax in (None, np.array([0.0], np.float32), np.array([np.inf], np.float32), np.array([3.5], np.float32)):
        check_16x16(x, amax)


@pytest.mark.parametrize("err_mode", [Q.ERR_MAE, Q.ERR_MAXABS])
@pytest.mark.parametrize("orient", [Q.ROWWISE, Q.COLWISE])
def test_4o6_16x16_f32_knobs(orient, err_mode):
    say("4o6 16x16 f32 knobs", orient, err_mode)
    check_16x16(make(80, 2064, seed=31, special=True), orient=orient, err_mode=err_mode, bound=Q.BOUND_HEADROOM)


@pytest.mark.slow
def test_4o6_16x16_f32_14336x4096():
    x = make(14336, 4096, seed=6)
    say("4o6 16x16 f32 full", x.shape)
    check_16x16(x)
