"""GPU parity of the four-over-six error modes and bounds (pytorch/ao #4852, PR body: the sweep over err_mode and
bound) for 1x16 blocks: bf16 and binary32 inputs, per-tensor and per-row g, and the grouped call, against the CPU
oracle bit for bit (codes, scales, g).  The inputs hold blocks where the modes choose differently, so a kernel that
measured with the wrong mode, or took g from the wrong bound, fails."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import nvfp4_quantization_amd as Q
from nvfp4_quantization_amd import workloads as W

pytestmark = pytest.mark.gpu

MODES = [Q.ERR_MSE, Q.ERR_MAE, Q.ERR_MAXABS]
BOUNDS = [Q.BOUND_STD, Q.BOUND_HEADROOM, 1, 101]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    Q.binding.lib()
    O.lib()


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def same_f32(a, b, what):
    a, b = np.asarray(a, np.float32).ravel(), np.asarray(b, np.float32).ravel()
    ok = (a.view(np.uint32) == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b))
    assert ok.all(), f"{what}: {np.count_nonzero(~ok)} mismatches, first {np.flatnonzero(~ok)[:4]}"


def same_u8(a, b, what):
    bad = np.argwhere(np.asarray(a) != np.asarray(b))
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first {bad[:4].tolist()}"


def bf16_input(rows, cols, seed, special=True):
    """Heavy-tailed rows; with special, a few NaN/inf (which make a per-tensor g NaN or inf, so per-tensor cases
    that must show the modes disagreeing take none)."""
    return W.heavy_tail_rows(rows, cols, seed=seed, frac_special=3e-4 if special else 0.0)


def f32_input(rows, cols, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-4, 4, (rows, 1)))).astype(np.float32)
    x[:, ::7] *= np.float32(3.3)
    if rows > 4:
        x[1, 5] = np.nan
        x[2, 9] = -np.inf
        x[3, :] = 0.0
    return x


@pytest.mark.parametrize("bound", BOUNDS)
@pytest.mark.parametrize("err_mode", MODES)
@pytest.mark.parametrize("gmode", [0, 1])
def test_bf16(gmode, err_mode, bound):
    x = bf16_input(272, 1040, seed=17 + gmode, special=gmode == 1)
    say("4o6 knobs bf16", gmode, err_mode, bound, x.shape)
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    a = Q.nvfp4_amax(xd, Q.ROWWISE, gmode)
    out = Q.nvfp4_quantize_4o6(xd, a, gmode, err_mode=err_mode, bound=bound)
    torch.cuda.synchronize()
    oa = O.amax(x, O.ROWWISE, gmode)
    same_f32(a.cpu().numpy(), oa, "amax")
    oc, os_, og, choice = O.quantize_4o6(x, oa, gmode, err_mode=err_mode, bound=bound)
    same_u8(out.codes.cpu().numpy(), oc, "codes")
    same_u8(out.scales.cpu().numpy(), os_, "scales")
    same_f32(out.g.cpu().numpy(), og, "g")
    other = O.quantize_4o6(x, oa, gmode, err_mode=(err_mode + 1) % 3, bound=bound)[3]
    assert choice.any() and (choice != other).any()


@pytest.mark.parametrize("err_mode", MODES)
@pytest.mark.parametrize("gmode", [0, 1])
def test_f32(gmode, err_mode):
    x = f32_input(300, 4112, seed=23 + gmode)
    say("4o6 knobs f32", gmode, err_mode, x.shape)
    xd = torch.from_numpy(x).cuda()
    a = Q.nvfp4_amax_f32(xd, gmode)
    out = Q.nvfp4_quantize_4o6_f32(xd, a, gmode, err_mode=err_mode, bound=Q.BOUND_HEADROOM)
    torch.cuda.synchronize()
    oa = O.amax_f32(x, gmode)
    oc, os_, og, _ = O.quantize_4o6_f32(x, oa, gmode, err_mode=err_mode, bound=Q.BOUND_HEADROOM)
    same_u8(out.codes.cpu().numpy(), oc, "codes")
    same_u8(out.scales.cpu().numpy(), os_, "scales")
    same_f32(out.g.cpu().numpy(), og, "g")


@pytest.mark.parametrize("gmode", [0, 1])
def test_empty_writes_g_of_the_bound(gmode):
    a = torch.tensor([7.0] if gmode == 0 else [], device="cuda")
    out = Q.nvfp4_quantize_4o6(torch.empty((0, 32), dtype=torch.int16, device="cuda"), a, gmode,
                               err_mode=Q.ERR_MAXABS, bound=Q.BOUND_HEADROOM)
    torch.cuda.synchronize()
    if gmode == 0:
        og = O.quantize_4o6(np.zeros((1, 16), np.uint16), np.array([7.0], np.float32), 0,
                            bound=Q.BOUND_HEADROOM)[2]
        same_f32(out.g.cpu().numpy(), og, "g")


@pytest.mark.parametrize("err_mode", [Q.ERR_MAE, Q.ERR_MAXABS])
@pytest.mark.parametrize("gmode", [0, 1])
def test_grouped(gmode, err_mode):
    shapes = [(64, 256), (33, 48), (300, 1040), (1, 16), (0, 32)]
    xs = [bf16_input(r, c, seed=40 + k) if r else np.zeros((0, c), np.uint16) for k, (r, c) in enumerate(shapes)]
    say("4o6 knobs grouped", gmode, err_mode, shapes)
    xd = [torch.from_numpy(x.view(np.int16)).cuda() for x in xs]
    amaxes = Q.nvfp4_amax_grouped(xd, gmode)
    outs = Q.nvfp4_quantize_grouped(xd, amaxes, Q.ROUND_4O6, gmode, err_mode=err_mode, bound=Q.BOUND_HEADROOM)
    torch.cuda.synchronize()
    for k, x in enumerate(xs):
        oa = O.amax(x, O.ROWWISE, gmode)
        if x.shape[0] == 0:
            if gmode == 0:
                og = O.quantize_4o6(np.zeros((1, 16), np.uint16), oa, 0, bound=Q.BOUND_HEADROOM)[2]
                same_f32(outs[k].g.cpu().numpy(), og, f"item {k} g")
            continue
        oc, os_, og, _ = O.quantize_4o6(x, oa, gmode, err_mode=err_mode, bound=Q.BOUND_HEADROOM)
        same_u8(outs[k].codes.cpu().numpy(), oc, f"item {k} codes")
        same_u8(outs[k].scales.cpu().numpy(), os_, f"item {k} scales")
        same_f32(outs[k].g.cpu().numpy(), og, f"item {k} g")


@pytest.mark.slow
@pytest.mark.parametrize("err_mode", [Q.ERR_MAE, Q.ERR_MAXABS])
def test_full_16384x8192(err_mode):
    """The four-over-six workload (per-row g) under the other error modes and the headroom bound, in full."""
    x = W.make("four_over_six_16384x8192")
    say("4o6 knobs full", err_mode, x.shape)
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    a = Q.nvfp4_amax(xd, Q.ROWWISE, Q.G_PER_ROW)
    out = Q.nvfp4_quantize_4o6(xd, a, Q.G_PER_ROW, err_mode=err_mode, bound=Q.BOUND_HEADROOM)
    torch.cuda.synchronize()
    oa = O.amax(x, O.ROWWISE, O.G_PER_ROW)
    oc, os_, og, _ = O.quantize_4o6(x, oa, O.G_PER_ROW, err_mode=err_mode, bound=Q.BOUND_HEADROOM)
    same_u8(out.codes.cpu().numpy(), oc, "codes")
    same_u8(out.scales.cpu().numpy(), os_, "scales")
    same_f32(out.g.cpu().numpy(), og, "g")
