"""GPU parity of the grouped calls (nvfp4_amax_grouped, nvfp4_quantize_grouped) against the CPU oracle.

A group holds row-wise tensors of different shapes (including an empty one, a single block, ragged row counts and a
tensor large enough to need many workgroups), each with its own sign mask, Philox seed and offset.  The amax of every
tensor must equal the oracle's bit for bit, and its codes, scales and g must equal the oracle's quantization of that
tensor alone (the definition of a grouped call), for RN, SR, RHT+SR and four-over-six, per-tensor and per-row g.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import nvfp4_quantization_amd as Q
from nvfp4_quantization_amd import workloads as W

pytestmark = pytest.mark.gpu

SHAPES = [(64, 256), (0, 32), (1, 16), (37, 160), (300, 48), (1024, 4096), (5, 1024)]
METHODS = {"rn": (Q.ROUND_RN, O.MODE_RN), "sr": (Q.ROUND_SR, O.MODE_SR), "rht_sr": (Q.ROUND_RHT_SR, O.MODE_RHT_SR),
           "4o6": (Q.ROUND_4O6, None)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    Q.binding.lib()          # fails loudly if the HIP library is missing
    O.lib()


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def same_f32(a, b, what):
    a = np.asarray(a, np.float32).ravel()
    b = np.asarray(b, np.float32).ravel()
    assert a.shape == b.shape, what
    bad = np.flatnonzero((a.view(np.uint32) != b.view(np.uint32)) & ~(np.isnan(a) & np.isnan(b)))
    assert bad.size == 0, f"{what}: {bad.size} float mismatches, first at {bad[:5]}"


def same_u8(a, b, what):
    bad = np.argwhere(np.asarray(a) != np.asarray(b))
    assert np.asarray(a).shape == np.asarray(b).shape and bad.size == 0, f"{what}: {len(bad)} byte mismatches"


def make_group(shapes, seed0):
    xs = []
    for k, (r, c) in enumerate(shapes):
        if k % 3 == 0:
            xs.append(W.lognormal_gradients(r, c, seed=seed0 + k) if r else np.zeros((0, c), np.uint16))
        elif k % 3 == 1:
            xs.append(W.activation_outliers(r, c, seed=seed0 + k) if r else np.zeros((0, c), np.uint16))
        else:
            xs.append(W.heavy_tail_rows(r, c, seed=seed0 + k, frac_special=1e-3) if r else np.zeros((0, c), np.uint16))
    masks = [W.sign_mask(seed0, k) for k in range(len(shapes))]
    seeds = [0x1234_5678 + 977 * k for k in range(len(shapes))]
    offsets = [3 * k + 1 for k in range(len(shapes))]
    return xs, masks, seeds, offsets


def run_group(xs, masks, seeds, offsets, method, gmode):
    q_round, o_mode = METHODS[method]
    xd = [torch.from_numpy(x.view(np.int16)).cuda() for x in xs]
    use_rht = method == "rht_sr"
    amaxes = Q.nvfp4_amax_grouped(xd, gmode, use_rht, masks)
    outs = Q.nvfp4_quantize_grouped(xd, amaxes, q_round, gmode, masks, seeds, offsets)
    torch.cuda.synchronize()
    for k, x in enumerate(xs):
        what = f"{method} item {k} {x.shape}"
        oa = O.amax(x, O.ROWWISE, gmode, use_rht, masks[k])
        same_f32(amaxes[k].cpu().numpy(), oa, what + " amax")
        if method == "4o6":
            oc, os_, og, _ = O.quantize_4o6(x, oa, gmode)
        else:
            oc, os_, og = O.quantize_1x16(x, oa, o_mode, O.ROWWISE, gmode, masks[k], seeds[k], offsets[k])
        same_u8(outs[k].codes.cpu().numpy(), oc, what + " codes")
        same_u8(outs[k].scales.cpu().numpy(), os_, what + " scales")
        same_f32(outs[k].g.cpu().numpy(), og, what + " g")


@pytest.mark.parametrize("gmode", [0, 1])
@pytest.mark.parametrize("method", list(METHODS))
def test_grouped_matches_oracle_per_tensor(method, gmode):
    say("grouped", method, "per-row" if gmode else "per-tensor", SHAPES)
    xs, masks, seeds, offsets = make_group(SHAPES, seed0=700 + 10 * gmode)
    run_group(xs, masks, seeds, offsets, method, gmode)


@pytest.mark.parametrize("method", ["rht_sr", "4o6"])
def test_largest_group(method):
    """NVFP4_MAX_GROUP small tensors in one launch (the launch-bound case grouping is for)."""
    shapes = [(16 + (k % 5) * 7, 64 * (1 + k % 4)) for k in range(Q.MAX_GROUP)]
    say("grouped, largest group", method, len(shapes))
    xs, masks, seeds, offsets = make_group(shapes, seed0=900)
    run_group(xs, masks, seeds, offsets, method, 0)


def test_group_limit_and_empty_group():
    x = torch.zeros((16, 16), dtype=torch.int16, device="cuda")
    with pytest.raises(Q.NVFP4Error):
        Q.nvfp4_amax_grouped([x] * (Q.MAX_GROUP + 1))
    assert Q.nvfp4_amax_grouped([]) == []
