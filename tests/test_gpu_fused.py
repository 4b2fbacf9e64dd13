"""GPU parity of nvfp4_amax_quantize (amax and 1x16 quantization in one call) against the CPU oracle.

Tensors that fit the chip in one wave of workgroups take the single-read kernels (the tile stays in registers while
the workgroups exchange their maxima): column-wise up to one 256 x 512 tile per CU, row-wise up to 8192 blocks per
CU.  Larger ones take the two-pass path.  Bar: amax, g, codes and scales bit-exact, as for the separate calls.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import nvfp4_quantization_amd as Q
from nvfp4_quantization_amd import workloads as W

pytestmark = pytest.mark.gpu

ROUNDING = {"rn": (Q.ROUND_RN, O.MODE_RN), "sr": (Q.ROUND_SR, O.MODE_SR), "rht_sr": (Q.ROUND_RHT_SR, O.MODE_RHT_SR)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    Q.binding.lib()
    O.lib()


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def check(x, mode, orient, mask=0x5A3C, seed=0xDEAD_BEEF_0123, offset=3, out=None, amax=None):
    say("amax_quantize", mode, "row" if orient == Q.ROWWISE else "col", x.shape, hex(mask), offset)
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    a, o = Q.nvfp4_amax_quantize(xd, orient, ROUNDING[mode][0], mask, seed, offset, amax=amax, out=out)
    torch.cuda.synchronize()
    oa = O.amax(x, orient, O.G_PER_TENSOR, mode == "rht_sr", mask)
    oc, os_, og = O.quantize_1x16(x, oa, ROUNDING[mode][1], orient, O.G_PER_TENSOR, mask, seed, offset)
    ga = a.cpu().numpy()
    assert (ga.view(np.uint32) == oa.view(np.uint32)).all() or (np.isnan(ga).all() and np.isnan(oa).all())
    assert np.array_equal(o.codes.cpu().numpy(), oc), "codes"
    assert np.array_equal(o.scales.cpu().numpy(), os_), "scales"
    g = o.g.cpu().numpy()
    assert (g.view(np.uint32) == og.view(np.uint32)).all() or (np.isnan(g).all() and np.isnan(og).all())


@pytest.mark.parametrize("mode", ["rn", "sr", "rht_sr"])
@pytest.mark.parametrize("shape", [(512, 200), (48, 8), (1040, 72), (16, 520), (2048, 1024), (4096, 1032),
                                   (48, 12), (64, 27), (4096, 4100)])
def test_colwise(mode, shape):
    x = W.lognormal_gradients(*shape, seed=(shape[0] * 5 + shape[1]) & 0xFFFF)
    check(x, mode, Q.COLWISE)


@pytest.mark.parametrize("mode", ["rn", "sr", "rht_sr"])
@pytest.mark.parametrize("shape", [(300, 160), (1, 16), (16, 16), (1000, 1040), (2048, 2048), (4096, 1056)])
def test_rowwise(mode, shape):
    """Ragged block counts: partial workgroups, lanes with fewer blocks than others, 1 or 2 blocks per lane."""
    x = W.outlier_columns(*shape, seed=(shape[0] * 3 + shape[1]) & 0xFFFF, n_cols=3)
    check(x, mode, Q.ROWWISE)


@pytest.mark.parametrize("mode", ["rn", "rht_sr"])
def test_rowwise_two_pass(mode):
    """More than 8192 blocks per CU: amax, then quantization."""
    check(W.lognormal_gradients(8208, 4096, seed=12), mode, Q.ROWWISE)


def test_consecutive_calls_reuse_the_barrier():
    """Back-to-back launches on one stream: every call sees only its own workgroups at the barrier."""
    x = W.lognormal_gradients(1024, 2048, seed=77)
    for call in range(6):
        check(x, "rht_sr", Q.COLWISE, mask=W.sign_mask(9, call), seed=9, offset=call)


@pytest.mark.parametrize("mode", ["rn", "rht_sr"])
def test_slow_route_after_a_timed_out_wait(monkeypatch, mode):
    """A zero wait bound sends workgroups that find a slot still empty down the slow route (each computes the maxima
    of the tiles it has not seen from the tensor itself); the result must not change."""
    monkeypatch.setenv("NVFP4_FUSED_WAIT_TICKS", "0")
    x = W.lognormal_gradients(2048, 1024, seed=91)
    for call in range(3):
        check(x, mode, Q.COLWISE, mask=W.sign_mask(4, call), seed=4, offset=call)
    monkeypatch.delenv("NVFP4_FUSED_WAIT_TICKS")
    check(x, mode, Q.COLWISE, mask=W.sign_mask(4, 7), seed=4, offset=7)     # and back on the fast route


@pytest.mark.parametrize("mode", ["sr", "rht_sr"])
def test_rowwise_slow_route(monkeypatch, mode):
    monkeypatch.setenv("NVFP4_FUSED_WAIT_TICKS", "0")
    x = W.outlier_columns(2048, 1024, seed=92, n_cols=5)
    for call in range(2):
        check(x, mode, Q.ROWWISE, mask=W.sign_mask(5, call), seed=5, offset=call)
    monkeypatch.delenv("NVFP4_FUSED_WAIT_TICKS")
    check(x, mode, Q.ROWWISE, mask=W.sign_mask(5, 2), seed=5, offset=2)


def test_concurrent_calls_on_two_streams():
    """Single-read calls in flight at once on two streams, on tensors of very different magnitudes: each launch
    exchanges its maxima in a slot region of its own, so neither sees the other's."""
    xa = W.lognormal_gradients(1024, 2048, seed=61)
    xb = W.gaussian(2048, 1024, seed=62, scale=1000.0)
    cases = [(xa, Q.COLWISE, "rht_sr"), (xb, Q.ROWWISE, "sr"), (xb, Q.COLWISE, "rn"), (xa, Q.ROWWISE, "rht_sr")]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    devs = [torch.from_numpy(x.view(np.int16)).cuda() for x, _, _ in cases]
    torch.cuda.synchronize()
    results = []
    for rep in range(3):
        for i, (x, orient, mode) in enumerate(cases):
            s_ = streams[i % 2]
            with torch.cuda.stream(s_):
                say("concurrent", rep, i, mode, x.shape)
                results.append((i, rep) + Q.nvfp4_amax_quantize(devs[i], orient, ROUNDING[mode][0], 0x3C5A, 8, rep,
                                                                stream=s_))
    torch.cuda.synchronize()
    for i, rep, a, o in results:
        x, orient, mode = cases[i]
        oa = O.amax(x, orient, O.G_PER_TENSOR, mode == "rht_sr", 0x3C5A)
        oc, os_, og = O.quantize_1x16(x, oa, ROUNDING[mode][1], orient, O.G_PER_TENSOR, 0x3C5A, 8, rep)
        assert (a.cpu().numpy().view(np.uint32) == oa.view(np.uint32)).all(), (i, rep)
        assert np.array_equal(o.codes.cpu().numpy(), oc), (i, rep)
        assert np.array_equal(o.scales.cpu().numpy(), os_), (i, rep)


def expect(x, orient, mode, mask, seed, offset, a, o, what):
    oa = O.amax(x, orient, O.G_PER_TENSOR, mode == "rht_sr", mask)
    oc, os_, og = O.quantize_1x16(x, oa, ROUNDING[mode][1], orient, O.G_PER_TENSOR, mask, seed, offset)
    assert (a.cpu().numpy().view(np.uint32) == oa.view(np.uint32)).all(), what
    assert np.array_equal(o.codes.cpu().numpy(), oc), what
    assert np.array_equal(o.scales.cpu().numpy(), os_), what
    assert (o.g.cpu().numpy().view(np.uint32) == og.view(np.uint32)).all(), what


def overlap_cases():
    xs = [W.lognormal_gradients(1024, 2048, seed=61), W.gaussian(2048, 1024, seed=62, scale=1000.0),
          W.outlier_columns(512, 4096, seed=63, n_cols=7), W.lognormal_gradients(2048, 4096, seed=64)]
    out = []
    for i in range(10):
        x = xs[i % 4]
        out.append((x, Q.COLWISE if i % 3 else Q.ROWWISE, ("rn", "sr", "rht_sr")[i % 3], W.sign_mask(70, i), 70, i))
    return out


def run_overlapping(cases, spin=200_000, rounds=2):
    """Every case on a stream of its own, each stream first held by a short spin so that the calls start together;
    no synchronisation until all are queued."""
    streams = [torch.cuda.Stream() for _ in cases]
    devs = [torch.from_numpy(c[0].view(np.int16)).cuda() for c in cases]
    torch.cuda.synchronize()
    results = []
    for rep in range(rounds):
        for i, (x, orient, mode, mask, seed, off) in enumerate(cases):
            with torch.cuda.stream(streams[i]):
                torch.cuda._sleep(spin)
                say("overlap", rep, i, mode, x.shape, orient)
                results.append((i, rep) + Q.nvfp4_amax_quantize(devs[i], orient, ROUNDING[mode][0], mask, seed,
                                                                off + 100 * rep, stream=streams[i]))
    torch.cuda.synchronize()
    for i, rep, a, o in results:
        x, orient, mode, mask, seed, off = cases[i]
        expect(x, orient, mode, mask, seed, off + 100 * rep, a, o, (i, rep))


def test_ten_overlapping_calls():
    """Ten single-read calls in flight at once on ten streams (more than the 8 slot regions, so launches may share
    one), column- and row-wise, on tensors of very different magnitudes: each must equal the oracle."""
    run_overlapping(overlap_cases())


def test_overlapping_calls_forced_into_one_region(monkeypatch):
    """Every launch in the same slot region while several run at once: a slot holding another launch's value is
    never taken as a maximum (it carries another epoch), so the launches fall back to reading the missing tiles
    and every result still equals the oracle."""
    monkeypatch.setenv("NVFP4_FUSED_REGION", "5")
    run_overlapping(overlap_cases()[:6], rounds=2)
    monkeypatch.delenv("NVFP4_FUSED_REGION")
    run_overlapping(overlap_cases()[:2], rounds=1)    # and the regions in turn again


def test_graph_replays_against_eager_calls_on_another_stream():
    """A captured single-read call (its epoch and region fixed at capture) replayed on one stream while eager calls
    run on another stream at the same time: the replays and the eager calls all equal the oracle."""
    xg = W.lognormal_gradients(2048, 1024, seed=33)
    xe = W.gaussian(1024, 2048, seed=34, scale=300.0)
    dg = torch.from_numpy(xg.view(np.int16)).cuda()
    de = torch.from_numpy(xe.view(np.int16)).cuda()
    sg, se = torch.cuda.Stream(), torch.cuda.Stream()
    a_g = torch.empty((1,), device="cuda")
    o_g = Q.alloc_out(1024, 2048, 0, dg.device)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=sg):
        Q.nvfp4_amax_quantize(dg, Q.COLWISE, Q.ROUND_RHT_SR, 0x2B2B, 3, 9, amax=a_g, out=o_g, stream=sg)
    torch.cuda.synchronize()
    for rep in range(4):
        say("graph vs eager", rep)
        a_g.fill_(1e30)
        o_g.codes.zero_()
        torch.cuda.synchronize()
        eager = []
        with torch.cuda.stream(sg):
            torch.cuda._sleep(200_000)
            graph.replay()
        with torch.cuda.stream(se):
            torch.cuda._sleep(200_000)
            for k in range(3):
                eager.append((k,) + Q.nvfp4_amax_quantize(de, Q.ROWWISE if k % 2 else Q.COLWISE, Q.ROUND_SR, 0, 5,
                                                          k, stream=se))
        torch.cuda.synchronize()
        expect(xg, Q.COLWISE, "rht_sr", 0x2B2B, 3, 9, a_g, o_g, ("graph", rep))
        for k, a, o in eager:
            expect(xe, Q.ROWWISE if k % 2 else Q.COLWISE, "sr", 0, 5, k, a, o, ("eager", rep, k))


def test_not_all_workgroups_waited_for(monkeypatch):
    """A zero bound on the wait for workgroups that have not started: a workgroup that polls before every other has
    announced itself stops waiting at once and reads the missing tiles; the result must not change."""
    monkeypatch.setenv("NVFP4_FUSED_ARRIVE_TICKS", "0")
    for call in range(3):
        check(W.lognormal_gradients(2048, 4096, seed=95), "rht_sr", Q.COLWISE, mask=W.sign_mask(8, call), seed=8,
              offset=call)
        check(W.outlier_columns(4096, 2048, seed=96, n_cols=4), "sr", Q.ROWWISE, mask=0, seed=8, offset=call)
    monkeypatch.delenv("NVFP4_FUSED_ARRIVE_TICKS")


def test_nan_and_zero_tensors():
    x = W.lognormal_gradients(256, 512, seed=5)
    x[100, 7] = 0x7FC0                      # bf16 NaN
    check(x, "rht_sr", Q.COLWISE)
    check(x, "rht_sr", Q.ROWWISE)
    check(np.zeros((256, 512), np.uint16), "sr", Q.COLWISE)
    check(np.zeros((256, 512), np.uint16), "sr", Q.ROWWISE)


def test_empty_tensor():
    xd = torch.empty((0, 64), dtype=torch.int16, device="cuda")
    a, o = Q.nvfp4_amax_quantize(xd, Q.COLWISE, Q.ROUND_RHT_SR, 0x1111, 1, 2)
    torch.cuda.synchronize()
    assert a.item() == 0.0 and o.g.item() == 0.0


@pytest.mark.slow
def test_full_wgrad_colwise_single_read():
    """The benchmarked workload (8192 x 4096: one tile per CU) through the single-read launch, two fresh calls."""
    x = W.make("wgrad_colwise_rht_sr_8192x4096")
    for call in (0, 1):
        check(x, "rht_sr", Q.COLWISE, mask=W.sign_mask(2, call), seed=2, offset=call)


@pytest.mark.slow
def test_full_fprop_rowwise_single_read():
    """8192 x 4096 row-wise (8 blocks per lane on 256 CUs) through the single-read launch."""
    x = W.make("fprop_rn_8192x4096")
    check(x, "rn", Q.ROWWISE)
    check(x, "rht_sr", Q.ROWWISE, mask=W.sign_mask(6, 0), seed=6, offset=0)


def test_graph_replays_match_eager():
    """The call captured in a HIP graph; replays (with eager work between them) match the eager result."""
    x = W.lognormal_gradients(2048, 1024, seed=31)
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    a_e, o_e = Q.nvfp4_amax_quantize(xd, Q.COLWISE, Q.ROUND_RHT_SR, 0x0F0F, 3, 4)
    torch.cuda.synchronize()
    a_g = torch.full((1,), 7.0, device="cuda")
    o_g = Q.alloc_out(1024, 2048, 0, xd.device)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        Q.nvfp4_amax_quantize(xd, Q.COLWISE, Q.ROUND_RHT_SR, 0x0F0F, 3, 4, amax=a_g, out=o_g)
    for rep in range(4):
        say("graph replay", rep)
        a_g.fill_(1e30)
        o_g.codes.zero_()
        Q.nvfp4_amax_quantize(xd, Q.COLWISE, Q.ROUND_RN, 0, 0, 0)      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(a_g.view(torch.int32), a_e.view(torch.int32))
        assert torch.equal(o_g.codes, o_e.codes) and torch.equal(o_g.scales, o_e.scales)
        assert torch.equal(o_g.g, o_e.g)
