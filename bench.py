#!/usr/bin/env python3
"""Benchmark of the NVFP4 quantizer on one MI355X.

One step = the whole hot path over one batch of synthetic input: the per-tensor amax of the Hadamard-transformed
blocks and the fused RHT + two-level scale + Philox SR + packing pass, on an 8192x4096 bf16 gradient quantized
column-wise (blocks along the 8192 dimension), with fresh random signs and a fresh Philox offset every step.  The
step is one nvfp4_amax_quantize call: at this size the tensor fits the chip, so a single launch reads it once, keeps
every tile in registers while the amax is agreed on, and quantizes it.

Metric: effective GB/s = (bf16 bytes in + E2M1 code bytes + E4M3 scale bytes + g) per step / step time.  Inputs
are resident in HBM when timing starts; the steps rotate over enough copies of the input and outputs
(> 2x the 256 MB Infinity Cache) that every step reads its input from HBM rather than from the cache.  The K timed
steps (each with its own sign mask and Philox offset) are captured once into a HIP graph and the timed region is one
replay of it, so host launch overhead is not part of the measurement; the same steps launched eagerly are timed too
and reported as `ms_per_step_eager`.

Also printed in the same JSON line:
  roofline      the step's kernel: algorithmic bytes / its mean duration (the step graph holds K launches of it,
                HIP events around the replay on the launch stream) against MI355X's 8 TB/s HBM peak, and the HBM
                traffic measured with rocprofv3 counters (null unless measured on the current kernel source);
  cpu_baseline  the CPU oracle (test infrastructure) on the same workload, timed on the host cores;
  extra         the two-pass step (nvfp4_amax + nvfp4_quantize_rht_sr), the quantize kernel alone given a
                device-resident amax (the pages' kernel-only comparison, with a roofline object of its own and its
                counter-measured traffic), the amax call, the row-wise RHT+SR pass,
                and under "configs" the other workloads: the 256x1024 RHT+SR/RN pair, the 8192x4096 row-wise RN
                activation pass, the 14336x4096 16x16 weight pass (W and W^T), the 16384x8192 four-over-six pass
                the decode of its output (to float, and to bf16 through the fused decode), and the fused decode of the
                column-wise RHT+SR output back through the inverse transform to bf16, and 32 small tensors quantized
                by two grouped launches against 64 single-tensor calls (each timed as a graph of K launches, inputs
                rotating through HBM).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E peak
MALL_BYTES = 256 << 20       # Infinity Cache
WORKLOAD = "wgrad_colwise_rht_sr_8192x4096"
ROWS, COLS = 8192, 4096
SEED = 2
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "k_amax_quant_colwise_rht_sr_8192x4096_traffic.txt")
QUANT_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "k_quant_colwise_rht_sr_8192x4096_traffic.txt")
COPY_BYTES = 128 << 20       # the calibration copy for the L2-to-memory byte counters
PERCENTILE_LAUNCHES = 200    # launches timed one by one for the percentiles


def algorithmic_bytes(rows: int, cols: int) -> int:
    """bf16 in + packed E2M1 codes + E4M3 scales + one FP32 global scale."""
    n = rows * cols
    return 2 * n + n // 2 + n // 16 + 4


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="target duration of the CPU-oracle baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--config-launches", type=int, default=50,
                   help="graph launches per kernel for the other workloads (0 skips them)")
    p.add_argument("--counter-launches", type=int, default=0, metavar="N",
                   help="for a rocprofv3 --pmc run: launch N steps eagerly, N quantize-only calls (amax given), "
                        "then N copies of a 128 MiB buffer (the calibration copy), and exit without timing")
    p.add_argument("--counter-configs", action="store_true",
                   help="with --counter-launches: also launch N 16x16 W+W^T quantizations of the 14336x4096 weight and "
                        "N four-over-six quantizations of the 16384x8192 tensor (per-row g, no NaN/Inf), amax given, "
                        "before the calibration copies")
    return p.parse_args()


def kernel_source_digest() -> str:
    """sha256 of the HIP kernel sources; a traffic figure is reported only for the source it was measured on."""
    h = hashlib.sha256()
    for name in ("nvfp4_kernels.hip", "nvfp4_launch.h"):
        with open(os.path.join(ROOT, "nvfp4_quantization_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(path: str = TRAFFIC_SUMMARY):
    """HBM bytes per launch of a kernel from its committed counter summary, or None when the kernels have changed."""
    fields = {}
    try:
        with open(path) as f:
            for line in f:
                key, sep, val = line.partition(":")
                if sep:
                    fields[key.strip()] = val.strip()
    except OSError:
        return None
    if fields.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return int(fields["traffic_bytes_per_launch"])


def run_step(Q, xs, outs, amaxes, k: int, masks):
    i = k % len(xs)
    Q.nvfp4_amax_quantize(xs[i], Q.COLWISE, Q.ROUND_RHT_SR, masks[k % len(masks)], SEED, k, amax=amaxes[i],
                          out=outs[i])


def run_two_pass_step(Q, xs, outs, amaxes, k: int, masks):
    i = k % len(xs)
    mask = masks[k % len(masks)]
    Q.nvfp4_amax(xs[i], Q.COLWISE, Q.G_PER_TENSOR, use_rht=True, sign_mask=mask, amax=amaxes[i])
    Q.nvfp4_quantize_rht_sr(xs[i], amaxes[i], mask, SEED, k, Q.COLWISE, Q.G_PER_TENSOR, out=outs[i])


def capture(fn, first: int, count: int) -> torch.cuda.CUDAGraph:
    """A HIP graph of fn(first), ..., fn(first + count - 1)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(first, first + count):
            fn(k)
    return g


def time_graph(g: torch.cuda.CUDAGraph) -> float:
    """Milliseconds of one replay of g (after an untimed one), bracketed by device synchronisation and events on the
    launch stream."""
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g.replay()
    torch.cuda.synchronize()
    start.record()
    g.replay()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop)


def gbs(nbytes: int, ms: float) -> float:
    return round(nbytes / (ms * 1e-3) / 1e9, 2)


_bench_lib = None


def bench_lib():
    """The streaming ceiling kernel and the stream-hold kernel (libnvfp4_bench.so, built with the HIP library)."""
    global _bench_lib
    if _bench_lib is None:
        import ctypes as C
        from nvfp4_quantization_amd._build import BENCH_LIB_PATH
        if not os.path.exists(BENCH_LIB_PATH):
            raise RuntimeError(f"{BENCH_LIB_PATH} is missing: build first (python -m nvfp4_quantization_amd._build)")
        L = C.CDLL(BENCH_LIB_PATH)
        L.nvfp4_bench_stream.restype = C.c_int
        L.nvfp4_bench_stream.argtypes = [C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p]
        L.nvfp4_bench_hold.restype = C.c_int
        L.nvfp4_bench_hold.argtypes = [C.c_int64, C.c_void_p]
        _bench_lib = L
    return _bench_lib


def launch_percentiles(fn, count: int) -> dict:
    """p10 / median / p90 of single-launch durations (microseconds): a hold kernel keeps the stream busy while the
    host queues count launches, each between two events on the launch stream, so that they run back to back.  Each
    figure includes the gap that an event record puts between two kernels (about 3 us here); the rocprofv3
    kernel trace gives the same percentiles without it."""
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(count + 1)]
    torch.cuda.synchronize()
    rc = bench_lib().nvfp4_bench_hold(50000, stream.cuda_stream)
    if rc:
        raise RuntimeError(f"hold kernel launch failed: {rc}")
    ev[0].record(stream)
    for k in range(count):
        fn(k)
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    us = np.array([1e3 * ev[k].elapsed_time(ev[k + 1]) for k in range(count)])
    p10, p50, p90 = np.percentile(us, [10, 50, 90])
    return {"p10_us": round(float(p10), 2), "median_us": round(float(p50), 2), "p90_us": round(float(p90), 2),
            "launches": count}


def stream_ceiling(xs, outs, launches: int) -> dict:
    """The streaming kernel with the quantizer's byte mix (32 B read, 8 + 1 B written per block) on the same
    rotating buffers: the practical bandwidth ceiling for this traffic."""
    L = bench_lib()
    nblocks = xs[0].numel() // 16
    n = len(xs)

    def launch(k):
        i = k % n
        rc = L.nvfp4_bench_stream(xs[i].data_ptr(), nblocks, outs[i].codes.data_ptr(), outs[i].scales.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
        if rc:
            raise RuntimeError(f"streaming kernel launch failed: {rc}")

    launch(0)
    ms = time_graph(capture(launch, 0, launches)) / launches
    b = 32 * nblocks + 9 * nblocks
    return {"kernel_us": round(1e3 * ms, 2), "gbs": gbs(b, ms), "frac_of_hbm_peak": round(gbs(b, ms) / HBM_PEAK_GBS, 4),
            "bytes_per_launch": b}


def config_figures(Q, W, dev, launches: int) -> dict:
    """Kernel times of the other workloads, each as the mean over a graph of `launches` launches whose inputs
    rotate over enough buffers to exceed twice the Infinity Cache."""
    out = {}

    def rotation(x_bits, extra_bytes):
        x = torch.from_numpy(x_bits.view(np.int16)).to(dev)
        n = max(2, -(-2 * MALL_BYTES // (x.numel() * 2 + extra_bytes)) + 1)
        return [x] + [x.clone() for _ in range(n - 1)]

    def timed(fn):
        return time_graph(capture(fn, 0, launches)) / launches

    # 256 x 1024, row-wise, RHT+SR and RN, amax and quantization in one call each (launch-bound at this size)
    xb = W.make("rht_sr_small_256x1024")
    x = torch.from_numpy(xb.view(np.int16)).to(dev)
    o = Q.alloc_out(256, 1024, Q.G_PER_TENSOR, dev)
    a = torch.empty(1, dtype=torch.float32, device=dev)
    m0 = W.sign_mask(0, 0)
    out["rht_sr_small_256x1024"] = {
        "call": "nvfp4_amax_quantize, row-wise",
        "rht_sr_us": round(1e3 * timed(lambda k: Q.nvfp4_amax_quantize(x, Q.ROWWISE, Q.ROUND_RHT_SR, m0, 0, k,
                                                                         amax=a, out=o)), 2),
        "rn_us": round(1e3 * timed(lambda k: Q.nvfp4_amax_quantize(x, Q.ROWWISE, Q.ROUND_RN, amax=a, out=o)), 2),
        "bytes_per_call": algorithmic_bytes(256, 1024)}

    # 8192 x 4096 activations, row-wise RN: single read, and the quantize kernel given the amax
    r, c = 8192, 4096
    xs = rotation(W.make("fprop_rn_8192x4096"), algorithmic_bytes(r, c) - 2 * r * c)
    n = len(xs)
    outs = [Q.alloc_out(r, c, Q.G_PER_TENSOR, dev) for _ in range(n)]
    am = [Q.nvfp4_amax(xs[i], Q.ROWWISE, Q.G_PER_TENSOR) for i in range(n)]
    b = algorithmic_bytes(r, c)
    single = timed(lambda k: Q.nvfp4_amax_quantize(xs[k % n], Q.ROWWISE, Q.ROUND_RN, amax=am[k % n], out=outs[k % n]))
    qonly = timed(lambda k: Q.nvfp4_quantize_rn(xs[k % n], am[k % n], Q.BLOCK_1X16, Q.ROWWISE, Q.G_PER_TENSOR,
                                                row_out=outs[k % n]))
    # the same calls writing the scales in the FP4 GEMM's tiled layout
    touts = [Q.alloc_out(r, c, Q.G_PER_TENSOR, dev, Q.SCALES_TILED) for _ in range(n)]
    single_t = timed(lambda k: Q.nvfp4_amax_quantize(xs[k % n], Q.ROWWISE, Q.ROUND_RN, amax=am[k % n],
                                                     out=touts[k % n]))
    qonly_t = timed(lambda k: Q.nvfp4_quantize_rn(xs[k % n], am[k % n], Q.BLOCK_1X16, Q.ROWWISE, Q.G_PER_TENSOR,
                                                  row_out=touts[k % n]))
    out["fprop_rn_8192x4096"] = {
        "single_read_us": round(1e3 * single, 2), "single_read_gbs": gbs(b, single),
        "quantize_kernel_us": round(1e3 * qonly, 2), "quantize_kernel_gbs": gbs(b, qonly),
        "quantize_kernel_frac_of_hbm_peak": round(gbs(b, qonly) / HBM_PEAK_GBS, 4),
        "tiled_scales": {"single_read_us": round(1e3 * single_t, 2), "quantize_kernel_us": round(1e3 * qonly_t, 2)}}
    del xs, outs, am, touts

    # 14336 x 4096 weight, 16x16 blocks, W and W^T from one read (amax given)
    r, c = 14336, 4096
    b16 = 2 * r * c + 2 * (r * c // 2) + 2 * (r * c // 16) + 4
    xs = rotation(W.make("weight_16x16_14336x4096"), b16 - 2 * r * c)
    n = len(xs)
    outs = [(Q.alloc_out(r, c, Q.G_PER_TENSOR, dev), Q.alloc_out(c, r, Q.G_PER_TENSOR, dev)) for _ in range(n)]
    am = [Q.nvfp4_amax(xs[i], Q.ROWWISE, Q.G_PER_TENSOR) for i in range(n)]
    t16 = timed(lambda k: Q.nvfp4_quantize_rn(xs[k % n], am[k % n], Q.BLOCK_16X16, Q.BOTH, Q.G_PER_TENSOR,
                                              row_out=outs[k % n][0], col_out=outs[k % n][1]))
    ta = timed(lambda k: Q.nvfp4_amax(xs[k % n], Q.ROWWISE, Q.G_PER_TENSOR, amax=am[k % n]))
    out["weight_16x16_14336x4096"] = {
        "quantize_kernel_us": round(1e3 * t16, 2), "quantize_kernel_gbs": gbs(b16, t16),
        "quantize_kernel_frac_of_hbm_peak": round(gbs(b16, t16) / HBM_PEAK_GBS, 4), "bytes_per_call": b16,
        "amax_us": round(1e3 * ta, 2)}
    # the same weight, four-over-six with 16x16 tiles (amax given): W alone, and W and W^T from one read
    b46t = 2 * r * c + r * c // 2 + r * c // 16 + 4
    t46t = timed(lambda k: Q.nvfp4_quantize_4o6_16x16(xs[k % n], am[k % n], row_out=outs[k % n][0]))
    t46b = timed(lambda k: Q.nvfp4_quantize_4o6_16x16(xs[k % n], am[k % n], Q.BOTH, row_out=outs[k % n][0],
                                                      col_out=outs[k % n][1]))
    out["four_over_six_16x16_14336x4096"] = {
        "call": "nvfp4_quantize_4o6_16x16", "quantize_kernel_us": round(1e3 * t46t, 2),
        "quantize_kernel_gbs": gbs(b46t, t46t), "quantize_kernel_frac_of_hbm_peak": round(gbs(b46t, t46t) / HBM_PEAK_GBS, 4),
        "bytes_per_call": b46t,
        "both_orientations": {"quantize_kernel_us": round(1e3 * t46b, 2), "quantize_kernel_gbs": gbs(b16, t46b),
                              "quantize_kernel_frac_of_hbm_peak": round(gbs(b16, t46b) / HBM_PEAK_GBS, 4),
                              "bytes_per_call": b16}}
    # the same weight widened to float32 (2 buffers)
    b46f = 4 * r * c + r * c // 2 + r * c // 16 + 4
    wf = [(t.to(torch.int32) << 16).view(torch.float32) for t in xs[:2]]
    amw = [Q.nvfp4_amax_f32(t, Q.G_PER_TENSOR) for t in wf]
    t46f = timed(lambda k: Q.nvfp4_quantize_4o6_16x16_f32(wf[k % 2], amw[k % 2], row_out=outs[k % n][0]))
    out["four_over_six_16x16_f32_14336x4096"] = {
        "call": "nvfp4_quantize_4o6_16x16_f32", "quantize_kernel_us": round(1e3 * t46f, 2),
        "quantize_kernel_gbs": gbs(b46f, t46f), "quantize_kernel_frac_of_hbm_peak": round(gbs(b46f, t46f) / HBM_PEAK_GBS, 4),
        "bytes_per_call": b46f}
    del wf, amw
    del xs, outs, am

    # 16384 x 8192 four-over-six with per-row g (per-row amax given), and the decode of its output
    r, c = 16384, 8192
    b46 = 2 * r * c + r * c // 2 + r * c // 16 + 4 * r
    xs = rotation(W.make("four_over_six_16384x8192"), b46 - 2 * r * c)
    n = len(xs)
    outs = [Q.alloc_out(r, c, Q.G_PER_ROW, dev) for _ in range(n)]
    am = [Q.nvfp4_amax(xs[i], Q.ROWWISE, Q.G_PER_ROW) for i in range(n)]
    t46 = timed(lambda k: Q.nvfp4_quantize_4o6(xs[k % n], am[k % n], Q.G_PER_ROW, out=outs[k % n]))
    tar = timed(lambda k: Q.nvfp4_amax(xs[k % n], Q.ROWWISE, Q.G_PER_ROW, amax=am[k % n]))
    out["four_over_six_16384x8192"] = {
        "quantize_kernel_us": round(1e3 * t46, 2), "quantize_kernel_gbs": gbs(b46, t46),
        "quantize_kernel_frac_of_hbm_peak": round(gbs(b46, t46) / HBM_PEAK_GBS, 4), "bytes_per_call": b46,
        "per_row_amax_us": round(1e3 * tar, 2),
        "note": "about 56% of rows hold an injected NaN or Inf, so their g is NaN or Inf and every code is 0x7"}
    # the same shapes and distributions without the injected NaN/Inf: every row takes both candidates
    xc = rotation(W.make("four_over_six_16384x8192", frac_special=0.0), b46 - 2 * r * c)
    amc = [Q.nvfp4_amax(xc[i], Q.ROWWISE, Q.G_PER_ROW) for i in range(n)]
    tc = timed(lambda k: Q.nvfp4_quantize_4o6(xc[k % n], amc[k % n], Q.G_PER_ROW, out=outs[k % n]))
    out["four_over_six_16384x8192_no_nan_inf"] = {
        "quantize_kernel_us": round(1e3 * tc, 2), "quantize_kernel_gbs": gbs(b46, tc),
        "quantize_kernel_frac_of_hbm_peak": round(gbs(b46, tc) / HBM_PEAK_GBS, 4)}
    # the same no-NaN/Inf input widened to float32, through the binary32-input four-over-six (2 buffers)
    b46f = 4 * r * c + r * c // 2 + r * c // 16 + 4 * r
    xf = [(t.to(torch.int32) << 16).view(torch.float32) for t in xc[:2]]
    amf = [Q.nvfp4_amax_f32(t, Q.G_PER_ROW) for t in xf]
    tf = timed(lambda k: Q.nvfp4_quantize_4o6_f32(xf[k % 2], amf[k % 2], Q.G_PER_ROW, out=outs[k % n]))
    out["four_over_six_f32_16384x8192"] = {
        "call": "nvfp4_quantize_4o6_f32, per-row g", "quantize_kernel_us": round(1e3 * tf, 2),
        "quantize_kernel_gbs": gbs(b46f, tf), "quantize_kernel_frac_of_hbm_peak": round(gbs(b46f, tf) / HBM_PEAK_GBS, 4),
        "bytes_per_call": b46f}
    del xs, xc, amc, xf, amf
    y = torch.empty((r, c), dtype=torch.float32, device=dev)
    bdq = r * c // 2 + r * c // 16 + 4 * r + 4 * r * c
    tdq = timed(lambda k: Q.nvfp4_dequantize(outs[k % n].codes, outs[k % n].scales, outs[k % n].g, Q.G_PER_ROW, y=y))
    out["dequantize_16384x8192"] = {
        "kernel_us": round(1e3 * tdq, 2), "gbs": gbs(bdq, tdq),
        "frac_of_hbm_peak": round(gbs(bdq, tdq) / HBM_PEAK_GBS, 4), "bytes_per_call": bdq}
    del y
    # the same decode written as bf16 by the fused decode (no rotation)
    yb = torch.empty((r, c), dtype=torch.bfloat16, device=dev)
    bdb = r * c // 2 + r * c // 16 + 4 * r + 2 * r * c
    tdb = timed(lambda k: Q.nvfp4_dequantize_fused(outs[k % n].codes, outs[k % n].scales, outs[k % n].g, Q.G_PER_ROW,
                                                   False, 0, True, y=yb))
    out["dequantize_bf16_16384x8192"] = {
        "call": "nvfp4_dequantize_fused, bf16 output",
        "kernel_us": round(1e3 * tdb, 2), "gbs": gbs(bdb, tdb),
        "frac_of_hbm_peak": round(gbs(bdb, tdb) / HBM_PEAK_GBS, 4), "bytes_per_call": bdb}
    del outs, am, yb
    torch.cuda.empty_cache()

    # 32 small tensors (256 x 1024, the pages' small RHT+SR case, each with its own seed): amax + RHT+SR quantization
    # as two grouped launches, against the same work as 64 single-tensor calls; both at the same bytes
    G, r, c = 32, 256, 1024
    gx = [torch.from_numpy(W.outlier_columns(r, c, seed=100 + k).view(np.int16)).to(dev) for k in range(G)]
    gm = [W.sign_mask(100 + k, 0) for k in range(G)]
    ga = [torch.empty(1, dtype=torch.float32, device=dev) for _ in range(G)]
    go = [Q.alloc_out(r, c, Q.G_PER_TENSOR, dev) for _ in range(G)]
    seeds = [7] * G

    def grouped(k):
        Q.nvfp4_amax_grouped(gx, Q.G_PER_TENSOR, True, gm, amaxes=ga)
        Q.nvfp4_quantize_grouped(gx, ga, Q.ROUND_RHT_SR, Q.G_PER_TENSOR, gm, seeds, [k] * G, outs=go)

    def separate(k):
        for i in range(G):
            Q.nvfp4_amax(gx[i], Q.ROWWISE, Q.G_PER_TENSOR, True, gm[i], amax=ga[i])
            Q.nvfp4_quantize_rht_sr(gx[i], ga[i], gm[i], 7, k, Q.ROWWISE, Q.G_PER_TENSOR, out=go[i])

    tg, ts = timed(grouped), timed(separate)
    bg = G * algorithmic_bytes(r, c)
    out["grouped_32x_256x1024_rht_sr"] = {
        "call": "nvfp4_amax_grouped + nvfp4_quantize_grouped (2 launches) vs nvfp4_amax + nvfp4_quantize_rht_sr per "
                "tensor (64 calls), row-wise",
        "grouped_us": round(1e3 * tg, 2), "separate_us": round(1e3 * ts, 2), "speedup": round(ts / tg, 2),
        "grouped_gbs": gbs(bg, tg), "bytes_per_call": bg}
    del gx, ga, go

    # 8192 x 4096 weight gradient quantized column-wise with RHT + SR, decoded back through the inverse transform
    # to bf16 (V = X^T, 4096 x 8192); outputs and decoded tensors rotate through HBM
    r, c = 8192, 4096
    bdr = algorithmic_bytes(r, c)          # codes + scales + g in, bf16 out: the quantizer's bytes reversed
    n = max(2, -(-2 * MALL_BYTES // bdr) + 1)
    x = torch.from_numpy(W.make(WORKLOAD).view(np.int16)).to(dev)
    mask = W.sign_mask(SEED, 0)
    qs = [Q.nvfp4_amax_quantize(x, Q.COLWISE, Q.ROUND_RHT_SR, mask, SEED, i)[1] for i in range(n)]
    ys = [torch.empty((c, r), dtype=torch.bfloat16, device=dev) for _ in range(n)]
    del x
    tdr = timed(lambda k: Q.nvfp4_dequantize_fused(qs[k % n].codes, qs[k % n].scales, qs[k % n].g, Q.G_PER_TENSOR,
                                                   True, mask, True, y=ys[k % n]))
    out["dequantize_rht_bf16_8192x4096"] = {
        "call": "nvfp4_dequantize_fused, inverse RHT, bf16 output, of the column-wise RHT+SR quantization",
        "kernel_us": round(1e3 * tdr, 2), "gbs": gbs(bdr, tdr),
        "frac_of_hbm_peak": round(gbs(bdr, tdr) / HBM_PEAK_GBS, 4), "bytes_per_call": bdr}
    del qs, ys
    torch.cuda.empty_cache()

    # the scales of the 8192 x 4096 row-wise quantization (8192 x 256) to the FP4 GEMM's tiled layout; 8 buffers
    rv, nb = 8192, 256
    ss = [torch.randint(0, 256, (rv, nb), dtype=torch.uint8, device=dev) for _ in range(8)]
    so = [torch.empty(Q.nvfp4_swizzled_scales_size(rv, nb), dtype=torch.uint8, device=dev) for _ in range(8)]
    tsw = timed(lambda k: Q.nvfp4_swizzle_scales(ss[k % 8], out=so[k % 8]))
    out["swizzle_scales_8192x256"] = {
        "call": "nvfp4_swizzle_scales (scales of the 8192x4096 row-wise quantization)",
        "kernel_us": round(1e3 * tsw, 2), "bytes_per_call": 2 * rv * nb}
    del ss, so
    return out


def cpu_baseline(Q, x_bits: np.ndarray, x0: torch.Tensor, masks, target_s: float) -> dict:
    """The CPU oracle (test infrastructure, untuned) on the same workload: full steps on every host core for about
    target_s seconds, then on one thread for about a third of that; and one step's output of the GPU compared byte
    for byte with the oracle's."""
    import oracle as O
    cores = len(os.sched_getaffinity(0))

    def oracle_step(k):
        m = masks[k % len(masks)]
        a = O.amax(x_bits, O.COLWISE, O.G_PER_TENSOR, True, m)
        return (a,) + tuple(O.quantize_1x16(x_bits, a, O.MODE_RHT_SR, O.COLWISE, O.G_PER_TENSOR, m, SEED, k))

    def timed_steps(threads, seconds):
        O.set_num_threads(threads)
        t0 = time.perf_counter()
        steps = 0
        while True:
            oracle_step(steps)
            steps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return steps, el, O.num_threads()

    steps, el, used = timed_steps(cores, target_s)
    steps1, el1, _ = timed_steps(1, target_s / 3)
    O.set_num_threads(cores)
    # step 0 on the GPU (fresh outputs) against the oracle's step 0
    a_gpu, o_gpu = Q.nvfp4_amax_quantize(x0, Q.COLWISE, Q.ROUND_RHT_SR, masks[0], SEED, 0)
    torch.cuda.synchronize()
    a, codes, scales, g = oracle_step(0)
    match = (np.array_equal(a_gpu.cpu().numpy().view(np.uint32), a.view(np.uint32))
             and np.array_equal(o_gpu.codes.cpu().numpy(), codes) and np.array_equal(o_gpu.scales.cpu().numpy(), scales)
             and np.array_equal(o_gpu.g.cpu().numpy().view(np.uint32), g.view(np.uint32)))
    nbytes = algorithmic_bytes(ROWS, COLS)
    return {"value": round(nbytes * steps / el / 1e9, 3), "unit": "GB/s", "cores": used, "kind": "oracle",
            "sample": f"{steps} full steps (amax + RHT+SR quantize) of the {ROWS}x{COLS} workload, {el:.1f} s wall",
            "single_thread": {"value": round(nbytes * steps1 / el1 / 1e9, 4), "unit": "GB/s",
                              "sample": f"{steps1} full steps on one thread, {el1:.1f} s wall"},
            "gpu_step_equals_oracle_bytes": bool(match)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the quantizer has no "
              "multi-GPU path: each GPU would quantize its own shard after a 4-byte MAX all-reduce of the amax).",
              file=sys.stderr)
        sys.exit(2)
    import nvfp4_quantization_amd as Q
    from nvfp4_quantization_amd import workloads as W

    Q.binding.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x_bits = W.make(WORKLOAD)
    x0 = torch.from_numpy(x_bits.view(np.int16)).to(dev)
    step_bytes = algorithmic_bytes(ROWS, COLS)
    nbuf = max(2, -(-2 * MALL_BYTES // step_bytes) + 1)          # footprint > 2x the Infinity Cache
    xs = [x0] + [x0.clone() for _ in range(nbuf - 1)]
    outs = [Q.alloc_out(COLS, ROWS, Q.G_PER_TENSOR, dev) for _ in range(nbuf)]
    amaxes = [torch.empty(1, dtype=torch.float32, device=dev) for _ in range(nbuf)]
    masks = [W.sign_mask(SEED, k) for k in range(64)]
    torch.cuda.synchronize()

    step = lambda k: run_step(Q, xs, outs, amaxes, k, masks)
    stream = torch.cuda.Stream()          # a dedicated stream (default priority) for every timed launch
    with torch.cuda.stream(stream):
        result = measure(args, Q, W, dev, x_bits, x0, xs, outs, amaxes, masks, step, nbuf, step_bytes)
    if result is None:
        return
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(Q, x_bits, x0, masks, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def measure(args, Q, W, dev, x_bits, x0, xs, outs, amaxes, masks, step, nbuf, step_bytes):
    if args.counter_launches:
        for k in range(args.counter_launches):
            step(k)
        for k in range(args.counter_launches):           # the quantize kernel alone, on the amax the steps wrote
            Q.nvfp4_quantize_rht_sr(xs[k % nbuf], amaxes[k % nbuf], masks[k % 64], SEED, k, Q.COLWISE,
                                    Q.G_PER_TENSOR, out=outs[k % nbuf])
        if args.counter_configs:
            # two input buffers each, alternating; every output buffer written in full by every launch
            r, c = 14336, 4096
            w0 = torch.from_numpy(W.make("weight_16x16_14336x4096").view(np.int16)).to(dev)
            ws = [w0, w0.clone()]
            wa = Q.nvfp4_amax(w0, Q.ROWWISE, Q.G_PER_TENSOR)
            wo = (Q.alloc_out(r, c, Q.G_PER_TENSOR, dev), Q.alloc_out(c, r, Q.G_PER_TENSOR, dev))
            for k in range(args.counter_launches):
                Q.nvfp4_quantize_rn(ws[k % 2], wa, Q.BLOCK_16X16, Q.BOTH, Q.G_PER_TENSOR, row_out=wo[0], col_out=wo[1])
            torch.cuda.synchronize()
            del ws, wo
            r, c = 16384, 8192
            f0 = torch.from_numpy(W.make("four_over_six_16384x8192", frac_special=0.0).view(np.int16)).to(dev)
            fs = [f0, f0.clone()]
            fa = Q.nvfp4_amax(f0, Q.ROWWISE, Q.G_PER_ROW)
            fo = Q.alloc_out(r, c, Q.G_PER_ROW, dev)
            for k in range(args.counter_launches):
                Q.nvfp4_quantize_4o6(fs[k % 2], fa, Q.G_PER_ROW, out=fo)
            torch.cuda.synchronize()
            del fs, fo
            torch.cuda.empty_cache()
        # four source/destination pairs in turn, so that no copy finds its source still in the L2 caches (32 MB)
        srcs = [torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).uniform_() for _ in range(4)]
        dsts = [torch.empty_like(srcs[0]) for _ in range(4)]
        for k in range(args.counter_launches):
            dsts[k % 4].copy_(srcs[k % 4])
        torch.cuda.synchronize()
        print(f"counter pass: {args.counter_launches} steps, {args.counter_launches} quantize-only calls and "
              f"{args.counter_launches} copies of {COPY_BYTES >> 20} MiB launched", flush=True)
        return None
    for k in range(args.warmup):                       # eager warm-up (also initialises the library)
        step(k)
    torch.cuda.synchronize()
    steps_graph = capture(step, args.warmup, args.steps)
    total_ms = time_graph(steps_graph)
    ms_per_step = total_ms / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # the same steps launched eagerly (host launch overhead included), for reference
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for k in range(args.steps):
        step(args.warmup + k)
    stop.record()
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(stop) / args.steps

    # the two-pass step, and kernel-level figures: K launches of one kernel in a graph, events around the replay
    two = lambda k: run_two_pass_step(Q, xs, outs, amaxes, k, masks)
    two_ms = time_graph(capture(two, 0, args.steps)) / args.steps
    quant = lambda k: Q.nvfp4_quantize_rht_sr(xs[k % nbuf], amaxes[k % nbuf], masks[k % 64], SEED, k, Q.COLWISE,
                                              Q.G_PER_TENSOR, out=outs[k % nbuf])
    q_ms = time_graph(capture(quant, 0, args.steps)) / args.steps
    q_gbs = step_bytes / (q_ms * 1e-3) / 1e9
    amax = lambda k: Q.nvfp4_amax(xs[k % nbuf], Q.COLWISE, Q.G_PER_TENSOR, True, masks[k % 64], amax=amaxes[k % nbuf])
    amax_ms = time_graph(capture(amax, 0, args.steps)) / args.steps
    row_outs = [Q.alloc_out(ROWS, COLS, Q.G_PER_TENSOR, dev) for _ in range(nbuf)]
    row_amax = Q.nvfp4_amax(x0, Q.ROWWISE, Q.G_PER_TENSOR, True, masks[0])
    rowq = lambda k: Q.nvfp4_quantize_rht_sr(xs[k % nbuf], row_amax, masks[0], SEED, k, Q.ROWWISE, Q.G_PER_TENSOR,
                                             out=row_outs[k % nbuf])
    row_ms = time_graph(capture(rowq, 0, args.steps)) / args.steps
    del row_outs
    # GEMM-ready outputs: the step writing its scales in the FP4 GEMM's tiled layout, against the step followed by
    # the separate re-layout of its scales
    tiled_outs = [Q.alloc_out(COLS, ROWS, Q.G_PER_TENSOR, dev, Q.SCALES_TILED) for _ in range(nbuf)]
    tiled = lambda k: Q.nvfp4_amax_quantize(xs[k % nbuf], Q.COLWISE, Q.ROUND_RHT_SR, masks[k % 64], SEED, k,
                                            amax=amaxes[k % nbuf], out=tiled_outs[k % nbuf])
    tiled_ms = time_graph(capture(tiled, 0, args.steps)) / args.steps

    def step_then_swizzle(k):
        step(k)
        Q.nvfp4_swizzle_scales(outs[k % nbuf].scales, out=tiled_outs[k % nbuf].scales)

    sts_ms = time_graph(capture(step_then_swizzle, 0, args.steps)) / args.steps
    del tiled_outs
    # single-launch durations (p10 / median / p90) of the step and of the quantize kernel, and the streaming ceiling
    n_pct = min(PERCENTILE_LAUNCHES, max(args.steps, 10))
    step_pct = launch_percentiles(lambda k: step(args.warmup + args.steps + k), n_pct)
    quant_pct = launch_percentiles(quant, n_pct)
    ceiling = stream_ceiling(xs, outs, args.steps)
    configs = config_figures(Q, W, dev, args.config_launches) if args.config_launches else {}

    result = {
        "metric": "effective GB/s (bf16 in + fp4/scale out) and % of HBM peak, 8192x4096 RHT+SR",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_eager": round(eager_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "input_dtype": "bf16",
        "output_dtype": "e2m1 codes + e4m3 block scales + f32 global scale",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "rows": ROWS, "cols": COLS, "orient": "colwise", "block": "1x16",
                   "rht": True, "rounding": "philox_sr", "gmode": "per_tensor",
                   "step": "nvfp4_amax_quantize (single read)", "input_buffers": nbuf},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {"kernel": "k_amax_quant_colwise4<RHT+SR> (single read: amax + quantize)", "bound": "hbm",
                     "achieved": round(value, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "algorithmic_bytes_per_launch": step_bytes, "mean_launch_ms": round(ms_per_step, 5),
                     "event_bracketed_launch_us": step_pct,
                     "frac_of_stream_ceiling": round(value / ceiling["gbs"], 4)},
        "extra": {
            "gemm_ready_step": {"tiled_scales_in_kernel_us": round(1e3 * tiled_ms, 2),
                                "step_then_nvfp4_swizzle_scales_us": round(1e3 * sts_ms, 2),
                                "note": "the step with scales written in the FP4 GEMM's tiled layout by the kernel, "
                                        "and the row-major step followed by the separate re-layout"},
            "stream_ceiling": ceiling,
            "two_pass_step_ms": round(two_ms, 5),
            "two_pass_step_gbs": round(step_bytes / (two_ms * 1e-3) / 1e9, 2),
            "quantize_kernel_ms": round(q_ms, 5),
            "quantize_kernel_gbs": round(q_gbs, 2),
            "quantize_kernel_frac_of_hbm_peak": round(q_gbs / HBM_PEAK_GBS, 4),
            "quantize_kernel_frac_of_stream_ceiling": round(q_gbs / ceiling["gbs"], 4),
            "quantize_kernel_event_bracketed_launch_us": quant_pct,
            "quantize_kernel_roofline": {"kernel": "k_quant_colwise4<RHT+SR> (quantize only, device-resident amax)",
                                         "bound": "hbm", "achieved": round(q_gbs, 2), "peak": HBM_PEAK_GBS,
                                         "unit": "GB/s", "frac": round(q_gbs / HBM_PEAK_GBS, 4),
                                         "traffic": measured_traffic(QUANT_TRAFFIC_SUMMARY),
                                         "algorithmic_bytes_per_launch": step_bytes,
                                         "mean_launch_ms": round(q_ms, 5)},
            "amax_call_ms": round(amax_ms, 5),
            "amax_call_gbs_read": round(2 * ROWS * COLS / (amax_ms * 1e-3) / 1e9, 2),
            "rowwise_rht_sr_kernel_ms": round(row_ms, 5),
            "rowwise_rht_sr_kernel_gbs": round(step_bytes / (row_ms * 1e-3) / 1e9, 2),
            "pages_context": "~1270 GB/s (~71% of HBM peak) fused RHT+SR kernel on an RTX 5090, shape unstated",
            "configs": configs,
        },
    }
    return result


if __name__ == "__main__":
    main()
