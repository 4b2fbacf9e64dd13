"""Seeded synthetic inputs for the NVFP4 quantizer (tests and benchmark).

This module only draws random tensors; it holds none of the quantizer's arithmetic, so the oracle side and the
GPU side can both be fed from it.  All draws use the torch CPU generator with fixed seeds in float32 and are then
cast to bfloat16 (round to nearest even).  Shapes and value distributions follow the workloads the pages
describe: an 8192x4096 activation/gradient tensor (nvfp4-sm120 README, quantizer speed), a 14336x4096 FFN weight
(same README, weight-quant amortisation, d=4096 / h=14336), outlier channels (blog post on polyfilling NVFP4 kernels
for the RTX 5090, section on the RHT: outliers concentrated in a few channels), and a heavy-tailed activation mix
with NaN/Inf for four-over-six (pytorch/ao PR #4852).

Every generator returns the bf16 bit patterns as a contiguous numpy ``uint16`` array of shape [rows, cols].
"""
from __future__ import annotations

import numpy as np
import torch


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def to_bits(x: torch.Tensor) -> np.ndarray:
    """float32 CPU tensor -> bf16 (RNE) -> uint16 bit patterns."""
    return np.ascontiguousarray(x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def outlier_columns(rows: int = 256, cols: int = 1024, seed: int = 0, n_cols: int = 4, factor: float = 50.0):
    """N(0,1) entries; ``n_cols`` columns (a random permutation's first entries) multiplied by ``factor``."""
    g = _gen(seed)
    x = torch.randn(rows, cols, generator=g)
    idx = torch.randperm(cols, generator=g)[:n_cols]
    x[:, idx] *= factor
    return to_bits(x)


def activation_outliers(rows: int = 8192, cols: int = 4096, seed: int = 1, frac: float = 0.01,
                        lo: float = 20.0, hi: float = 100.0):
    """N(0,1) entries; round(frac*cols) columns each scaled by its own U(lo, hi) factor."""
    g = _gen(seed)
    x = torch.randn(rows, cols, generator=g)
    n = max(1, int(round(frac * cols)))
    idx = torch.randperm(cols, generator=g)[:n]
    fac = lo + (hi - lo) * torch.rand(n, generator=g)
    x[:, idx] *= fac
    return to_bits(x)


def lognormal_gradients(rows: int = 8192, cols: int = 4096, seed: int = 2, sigma: float = 2.0):
    """Magnitudes exp(sigma * z), z ~ N(0,1), with independent random signs (Bernoulli 1/2)."""
    g = _gen(seed)
    mag = torch.exp(sigma * torch.randn(rows, cols, generator=g))
    sign = torch.where(torch.rand(rows, cols, generator=g) < 0.5, -1.0, 1.0)
    return to_bits(mag * sign)


def weight_outliers(rows: int = 14336, cols: int = 4096, seed: int = 3, std: float = 0.02, frac: float = 1e-3,
                    factor: float = 30.0):
    """N(0, std^2) weight; round(frac*rows*cols) distinct positions multiplied by ``factor``."""
    g = _gen(seed)
    x = std * torch.randn(rows, cols, generator=g)
    n = int(round(frac * rows * cols))
    pos = torch.randperm(rows * cols, generator=g)[:n]
    x.view(-1)[pos] *= factor
    return to_bits(x)


def heavy_tail_rows(rows: int = 16384, cols: int = 8192, seed: int = 4, frac_special: float = 1e-4,
                    inject: bool = True):
    """Each row is N(0,1) or Student-t(3) (Bernoulli 1/2 per row); t(3) is built as z / sqrt(chi2_3 / 3) from
    seeded normals.  Then round(frac_special*rows*cols) positions (drawn with replacement) are set to NaN, +inf or
    -inf by their draw index modulo 3.  ``inject=False`` returns the same tensor without them."""
    g = _gen(seed)
    is_t = torch.rand(rows, 1, generator=g) < 0.5
    z = torch.randn(rows, cols, generator=g)
    chi2 = torch.zeros(rows, cols)
    for _ in range(3):
        n = torch.randn(rows, cols, generator=g)
        chi2 += n * n
    t3 = torch.randn(rows, cols, generator=g) / torch.sqrt(chi2 / 3.0)
    x = torch.where(is_t, t3, z)
    del z, chi2, t3
    n_special = int(round(frac_special * rows * cols))
    pos = torch.randint(0, rows * cols, (n_special,), generator=g)
    if inject and n_special:
        kinds = torch.arange(n_special) % 3
        vals = torch.tensor([float("nan"), float("inf"), float("-inf")])[kinds]
        x.view(-1)[pos] = vals
    return to_bits(x)


def gaussian(rows: int, cols: int, seed: int, scale: float = 1.0):
    g = _gen(seed)
    return to_bits(scale * torch.randn(rows, cols, generator=g))


def sign_mask(seed: int, call: int) -> int:
    """The 16 random RHT signs for one call, drawn from the CPU generator (seed, call)."""
    g = _gen((int(seed) * 1_000_003 + int(call)) & 0x7FFF_FFFF_FFFF_FFFF)
    return int(torch.randint(0, 1 << 16, (1,), generator=g).item())


# Full-size workloads, by name (sizes as in the pages' workloads).
WORKLOADS = {
    "rht_sr_small_256x1024": dict(fn=outlier_columns, rows=256, cols=1024, seed=0),
    "fprop_rn_8192x4096": dict(fn=activation_outliers, rows=8192, cols=4096, seed=1),
    "wgrad_colwise_rht_sr_8192x4096": dict(fn=lognormal_gradients, rows=8192, cols=4096, seed=2),
    "weight_16x16_14336x4096": dict(fn=weight_outliers, rows=14336, cols=4096, seed=3),
    "four_over_six_16384x8192": dict(fn=heavy_tail_rows, rows=16384, cols=8192, seed=4),
}


def make(name: str, **overrides) -> np.ndarray:
    spec = dict(WORKLOADS[name])
    fn = spec.pop("fn")
    spec.update(overrides)
    return fn(**spec)
