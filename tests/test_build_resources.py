"""Register use of the built kernels (from the compiler's resource-usage remarks that the build records): no
kernel may spill vector registers or use scratch memory (a spill in the hot loop turns into memory traffic per
block; scalar registers spilled into vector-register lanes cost no memory), and the kernels that hold a whole tile
in registers must keep one 1024-thread workgroup per CU (4 waves per SIMD)."""
import os

import pytest

from nvfp4_quantization_amd import _build

pytestmark = pytest.mark.skipif(not os.path.exists(_build.RESOURCE_REPORT),
                                reason="no build record (run the build first)")


def kernels():
    rows = []
    with open(_build.RESOURCE_REPORT) as f:
        for line in f:
            rows.append(dict(kv.split("=", 1) for kv in line.split()))
    return rows


def test_every_kernel_is_listed():
    names = " ".join(r["name"] for r in kernels())
    for k in ("k_amax_quant_colwise4", "k_amax_quant_rowwise", "k_quant_colwise4", "k_quant_colwise", "k_quant_rowwise",
              "k_quant_16x16",
              "k_quant_4o6_rows", "k_quant_4o6_tensor", "k_dequantize", "k_amax_colwise", "k_amax_rowwise_tensor",
              "k_quant_4o6_16x16", "k_swizzle_scales", "k_quant_rowwise_tiled", "k_dequantize_fused",
              "k_quant_grouped", "k_quant_4o6_grouped"):
        assert k in names, k


def test_no_spills_to_memory():
    spilled = [(r["name"], r.get("vgpr_spill"), r.get("scratch")) for r in kernels()
               if int(r.get("vgpr_spill", 0)) or int(r.get("scratch", 0))]
    assert not spilled, spilled


def test_tile_kernels_keep_four_waves_per_simd():
    for r in kernels():
        if any(k in r["name"] for k in ("k_quant_colwiseI", "k_quant_16x16")):
            assert int(r["vgpr"]) <= 128 and int(r["occupancy"]) >= 4, r


def test_narrow_column_kernels_keep_eight_waves_per_simd():
    """The narrow-tile column-wise kernels hold 16 rows x 4 columns per lane in 64 registers so that two 1024-thread
    workgroups fit a CU; the single-read launcher relies on it (up to two workgroups per CU, all resident)."""
    seen = 0
    for r in kernels():
        if "k_quant_colwise4" in r["name"] or "k_amax_quant_colwise4" in r["name"]:
            assert int(r["vgpr"]) <= 64 and int(r["occupancy"]) >= 8, r
            assert int(r["lds"]) <= 80 * 1024, r
            seen += 1
    assert seen == 6


def test_looping_grids_fit_their_occupancy():
    """Kernels whose launchers size a looping grid to a fixed number of resident workgroups per CU must keep that
    occupancy: k_quant_4o6_16x16 two 1024-thread workgroups (8 waves per SIMD), k_quant_rowwise_tiled three
    512-thread ones (6 waves per SIMD), the single-read row-wise kernel one 1024-thread workgroup (4)."""
    need = {"k_quant_4o6_16x16": 8, "k_quant_rowwise_tiled": 6, "k_amax_quant_rowwise": 4}
    seen = set()
    for r in kernels():
        for k, occ in need.items():
            if k in r["name"]:
                assert int(r["occupancy"]) >= occ, r
                seen.add(k)
    assert seen == set(need)
