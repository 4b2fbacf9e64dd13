"""Pins for the oracle's Philox4x32-10 generator and its 16-point Random Hadamard Transform (CPU only).

Philox is pinned to the published known-answer vectors and cross-checked on random counters and keys against the
open-source rocRAND implementation (compiled for the host).  The RHT is pinned to the Sylvester Hadamard matrix
written out from its definition H[i][j] = (-1)^popcount(i & j) and to the exact error bound of the binary32
butterfly.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from conftest import read_golden


def test_philox_known_answers(oracle):
    rows = read_golden("philox4x32_10_kat.txt")
    assert len(rows) == 3
    for r in rows:
        v = [int(h, 16) for h in r]
        assert oracle.philox4x32_10(v[0:4], v[4:6]) == v[6:10]


_ROCRAND_PROBE = r"""
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
struct Engine : rocrand_device::philox4x32_10_engine {
    uint4 run(uint4 c, uint2 k) { return ten_rounds(c, k); }
};
int main() {
    Engine e;
    unsigned c0, c1, c2, c3, k0, k1;
    while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        uint4 r = e.run(uint4{c0, c1, c2, c3}, uint2{k0, k1});
        std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
"""


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand) and os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
            return cand
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc / rocRAND headers not available")
def test_philox_matches_rocrand_on_random_inputs(oracle):
    rng = np.random.default_rng(5)
    cases = rng.integers(0, 2**32, size=(500, 6), dtype=np.uint64)
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "p.cpp"), os.path.join(d, "p")
        with open(src, "w") as f:
            f.write(_ROCRAND_PROBE)
        subprocess.run([_hipcc(), "-x", "hip", "--offload-arch=gfx950", "-O1", src, "-o", exe], check=True,
                       capture_output=True)
        inp = "\n".join(" ".join("%x" % v for v in row) for row in cases)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout.split("\n")
    for row, line in zip(cases, out):
        want = [int(h, 16) for h in line.split()]
        assert oracle.philox4x32_10([int(v) for v in row[:4]], [int(v) for v in row[4:]]) == want


def test_block_random_bytes_layout(oracle):
    """Reading: key = (seed lo, seed hi), counter = (block lo, block hi, offset lo, offset hi), bytes taken
    little-endian from words 0..3."""
    seed, offset, n = 0x0123456789ABCDEF, 0xFEDCBA9876543210, 0x00000003_80000001
    words = oracle.philox4x32_10([n & 0xFFFFFFFF, n >> 32, offset & 0xFFFFFFFF, offset >> 32],
                                 [seed & 0xFFFFFFFF, seed >> 32])
    expect = np.array(words, dtype="<u4").view(np.uint8)
    np.testing.assert_array_equal(oracle.block_random_bytes(seed, offset, n), expect)


def test_random_bytes_are_uniform(oracle):
    """Byte histogram of 40,000 blocks (640,000 bytes) passes a chi-square test at the 1e-4 level."""
    from scipy.stats import chi2
    counts = np.zeros(256)
    for n in range(40_000):
        counts += np.bincount(oracle.block_random_bytes(1234, 7, n), minlength=256)
    exp = counts.sum() / 256
    stat = ((counts - exp) ** 2 / exp).sum()
    assert stat < chi2.ppf(1 - 1e-4, 255)


def _sylvester16():
    return np.array([[(-1) ** bin(i & j).count("1") for j in range(16)] for i in range(16)], dtype=np.float64)


def test_sylvester_matrix_is_hadamard():
    H = _sylvester16()
    np.testing.assert_array_equal(H @ H.T, 16 * np.eye(16))


def test_rht_of_unit_vectors_is_quarter_hadamard_column(oracle):
    H = _sylvester16()
    for j in range(16):
        e = np.zeros(16, np.float32)
        e[j] = 1.0
        np.testing.assert_array_equal(oracle.rht16(e, 0), (H[:, j] / 4).astype(np.float32))
        # sign mask bit j negates input element j before the transform
        np.testing.assert_array_equal(oracle.rht16(e, 1 << j), (-H[:, j] / 4).astype(np.float32))
        np.testing.assert_array_equal(oracle.rht16(e, 0xFFFF ^ (1 << j)), (H[:, j] / 4).astype(np.float32))


def test_rht_is_its_own_inverse_on_small_integers(oracle):
    """(H/4)(H/4) = I; with small integer inputs every intermediate is exact."""
    rng = np.random.default_rng(2)
    for _ in range(200):
        v = rng.integers(-1024, 1025, size=16).astype(np.float32)
        np.testing.assert_array_equal(oracle.rht16(oracle.rht16(v, 0), 0), v)


def test_rht_matches_dense_definition_within_rounding(oracle):
    """y = (1/4) H diag(s) v in binary64 versus the binary32 butterfly: four roundings per output, so
    |y32 - y64| <= 4 * 2^-24 * (1/4) * sum|v| (times a hair for the second-order terms)."""
    H = _sylvester16()
    rng = np.random.default_rng(9)
    for trial in range(2000):
        v = (rng.standard_normal(16) * np.exp(3 * rng.standard_normal(16))).astype(np.float32)
        mask = int(rng.integers(0, 1 << 16))
        s = np.array([-1.0 if (mask >> i) & 1 else 1.0 for i in range(16)])
        exact = H @ (s * v.astype(np.float64)) / 4
        got = oracle.rht16(v, mask).astype(np.float64)
        bound = 4 * 2.0**-24 * np.abs(v.astype(np.float64)).sum() / 4 * 1.0001
        assert np.all(np.abs(got - exact) <= bound), trial


def test_rht_orthonormal_energy(oracle):
    rng = np.random.default_rng(4)
    v = rng.standard_normal(16).astype(np.float32)
    y = oracle.rht16(v, 0xA5C3)
    assert abs(np.sum(y.astype(np.float64) ** 2) - np.sum(v.astype(np.float64) ** 2)) < 1e-5 * np.sum(v**2)


def test_rht_propagates_nan_and_inf(oracle):
    v = np.ones(16, np.float32)
    v[5] = np.nan
    assert np.all(np.isnan(oracle.rht16(v, 0x1234)))
    v[5] = np.inf
    y = oracle.rht16(v, 0)
    assert np.all(np.isinf(y))
