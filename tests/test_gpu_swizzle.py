"""GPU parity of the FP4 GEMM's tiled scale layout (nvfp4_swizzle_scales) against the CPU oracle, byte for byte.

Scale matrices come from a seeded generator or from the oracle's own quantization; shapes cover single and many
tiles, ragged row and column tiles (zero padding), scale counts per row that are not a multiple of 4 and a scale
pointer that is not 4-byte aligned (the byte-load path), and the 8192 x 4096 activation's scales.  The output
buffer is filled with 0xAB first, so that padding left unwritten would show.
"""
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
    Q.binding.lib()
    O.lib()


def say(*a):
    print("[case]", *a, flush=True)


def run(s_host, byte_offset=0):
    rv, nb = s_host.shape
    big = torch.zeros(rv * nb + 64, dtype=torch.uint8, device="cuda")
    view = big[byte_offset:byte_offset + rv * nb].view(rv, nb)
    view.copy_(torch.from_numpy(s_host))
    out = torch.full((Q.nvfp4_swizzled_scales_size(rv, nb),), 0xAB, dtype=torch.uint8, device="cuda")
    Q.nvfp4_swizzle_scales(view, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("shape", [(1, 1), (32, 4), (127, 3), (128, 4), (129, 5), (300, 65), (256, 64), (1000, 17),
                                   (4096, 512)])
@pytest.mark.parametrize("byte_offset", [0, 1])
def test_random_scales(shape, byte_offset):
    say("swizzle", shape, "offset", byte_offset)
    s = np.random.default_rng(shape[0] * 31 + shape[1]).integers(0, 256, shape, dtype=np.uint8)
    np.testing.assert_array_equal(run(s, byte_offset), O.swizzle_scales(s))


def test_empty():
    out = torch.full((16,), 0xAB, dtype=torch.uint8, device="cuda")
    Q.nvfp4_swizzle_scales(torch.empty((0, 8), dtype=torch.uint8, device="cuda"), out=out)
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == 0xAB).all() and Q.nvfp4_swizzled_scales_size(0, 8) == 0


def test_quantized_activation_8192x4096():
    """Row-wise RN quantization followed by the tiled layout, on both sides."""
    x = W.make("fprop_rn_8192x4096")
    say("swizzle of the 8192x4096 row-wise RN scales")
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    a = Q.nvfp4_amax(xd, Q.ROWWISE, Q.G_PER_TENSOR)
    qd, _ = Q.nvfp4_quantize_rn(xd, a, Q.BLOCK_1X16, Q.ROWWISE, Q.G_PER_TENSOR)
    sw = Q.nvfp4_swizzle_scales(qd.scales)
    torch.cuda.synchronize()
    _, so, _ = O.quantize_1x16(x, O.amax(x), O.MODE_RN)
    np.testing.assert_array_equal(sw.cpu().numpy(), O.swizzle_scales(so))
