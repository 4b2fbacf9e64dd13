"""The allocation-free entry point: nvfp4_amax_quantize keeps its cross-workgroup scratch (the exchange slots) in a
file-scope device array and allocates nothing, for callers that cannot allocate.  Through the C ABI, two calls in a
row (the second on a smaller input) must equal the two separate calls (nvfp4_amax, then nvfp4_quantize_rht_sr)
bit for bit, and the device's free memory must not change across them.
"""
import sys

import numpy as np
import pytest
import torch

import nvfp4_quantization_amd as Q
from nvfp4_quantization_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    Q.binding.lib()


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def separate_calls(xd, orient, mask, seed, offset):
    a = Q.nvfp4_amax(xd, orient, Q.G_PER_TENSOR, True, mask)
    o = Q.nvfp4_quantize_rht_sr(xd, a, mask, seed, offset, orient, Q.G_PER_TENSOR)
    return a, o


def test_two_calls_second_smaller_equal_the_separate_calls():
    big = W.make("wgrad_colwise_rht_sr_8192x4096")
    small = W.lognormal_gradients(1024, 2048, seed=21)
    cases = [(big, 2, 0), (small, 2, 1)]
    devs = [torch.from_numpy(x.view(np.int16)).cuda() for x, _, _ in cases]
    outs = [(torch.empty((1,), dtype=torch.float32, device="cuda"),
             Q.alloc_out(x.shape[1], x.shape[0], Q.G_PER_TENSOR, "cuda")) for x, _, _ in cases]
    refs = [separate_calls(d, Q.COLWISE, W.sign_mask(s, c), s, c) for d, (_, s, c) in zip(devs, cases)]
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for d, (x, s, c), (a, o) in zip(devs, cases, outs):
        say("no-alloc call", x.shape, "call", c)
        Q.nvfp4_amax_quantize(d, Q.COLWISE, Q.ROUND_RHT_SR, W.sign_mask(s, c), s, c, amax=a, out=o)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0, "the call allocated device memory"
    for (a, o), (ra, ro) in zip(outs, refs):
        assert torch.equal(a.view(torch.int32), ra.view(torch.int32))
        assert torch.equal(o.codes, ro.codes)
        assert torch.equal(o.scales, ro.scales)
        assert torch.equal(o.g.view(torch.int32), ro.g.view(torch.int32))
