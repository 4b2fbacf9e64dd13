"""The Python binding refuses caller-supplied buffers of the wrong dtype or size before anything reaches the C ABI
(no GPU needed: the library is replaced by a stand-in that fails if reached, and CPU tensors stand in for device
tensors).  A wrong-sized output,
amax or decode buffer would otherwise be read or written past its end by the kernels."""
import pytest
import torch

import nvfp4_quantization_amd as Q
from nvfp4_quantization_amd import binding as B

X = torch.zeros((32, 64), dtype=torch.int16)


class _NoLib:
    """Stands in for the HIP library: reaching it means a check was missed."""
    def __getattr__(self, name):
        if name == "nvfp4_swizzled_scales_size":        # host-only size helper
            return lambda rv, nb: ((rv + 127) // 128) * 128 * ((nb + 3) // 4) * 4
        def reached(*args):
            raise AssertionError(f"{name} reached: a buffer check is missing")
        return reached


@pytest.fixture(autouse=True)
def _no_gpu(monkeypatch):
    monkeypatch.setattr(B, "lib", lambda: _NoLib())
    monkeypatch.setattr(B, "_bf16", lambda x: 0x10000)   # x itself is checked by the device test; not here
    monkeypatch.setattr(B, "_f32", lambda x: 0x10000)
    # CPU tensors pass for device tensors here, so that each check under test is the first one to fail
    monkeypatch.setattr(torch.Tensor, "is_cuda", property(lambda self: True))


def out(rv, cv, gmode=0, codes=None, scales=None, g=None, layout=0):
    return B.Quantized(codes if codes is not None else torch.zeros((rv, cv // 2), dtype=torch.uint8),
                       scales if scales is not None else torch.zeros((rv, cv // 16), dtype=torch.uint8),
                       g if g is not None else torch.zeros((rv if gmode else 1,), dtype=torch.float32), layout)


def test_output_buffers_checked():
    with pytest.raises(ValueError, match="codes"):
        B._out(out(32, 64, codes=torch.zeros((32, 31), dtype=torch.uint8)), 32, 64, 0)
    with pytest.raises(TypeError, match="codes"):
        B._out(out(32, 64, codes=torch.zeros((32, 32), dtype=torch.int16)), 32, 64, 0)
    with pytest.raises(ValueError, match="scales"):
        B._out(out(32, 64, scales=torch.zeros((32, 3), dtype=torch.uint8)), 32, 64, 0)
    with pytest.raises(ValueError, match="g"):
        B._out(out(32, 64, gmode=0), 32, 64, 1)        # a per-tensor g buffer given for per-row g
    with pytest.raises(TypeError, match="g"):
        B._out(out(32, 64, g=torch.zeros((1,), dtype=torch.float64)), 32, 64, 0)
    with pytest.raises(ValueError, match="layout"):
        B._out(out(32, 64, layout=7), 32, 64, 0)
    with pytest.raises(ValueError, match="contiguous"):
        B._out(out(32, 64, codes=torch.zeros((32, 64), dtype=torch.uint8)[:, ::2]), 32, 64, 0)


def test_tiled_scales_size_checked():
    n = Q.nvfp4_swizzled_scales_size(32, 4)
    assert n == 128 * 4
    with pytest.raises(ValueError, match="scales"):
        B._out(out(32, 64, scales=torch.zeros((32 * 4,), dtype=torch.uint8), layout=1), 32, 64, 0)


def test_entry_points_check_amax_and_outputs():
    a1 = torch.zeros((1,), dtype=torch.float32)
    with pytest.raises(ValueError, match="amax"):
        Q.nvfp4_quantize_sr(X, a1, 1, 2, Q.ROWWISE, Q.G_PER_ROW, out=out(32, 64, 1))   # per-row needs 32 entries
    with pytest.raises(ValueError, match="amax"):                                          # view rows = cols = 64
        Q.nvfp4_quantize_rht_sr(X, torch.zeros((32,), dtype=torch.float32), 3, 1, 2, Q.COLWISE, Q.G_PER_ROW,
                                out=out(64, 32, 1))
    with pytest.raises(ValueError, match="codes"):
        Q.nvfp4_quantize_rn(X, a1, Q.BLOCK_1X16, Q.ROWWISE, 0, row_out=out(32, 32))       # codes for 32 columns
    with pytest.raises(TypeError, match="amax"):
        Q.nvfp4_quantize_4o6(X, torch.zeros((32,), dtype=torch.float16), Q.G_PER_ROW, out=out(32, 64, 1))
    with pytest.raises(ValueError, match="amax"):
        Q.nvfp4_amax(X, Q.ROWWISE, Q.G_PER_ROW, amax=torch.zeros((1,), dtype=torch.float32))
    with pytest.raises(ValueError, match="amax"):
        Q.nvfp4_amax_quantize(X, Q.COLWISE, Q.ROUND_RHT_SR, amax=torch.zeros((2,), dtype=torch.float32),
                              out=out(64, 32))


def test_decode_buffers_checked():
    o = out(32, 64, 1)
    with pytest.raises(ValueError, match="y"):
        Q.nvfp4_dequantize(o.codes, o.scales, o.g, Q.G_PER_ROW, y=torch.zeros((32, 32), dtype=torch.float32))
    with pytest.raises(TypeError, match="y"):
        Q.nvfp4_dequantize(o.codes, o.scales, o.g, Q.G_PER_ROW, y=torch.zeros((32, 64), dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="y"):
        Q.nvfp4_dequantize_fused(o.codes, o.scales, o.g, Q.G_PER_ROW, out_bf16=True,
                                 y=torch.zeros((32, 64), dtype=torch.float32))
    with pytest.raises(TypeError, match="y"):
        Q.nvfp4_dequantize_fused(o.codes, o.scales, o.g, Q.G_PER_ROW, out_bf16=False,
                                 y=torch.zeros((32, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="g"):
        Q.nvfp4_dequantize(o.codes, o.scales, torch.zeros((1,), dtype=torch.float32), Q.G_PER_ROW)
    with pytest.raises(ValueError, match="scales"):
        Q.nvfp4_dequantize(o.codes, torch.zeros((32, 3), dtype=torch.uint8), o.g, Q.G_PER_ROW)


def test_grouped_items_checked():
    with pytest.raises(ValueError, match="amax"):
        Q.nvfp4_quantize_grouped([X], [torch.zeros((3,), dtype=torch.float32)], Q.ROUND_RN, Q.G_PER_ROW,
                                 outs=[out(32, 64, 1)])
    with pytest.raises(ValueError, match="amax"):
        Q.nvfp4_amax_grouped([X, X], Q.G_PER_ROW, amaxes=[torch.zeros((32,)), torch.zeros((1,))])
