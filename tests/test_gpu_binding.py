"""The Python binding refuses wrong output buffers before any launch.

The C ABI sees only pointers, so a caller-supplied output of the wrong shape or
dtype would be written past its end. Every such argument is checked in the
binding and raises (TypeError for dtype / device / layout, ValueError for shape)
before the library is called; nothing here reaches a kernel.
"""
import pytest
import torch

import mx_fp4_weight_amd as mxs

pytestmark = pytest.mark.gpu


def z(shape, dtype):
    return torch.zeros(shape, dtype=dtype, device="cuda")


def test_quantize_outputs_checked():
    w = z((32, 64), torch.float32)
    with pytest.raises(ValueError):
        mxs.mxfp4_quantize(w, codes=z((32, 31), torch.uint8))
    with pytest.raises(ValueError):
        mxs.mxfp4_quantize(w, scales=z((31, 2), torch.uint8))
    with pytest.raises(TypeError):
        mxs.mxfp4_quantize(w, codes=z((32, 32), torch.int8))
    with pytest.raises(ValueError):
        mxs.mxfp4_quantize(w, dev_flags=z((0,), torch.int32))
    with pytest.raises(ValueError):
        mxs.nvfp4_quantize(w, scales=z((32, 2), torch.uint8))
    with pytest.raises(ValueError):
        mxs.nvfp4_quantize(w, global_scale=z((2,), torch.float32))


def test_gemm_outputs_checked():
    c, s, x = z((16, 256), torch.uint8), z((16, 16), torch.uint8), z((5, 512), torch.bfloat16)
    with pytest.raises(ValueError):
        mxs.mxfp4_verify_gemm(c, s, x, y=z((5, 15), torch.float32))
    with pytest.raises(TypeError):
        mxs.mxfp4_verify_gemm(c, s, x, y=z((5, 16), torch.float64))
    nvs, g = z((16, 32), torch.uint8), z((1,), torch.float32)
    with pytest.raises(ValueError):
        mxs.nvfp4_verify_gemm(c, nvs, g, x, y=z((4, 16), torch.float32))
    ac, asc = z((5, 512), torch.uint8), z((5, 16), torch.uint8)
    with pytest.raises(ValueError):
        mxs.mx_verify_gemm_act(c, s, ac, asc, mxs.ACT_FP8, y=z((16, 5), torch.float32))
    with pytest.raises(ValueError):
        mxs.mx_quantize_act(x, mxs.ACT_FP4, codes=z((5, 512), torch.uint8))
    with pytest.raises(ValueError):
        mxs.mx_quantize_act(x, 3)


def test_accept_outputs_checked():
    b, kd, v = 2, 3, 64
    t, d = z((b, kd + 1, v), torch.float32), z((b, kd, v), torch.float32)
    tok, u = z((b, kd), torch.int32), z((b, kd + 1), torch.float32)
    with pytest.raises(ValueError):
        mxs.spec_accept(t, d, tok, u, out_tokens=z((b, kd), torch.int32))
    with pytest.raises(TypeError):
        mxs.spec_accept(t, d, tok, u, out_num=z((b,), torch.int64))
    with pytest.raises(ValueError):
        mxs.spec_accept_sampled(t, d, tok, u, out_num=z((b + 1,), torch.int32))
    with pytest.raises(ValueError):
        mxs.spec_accept_noalloc(t, d, tok, u, z((b, kd + 1), torch.int32), z((1,), torch.int32))
