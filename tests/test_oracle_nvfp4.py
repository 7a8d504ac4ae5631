"""Pins of the NVFP4 oracle (oracle/nvfp4.py): the E4M3 scale format, the two-level quantizer,
the storage rate printed in the lecture, and the fp64 GEMM."""
import numpy as np
import pytest

import synth
from oracle import mx as omx
from oracle import nvfp4 as nv


def test_e4m3_decode_from_the_bit_fields():
    """4 exponent bits (bias 7), 3 fraction bits, subnormals at exponent 0, S.1111.111 = NaN."""
    want = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
            0x3F: 1.875, 0x40: 2.0, 0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}
    for b, v in want.items():
        assert nv.e4m3_decode(b) == v, hex(b)
    assert np.isnan(nv.e4m3_decode(0x7F)) and np.isnan(nv.e4m3_decode(0xFF))
    vals = nv.e4m3_decode(np.arange(127))
    assert np.all(np.diff(vals) > 0)          # non-negative encodings increase with the byte
    assert np.unique(vals).size == 127


def test_e4m3_encode_nearest_ties_even_saturating():
    r = synth.rng(41, 0)
    table = nv.E4M3_TABLE[:127]
    mids = (table[:-1] + table[1:]) / 2
    t = np.concatenate([r.random(5000) * 600, 2.0 ** r.uniform(-14, 10, 5000), mids, table]).astype(np.float32)
    assert np.array_equal(nv.e4m3_encode(t), nv.e4m3_encode_brute(t))
    # every midpoint goes to the neighbour with an even fraction
    enc = nv.e4m3_encode(mids.astype(np.float32))
    assert np.all(enc % 2 == 0)
    assert nv.e4m3_encode(np.float32(1e6)) == 0x7E and nv.e4m3_encode(np.float32(448.0)) == 0x7E
    assert nv.e4m3_encode(np.float32(2.0 ** -10)) == 0 and nv.e4m3_encode(np.float32(2.0 ** -9 * 1.5)) == 2


@pytest.mark.parametrize("n,k", [(4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336), (8192, 28672),
                                 (128256, 8192)])
def test_storage_is_four_and_a_half_bits(n, k):
    """(16·4 + 8)/16 = 4.5 bits per value counting the block scale (the lecture's formula)."""
    bytes_ = n * k // 2 + n * k // nv.BLOCK
    assert 8 * bytes_ / (n * k) == 4.5


def _quant(seed, n=64, k=256, sigma=0.02):
    w = synth.weights(seed, 0, n, k, sigma=sigma)
    return w, nv.quantize(w)


def test_global_scale_puts_the_largest_block_at_448():
    w, (codes, scales, g, flags) = _quant(42)
    amax = np.abs(w).max()
    assert g == np.float32(amax / np.float32(2688.0)) and flags == 0
    r, c = np.unravel_index(np.argmax(np.abs(w)), w.shape)
    assert scales[r, c // 16] == 0x7E
    # and that block's largest value gets the largest code (6)
    code = omx.unpack_nibbles(codes, w.shape[1])[r, c]
    assert code & 7 == 7


def test_block_max_decodes_to_six_times_the_scale():
    """With the scale rounded to E4M3 (relative step <= 1/8), amax / scale lies in (5.6, 6.4):
    the block maximum always gets code 6 (magnitude 7) unless the scale saturated or is subnormal."""
    w, (codes, scales, g, _) = _quant(43, n=128, k=512, sigma=1.0)
    unp = omx.unpack_nibbles(codes, 512).reshape(128, 32, 16)
    blocks = w.reshape(128, 32, 16)
    imax = np.abs(blocks).argmax(axis=-1)
    s = nv.e4m3_decode(scales)
    normal = (scales >= 0x08) & (scales < 0x7E)
    top = np.take_along_axis(unp, imax[..., None], -1)[..., 0] & 7
    assert np.all(top[normal] == 7)
    assert normal.mean() > 0.9


def test_error_within_half_a_grid_step():
    w, (codes, scales, g, _) = _quant(44, n=96, k=320, sigma=0.5)
    wq = nv.dequantize(codes, scales, g)
    d = (nv.e4m3_decode(scales) * np.float64(g)).repeat(16, axis=1)
    x = np.abs(w.astype(np.float64) / d)
    # grid step around |x|: 0.5 below 2, 1 in [2, 4), 2 above; half of it, plus saturation above 6
    half = np.where(x < 2, 0.25, np.where(x < 4, 0.5, 1.0)) * d
    err = np.abs(w - wq)
    assert np.all((err <= half * (1 + 1e-6)) | (x > 6))


def test_idempotent_on_its_own_output():
    w, (codes, scales, g, _) = _quant(45, n=64, k=256, sigma=0.3)
    wq = nv.dequantize(codes, scales, g).astype(np.float32)
    c2, s2, g2, _ = nv.quantize(wq)
    assert g2 == g and np.array_equal(s2, scales) and np.array_equal(c2, codes)


def test_nonfinite_blocks_refused_and_left_out_of_amax():
    w = synth.weights(46, 0, 8, 64)
    w[2, 5] = np.nan
    w[6, 40] = np.inf
    codes, scales, g, flags = nv.quantize(w)
    assert flags == nv.FLAG_NONFINITE
    assert scales[2, 0] == 0x7F and scales[6, 2] == 0x7F
    assert np.all(omx.unpack_nibbles(codes, 64)[2, :16] == 0)
    fin = np.where(np.isfinite(w), w, 0)
    assert g == np.float32(np.abs(fin).max() / np.float32(2688.0))


def test_zero_tensor_and_signed_zeros():
    w = np.zeros((2, 32), np.float32)
    w[1, 3] = -0.0
    codes, scales, g, flags = nv.quantize(w)
    assert g == 1.0 and flags == 0 and np.all(scales == 0)
    unp = omx.unpack_nibbles(codes, 32)
    assert unp[1, 3] == 8 and unp[0, 3] == 0


def test_gemm_one_hot_and_matmul():
    w, (codes, scales, g, _) = _quant(47, n=48, k=512)
    wq = nv.dequantize(codes, scales, g)
    k = 512
    for col in [0, 15, 16, 255, 511]:
        x = np.zeros((1, k), np.float32)
        x[0, col] = 1.0
        y = nv.verify_gemm(codes, scales, g, synth.f32_to_bf16_bits(x))
        assert np.array_equal(y[0], wq[:, col])
    xb = synth.activations(47, 1, 5, k)
    xf = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_allclose(nv.verify_gemm(codes, scales, g, xb), xf @ wq.T, rtol=1e-12, atol=1e-15)
