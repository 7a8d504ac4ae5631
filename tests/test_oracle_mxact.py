"""Pins of the MX activation oracle (oracle/mxact.py) against brute force, closed forms and
special cases that reduce to the weight-only product."""
import numpy as np
import pytest

import synth
from oracle import gemm as ogemm
from oracle import mx as omx
from oracle import mxact as oa
from oracle import nvfp4 as onv

# every finite E4M3 value with its byte, both signs, from the bit fields (not from the encoder)
_BYTES = np.array([b for b in range(256) if (b & 0x7F) != 0x7F])
_VALS = onv.e4m3_decode(_BYTES)


def brute_e4m3(x):
    """Nearest finite E4M3 value by scanning all 254 encodings; ties to the even fraction; |x| >= 448
    saturates; the sign bit of x is kept on zero."""
    x = np.asarray(x, np.float64)
    d = np.abs(x[..., None] - _VALS)
    # both zeros are at distance |x|: keep the one with x's sign
    zero_wrong_sign = (_VALS == 0) & (np.signbit(_VALS) != np.signbit(x)[..., None])
    d = np.where(zero_wrong_sign, np.inf, d)
    best = d == d.min(axis=-1, keepdims=True)
    even = (_BYTES & 1) == 0
    pick = np.where((best & even).any(-1), np.argmax(best & even, -1), np.argmax(best, -1))
    out = _BYTES[pick].astype(np.uint8)
    sat = np.abs(x) >= 448
    return np.where(sat, np.where(np.signbit(x), 0xFE, 0x7E), out).astype(np.uint8)


def test_signed_encoder_matches_brute_force_on_a_dense_sweep():
    """Every bf16 value in [2^-12, 600) (both signs) and every E4M3 midpoint."""
    bits = np.arange(0x3980, 0x4416, dtype=np.uint32)        # bf16 2^-12 .. ~600
    pos = (bits << 16).view(np.float32).astype(np.float64)
    table = onv.E4M3_TABLE[:127]
    mids = (table[:-1] + table[1:]) / 2
    x = np.concatenate([pos, -pos, mids, -mids, [0.0, -0.0, 2.0 ** -10, -(2.0 ** -10)]])
    assert np.array_equal(oa.e4m3_signed_encode(x), brute_e4m3(x))


def _block_rows(seed, nblocks=400):
    r = synth.rng(61, 1, seed)
    v = r.standard_normal((nblocks, 32)) * 2.0 ** r.integers(-40, 40, (nblocks, 1))
    return synth.f32_to_bf16_bits(v.astype(np.float32))


def test_scale_rule_and_block_maximum():
    """e = floor(log2 amax) - 8: the block maximum decodes into [256, 448] * 2^e, and every
    element is the nearest grid point of v / 2^e (brute force)."""
    xb = _block_rows(0)
    codes, scales, flags = oa.quantize_fp8(xb.reshape(-1, 32))
    assert flags == 0
    v = oa.bf16_to_f64(xb).reshape(-1, 32)
    e = scales.astype(np.int64)[:, 0] - 127
    amax = np.abs(v).max(axis=1)
    assert np.all(2.0 ** (e + 8) <= amax) and np.all(amax < 2.0 ** (e + 9))
    vals = onv.e4m3_decode(codes)
    top = np.abs(vals[np.arange(len(v)), np.abs(v).argmax(axis=1)])
    assert np.all((top >= 256) & (top <= 448))
    x = v / 2.0 ** e[:, None]
    assert np.array_equal(codes, brute_e4m3(x))


def test_error_within_half_a_step():
    xb = _block_rows(1)
    codes, scales, _ = oa.quantize_fp8(xb.reshape(-1, 32))
    v = oa.bf16_to_f64(xb).reshape(-1, 32)
    s = 2.0 ** (scales.astype(np.float64) - 127)
    x = np.abs(v) / s
    # E4M3 spacing at |x|: 2^(floor(log2 x) - 3) in the normal range, 2^-9 below 2^-6
    step = np.where(x < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(x, 1e-300))) - 3))
    err = np.abs(onv.e4m3_decode(codes) - v / s)
    assert np.all((err <= step / 2 * (1 + 1e-12)) | (x >= 448))


def test_hand_built_blocks():
    rows = np.zeros((6, 32), np.float32)
    rows[0, 0] = 256.0                   # e = 0: x = v exactly
    rows[0, 1:8] = [1.0625, 1.1875, 17.0, 19.0, 0.001953125 * 1.5, 2.0 ** -10, -(2.0 ** -10)]
    rows[1, 0] = 480.0                   # e = 0 (floor(log2 480) = 8): 480 saturates to 448
    rows[1, 1] = -470.0
    rows[2, 3] = -0.0                    # all-zero block with a signed zero
    rows[3, :] = 3.0                     # amax 3: e = 1 - 8 = -7, x = 384
    rows[4, 0] = 2.0 ** -133             # smallest bf16 subnormal: e clamps at -127
    rows[5, 5] = np.nan
    codes, scales, flags = oa.quantize_fp8(synth.f32_to_bf16_bits(rows))
    assert flags == oa.FLAG_NONFINITE
    assert scales[0, 0] == 127 and scales[1, 0] == 127 and scales[3, 0] == 120
    assert list(codes[0, :8]) == [0x78, 0x38, 0x3A, 0x58, 0x5A, 0x02, 0x00, 0x80]
    assert codes[1, 0] == 0x7E and codes[1, 1] == 0xFE
    assert scales[2, 0] == 0 and codes[2, 3] == 0x80 and np.all(np.delete(codes[2], 3) == 0)
    assert np.all(codes[3] == 0x7C)          # 384 = 1.5 * 2^8: exponent field 15, fraction 4
    assert scales[4, 0] == 0 and codes[4, 0] == onv.e4m3_encode(2.0 ** -6)   # 2^-133 * 2^127
    assert scales[5, 0] == 0xFF and np.all(codes[5] == 0)


def test_tie_cases_round_to_even():
    """Midpoints between E4M3 neighbours at scale 2^0 go to the even fraction: 1.0625 between
    1.0 (0x38) and 1.125 (0x39) -> 0x38; 1.1875 between 1.125 and 1.25 -> 1.25 (0x3A); 17 between
    16 and 18 -> 16 (0x58); 19 between 18 and 20 -> 20 (0x5A)."""
    x = np.array([1.0625, 1.1875, 17.0, 19.0, -1.0625])
    assert list(oa.e4m3_signed_encode(x)) == [0x38, 0x3A, 0x58, 0x5A, 0xB8]


def test_idempotent_on_its_grid():
    xb = _block_rows(2)
    codes, scales, _ = oa.quantize_fp8(xb.reshape(-1, 32))
    deq = oa.dequantize(codes, scales, oa.FMT_FP8, 32)
    # the dequantized values are bf16 values (<= 4 significant bits, exponents in range)
    back = synth.f32_to_bf16_bits(deq.astype(np.float32))
    assert np.array_equal(oa.bf16_to_f64(back), deq)
    c2, s2, _ = oa.quantize_fp8(back)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


def test_fp4_activations_are_the_weight_codec():
    xb = synth.activations(62, 0, 7, 256)
    c, s, f = oa.quantize_fp4(xb)
    rc, rs, rf = omx.quantize(oa.bf16_to_f64(xb).astype(np.float32))
    assert np.array_equal(c, rc) and np.array_equal(s, rs) and f == rf == 0
    assert omx.storage_bits_per_value(7, 256) == 4.25


def test_gemm_one_hot_and_matmul():
    n, k = 48, 256
    wc, ws, _ = omx.quantize(synth.weights(63, 0, n, k))
    wq = omx.dequantize(wc, ws, k)
    for fmt in (oa.FMT_FP8, oa.FMT_FP4):
        x = np.zeros((3, k), np.float32)
        x[0, 5] = 1.0
        x[1, 200] = -2.0
        x[2, 31] = 0.5
        ac, asc, _ = oa.quantize(synth.f32_to_bf16_bits(x), fmt)
        y = oa.gemm(wc, ws, n, k, ac, asc, fmt)
        assert np.array_equal(y[0], wq[:, 5]) and np.array_equal(y[1], -2 * wq[:, 200])
        assert np.array_equal(y[2], 0.5 * wq[:, 31])
        xb = synth.activations(63, fmt, 5, k)
        ac, asc, _ = oa.quantize(xb, fmt)
        np.testing.assert_allclose(oa.gemm(wc, ws, n, k, ac, asc, fmt),
                                   oa.dequantize(ac, asc, fmt, k) @ wq.T, rtol=1e-12, atol=1e-300)


@pytest.mark.parametrize("fmt", [oa.FMT_FP8, oa.FMT_FP4])
def test_on_grid_activations_reduce_to_the_weight_only_product(fmt):
    """Activations that are already MX values (one E2M1 / E4M3 grid value times a block power of
    two, the block maximum at the top binade) quantize without error, so the W4A8 / W4A4 product
    equals the weight-only fp64 product of the same bf16 activations."""
    n, k, m = 40, 512, 6
    wc, ws, _ = omx.quantize(synth.weights(64, fmt, n, k))
    r = synth.rng(64, 1, fmt)
    if fmt == oa.FMT_FP8:
        grid = onv.e4m3_decode(np.arange(0x08, 0x7F))             # normal E4M3 values
        top = 448.0
    else:
        grid = omx._E2M1[1:8]
        top = 6.0
    vals = r.choice(grid, (m, k)) * r.choice([-1.0, 1.0], (m, k))
    vals[:, ::32] = top                                         # every block's maximum
    scale = 2.0 ** r.integers(-20, 20, (m, k // 32)).repeat(32, axis=1)
    x = (vals * scale).astype(np.float32)
    xb = synth.f32_to_bf16_bits(x)
    assert np.array_equal(oa.bf16_to_f64(xb), x.astype(np.float64))
    ac, asc, _ = oa.quantize(xb, fmt)
    assert np.array_equal(oa.dequantize(ac, asc, fmt, k), x.astype(np.float64))
    np.testing.assert_allclose(oa.gemm(wc, ws, n, k, ac, asc, fmt), ogemm.verify_gemm(wc, ws, n, k, xb),
                               rtol=1e-12, atol=1e-300)


def test_activation_quantization_error_is_the_expected_size():
    """On N(0,1) activations, MX-FP8 changes the product by ~1-3% relative L2 and MX-FP4 by ~10-20%
    (the reason the weight-only path keeps bf16 activations)."""
    n, k, m = 256, 2048, 8
    wc, ws, _ = omx.quantize(synth.weights(65, 0, n, k))
    xb = synth.activations(65, 0, m, k)
    ref = ogemm.verify_gemm(wc, ws, n, k, xb)
    rel = {}
    for fmt in (oa.FMT_FP8, oa.FMT_FP4):
        ac, asc, _ = oa.quantize(xb, fmt)
        y = oa.gemm(wc, ws, n, k, ac, asc, fmt)
        rel[fmt] = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert 0.005 < rel[oa.FMT_FP8] < 0.05, rel
    assert 0.05 < rel[oa.FMT_FP4] < 0.3, rel
