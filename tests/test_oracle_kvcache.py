"""Pins of the MX-FP4 KV cache codec oracle (oracle.kvcache).

The codec is the weight codec of oracle.mx applied to every token's head vector, so the
format pins of tests/test_oracle_mx.py (value grid, 4.25 bits, brute-force rounding) carry
over; here: each written entry equals oracle.mx.quantize of that row (its own, independently
pinned quantizer) and nothing else in the cache changes; slots outside the cache are flagged
and skipped; decoding returns the E2M1 x 2^(s-127) values within the O4 error bound; the
footprint is 4.25 / 16 of bf16 exactly.
"""
import numpy as np

import synth
from oracle import kvcache, mx


def test_append_writes_the_rows_it_is_given():
    cap, heads, d = 9, 3, 128
    codes = np.full((cap, heads, d // 2), 0x5A, np.uint8)
    scales = np.full((cap, heads, d // 32), 0x33, np.uint8)
    kv = synth.activations(5, 1, 4 * heads, d).reshape(4, heads, d)
    slots = [7, 0, 3, 12]                      # 12 is outside the cache
    f = kvcache.append(codes, scales, kv, slots)
    assert f == kvcache.FLAG_SLOT_RANGE
    for i, s in enumerate(slots[:3]):
        c, sc, _ = mx.quantize(kvcache.bf16_to_f32(kv[i]))
        assert np.array_equal(codes[s], c) and np.array_equal(scales[s], sc)
    untouched = [s for s in range(cap) if s not in slots]
    assert np.all(codes[untouched] == 0x5A) and np.all(scales[untouched] == 0x33)


def test_bf16_input_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0001, 0x7F7F, 0x8000], np.uint16)
    assert kvcache.bf16_to_f32(bits).tolist() == [1.0, -1.0, float(np.float32(2.0 ** -133)),
                                                   float(np.float32(3.3895313892515355e38)), -0.0]


def test_read_is_within_the_block_bound():
    cap, heads, d = 4, 2, 128
    codes = np.zeros((cap, heads, d // 2), np.uint8)
    scales = np.zeros((cap, heads, d // 32), np.uint8)
    kv = synth.activations(5, 2, cap * heads, d, sigma=3.0).reshape(cap, heads, d)
    assert kvcache.append(codes, scales, kv, range(cap)) == 0
    got = kvcache.read(codes, scales, range(cap))
    x = kvcache.bf16_to_f32(kv).astype(np.float64)
    # |x - x^| <= half the local grid spacing x 2^e (at most 1 x 2^e below 6, 2 x 2^e when a
    # block maximum in (6, 8) x 2^e saturates), and the block max decodes to 4 or 6 x 2^e
    e = scales.astype(np.int64) - 127
    unit = np.repeat(2.0 ** e, 32, axis=-1).reshape(x.shape)
    xs = np.abs(x) / unit
    half = np.where(xs < 2.0, 0.25, np.where(xs < 4.0, 0.5, np.where(xs <= 6.0, 1.0, 2.0)))
    assert np.all(np.abs(x - got) <= half * unit)
    blk = np.abs(got).reshape(cap, heads, d // 32, 32).max(-1) / 2.0 ** e
    assert np.all(np.isin(blk, [4.0, 6.0]))


def test_nonfinite_block_refused():
    codes = np.zeros((2, 1, 16), np.uint8)
    scales = np.zeros((2, 1, 1), np.uint8)
    kv = np.full((1, 1, 32), 0x3F80, np.uint16)
    kv[0, 0, 5] = 0x7F80  # +inf
    assert kvcache.append(codes, scales, kv, [1]) == kvcache.FLAG_NONFINITE
    assert scales[1, 0, 0] == 0xFF and np.all(codes[1] == 0)


def test_footprint():
    assert kvcache.footprint_bytes(1, 8, 128) * 8 / (8 * 128) == 4.25
    assert kvcache.footprint_bytes(1000, 8, 128) / (1000 * 8 * 128 * 2) == 4.25 / 16
