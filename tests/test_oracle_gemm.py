"""Pins of the oracle's verification GEMM.

* exact rational brute force (fractions) on a small case — no library routine;
* one-hot activations return exactly one column of the dequantized weights;
* all-ones codes with unit scale give the row sums of X;
* transposition / row-selection consistency.
"""
from fractions import Fraction

import numpy as np

import synth
from oracle import gemm, mx


def _small_case(m=3, n=5, k=64, seed=11):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    codes, scales, _ = mx.quantize(w)
    x = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    return codes, scales, x, m, n, k


def test_exact_rational_bruteforce():
    codes, scales, x, m, n, k = _small_case()
    y = gemm.verify_gemm(codes, scales, n, k, x)
    flat = codes.reshape(-1)
    for t in range(m):
        for r in range(n):
            acc = Fraction(0)
            for c in range(k):
                byte = int(flat[r * k // 2 + c // 2])
                nib = byte & 0xF if c % 2 == 0 else byte >> 4
                wv = Fraction(mx.e2m1_decode(nib)) * Fraction(2) ** (int(scales[r, c // 32]) - 127)
                xv = Fraction(float(np.array([int(x[t, c]) << 16], np.uint32).view(np.float32)[0]))
                acc += wv * xv
            assert abs(y[t, r] - float(acc)) <= 1e-12 * max(1.0, abs(float(acc)))


def test_one_hot_activations_pick_columns():
    codes, scales, _, _, n, k = _small_case(n=7, k=96)
    w = mx.dequantize(codes, scales, k)
    for col in [0, 1, 31, 32, 95]:
        x = np.zeros((1, k), np.float32)
        x[0, col] = 1.0
        y = gemm.verify_gemm(codes, scales, n, k, synth.f32_to_bf16_bits(x))
        assert np.array_equal(y[0], w[:, col])


def test_all_ones_codes_sum_activations():
    n, k, m = 4, 128, 2
    codes = np.full((n, k // 2), 0x22, np.uint8)      # E2M1 code 2 = 1.0 in both nibbles
    scales = np.full((n, k // 32), 127, np.uint8)     # 2^0
    rng = np.random.default_rng(5)
    x = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    y = gemm.verify_gemm(codes, scales, n, k, x)
    xs = gemm.bf16_bits_to_f64(x).sum(axis=1)
    for t in range(m):
        assert np.allclose(y[t], xs[t], rtol=0, atol=1e-12)


def test_scale_powers_and_signs():
    n, k = 2, 32
    codes = np.zeros((n, k // 2), np.uint8)
    codes[0, 0] = 0x07          # col0 = +6, col1 = +0
    codes[1, 0] = 0xF0          # col0 = +0, col1 = -6
    scales = np.array([[130], [120]], np.uint8)   # 2^3, 2^-7
    x = np.zeros((1, k), np.float32)
    x[0, 0], x[0, 1] = 1.0, 2.0
    y = gemm.verify_gemm(codes, scales, n, k, synth.f32_to_bf16_bits(x))
    assert y[0, 0] == 6 * 8 and y[0, 1] == -6 * 2 * 2.0 ** -7


def test_row_subset_matches_full():
    codes, scales, x, m, n, k = _small_case(n=9, k=64)
    full = gemm.verify_gemm(codes, scales, n, k, x)
    sub = gemm.verify_gemm(codes, scales, n, k, x, rows=np.array([8, 0, 3]))
    assert np.array_equal(sub, full[:, [8, 0, 3]])
    b = gemm.abs_bound(codes, scales, n, k, x)
    assert np.all(b >= np.abs(full) - 1e-15)


def test_abs_bound_bruteforce_and_properties():
    """abs_bound = sum_k |x_k w_k|: exact rational brute force over the nibbles; equal to |y| when
    every product is non-negative; unchanged when activations change sign."""
    codes, scales, x, m, n, k = _small_case(m=2, n=3, k=64, seed=5)
    b = gemm.abs_bound(codes, scales, n, k, x)
    flat = codes.reshape(-1)
    for t in range(m):
        for r in range(n):
            acc = Fraction(0)
            for c in range(k):
                byte = int(flat[r * k // 2 + c // 2])
                nib = byte & 0xF if c % 2 == 0 else byte >> 4
                wv = Fraction(mx.e2m1_decode(nib)) * Fraction(2) ** (int(scales[r, c // 32]) - 127)
                xv = Fraction(float(np.array([int(x[t, c]) << 16], np.uint32).view(np.float32)[0]))
                acc += abs(wv * xv)
            assert abs(b[t, r] - float(acc)) <= 1e-12 * float(acc)
    # non-negative weights (codes 0..7) and activations: the bound is the product itself
    pos_codes = (codes & 0x77).astype(np.uint8)
    xf = (np.asarray(x, np.uint32) << 16).view(np.float32)
    xa = synth.f32_to_bf16_bits(np.abs(xf))  # |bf16| is a bf16 value: exact
    y = gemm.verify_gemm(pos_codes, scales, n, k, xa)
    assert np.allclose(gemm.abs_bound(pos_codes, scales, n, k, xa), y, rtol=1e-14, atol=0)
    # the sign of the activations does not matter
    neg = (np.asarray(x, np.uint16) ^ np.uint16(0x8000)).astype(np.uint16)
    assert np.array_equal(gemm.abs_bound(codes, scales, n, k, neg), b)
