"""Pins of the oracle's MX-FP4 codec against what the pages and arithmetic fix.

* the E2M1 grid, encodings and value count (golden e2m1_format.json);
* E8M0 = bare power of two;
* 4.25 bits per value for every workload shape;
* the quantizer against an independent brute-force nearest-grid search
  (distance argmin, ties to the even encoding, saturation), on a dense fp32
  sweep, all midpoints and hand-built blocks;
* invariants: block maximum decodes to 4 or 6 times the scale, error within
  half a grid step, idempotence, packing addresses.
"""
import math

import numpy as np
import pytest

from oracle import mx
from tests.conftest import golden

CONFIG_SHAPES = [
    (1024, 1024),
    (4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336),
    (8192, 8192), (1024, 8192), (28672, 8192), (8192, 28672), (128256, 8192),
    (128256, 4096),
]


def test_e2m1_grid_matches_page():
    g = golden("e2m1_format.json")
    vals = [mx.e2m1_decode(c) for c in range(16)]
    assert vals[:8] == g["e2m1_magnitudes"]
    assert [-v for v in vals[:8]] == vals[8:]          # sign bit is bit 3
    assert len(vals) == g["e2m1_encodings"]
    assert len(set(vals)) == g["e2m1_distinct_values"]  # +0 and -0 compare equal
    assert math.copysign(1.0, vals[8]) == -1.0          # code 8 is -0
    # field widths: 1 sign + 2 exponent + 1 fraction = 4 bits
    f = g["e2m1_fields"]
    assert f["sign_bits"] + f["exponent_bits"] + f["fraction_bits"] == 4


def test_e8m0_is_power_of_two():
    for s in range(255):
        v = mx.e8m0_decode(s)
        m, e = math.frexp(v)
        assert m == 0.5 and e - 1 == s - 127
    assert math.isnan(mx.e8m0_decode(255))


@pytest.mark.parametrize("n,k", CONFIG_SHAPES)
def test_storage_is_4_25_bits(n, k):
    g = golden("e2m1_format.json")
    assert mx.storage_bits_per_value(n, k) == g["mxfp4_bits_per_value"]
    per_block = (g["mx_block_elements"] * 4 + g["mx_scale_bits"]) / g["mx_block_elements"]
    assert per_block == g["mxfp4_bits_per_value"]
    assert mx.mx_bytes(n, k) * 8 == n * k * 4.25


# ---------------------------------------------------------------- brute force
_GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def brute_code(x: float) -> int:
    """Nearest E2M1 magnitude by distance; ties to the even code; beyond 6 saturates."""
    a = abs(x)
    if a >= 6.0:
        c = 7
    else:
        d = [abs(a - g) for g in _GRID]
        best = min(d)
        cands = [i for i, di in enumerate(d) if di == best]
        c = cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]
    return c | (8 if math.copysign(1.0, x) < 0 else 0)


def brute_block(v):
    """Independent per-block reference: exponent by scanning powers of two."""
    v = [float(np.float32(t)) for t in v]
    amax = max(abs(t) for t in v)
    if amax == 0.0:
        e = -127
    else:
        e = 200
        while 2.0 ** e > amax:   # largest e with 2^e <= amax
            e -= 1
        e = max(-127, min(127, e - 2))
    codes = [brute_code(t * 2.0 ** (-e)) for t in v]
    return codes, e + 127


def test_magnitude_code_dense_sweep():
    # every fp32 in [0, 8] with the last 12 mantissa bits stepped, plus both signs
    bits = np.arange(0, np.float32(8.0).view(np.uint32) + 1, 4096, dtype=np.uint32)
    xs = bits.view(np.float32).astype(np.float64)
    got = mx._magnitude_code(xs)
    want = np.array([brute_code(float(x)) & 7 for x in xs])
    assert np.array_equal(got, want)


def test_all_midpoints_and_neighbours():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    ties_to = [0, 2, 2, 4, 4, 6, 6]
    for m, t in zip(mids, ties_to):
        assert mx._magnitude_code(np.array([m]))[0] == t
        assert brute_code(m) == t
        lo = np.nextafter(np.float32(m), np.float32(0))
        hi = np.nextafter(np.float32(m), np.float32(10))
        assert mx._magnitude_code(np.array([float(lo)]))[0] == brute_code(float(lo))
        assert mx._magnitude_code(np.array([float(hi)]))[0] == brute_code(float(hi))
    # saturation: (6, 8) and beyond all land on 6
    for x in [6.0, 6.5, 7.99, 100.0]:
        assert mx._magnitude_code(np.array([x]))[0] == 7


def test_quantize_blocks_vs_brute_force_random():
    rng = np.random.default_rng(1234)
    blocks = []
    for scale in [1e-30, 1e-6, 0.02, 1.0, 7.0, 1e6, 1e30]:
        blocks.append(rng.standard_normal((40, 32)).astype(np.float32) * np.float32(scale))
    # heavy tails and exact grid values
    blocks.append((rng.standard_t(2, (40, 32)) * 0.1).astype(np.float32))
    blocks.append((rng.integers(-7, 8, (40, 32)) * 0.5).astype(np.float32))
    v = np.concatenate(blocks)
    codes, sb, bad = mx.quantize_blocks(v)
    assert not bad.any()
    for i in range(v.shape[0]):
        c, s = brute_block(v[i])
        assert list(codes[i]) == c, i
        assert sb[i] == s, i


def test_hand_built_blocks():
    # all zeros, with signed zeros: scale byte 0, codes keep the sign
    z = np.zeros((1, 32), np.float32)
    z[0, 3] = -0.0
    codes, sb, bad = mx.quantize_blocks(z)
    assert sb[0] == 0 and codes[0, 3] == 8 and codes[0, 0] == 0 and not bad[0]
    # every tie with amax = 4 (e = 0): values exactly on midpoints
    v = np.zeros((1, 32), np.float32)
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    v[0, :7] = ties
    v[0, 7:14] = [-t for t in ties]
    v[0, 14] = 4.0
    codes, sb, _ = mx.quantize_blocks(v)
    assert sb[0] == 127
    assert list(codes[0, :7]) == [0, 2, 2, 4, 4, 6, 6]
    assert list(codes[0, 7:14]) == [8, 10, 10, 12, 12, 14, 14]
    # amax in (6, 8) * 2^e saturates to 6: 7.5 with e = 0
    v = np.zeros((1, 32), np.float32)
    v[0, 0] = 7.5
    v[0, 1] = -7.9
    codes, sb, _ = mx.quantize_blocks(v)
    assert sb[0] == 127 and codes[0, 0] == 7 and codes[0, 1] == 15
    # denormal block: exponent clamps at -127
    v = np.zeros((1, 32), np.float32)
    v[0, 0] = np.float32(1e-45)           # smallest denormal, 2^-149
    v[0, 1] = np.float32(2.0 ** -127)     # a denormal power of two
    codes, sb, _ = mx.quantize_blocks(v)
    assert sb[0] == 0
    assert codes[0, 1] == 2               # 2^-127 / 2^-127 = 1.0 -> code 2
    assert codes[0, 0] == 0               # 2^-22 rounds to 0
    # largest finite fp32: exponent 127 - 2 = 125
    v = np.zeros((1, 32), np.float32)
    v[0, 0] = np.finfo(np.float32).max
    codes, sb, _ = mx.quantize_blocks(v)
    assert sb[0] == 125 + 127 and codes[0, 0] == 7
    # non-finite block is refused and reported, its neighbours are unaffected
    v = np.ones((3, 32), np.float32)
    v[1, 5] = np.nan
    v[2, 0] = -np.inf
    codes, sb, bad = mx.quantize_blocks(v)
    assert list(bad) == [False, True, True]
    assert sb[1] == 0xFF and sb[2] == 0xFF and not codes[1:].any()
    assert sb[0] == 125 and (codes[0] == 6).all()  # 1.0 = 4 * 2^-2 -> code 6 (4.0)


def test_block_max_and_error_bound():
    rng = np.random.default_rng(7)
    v = (rng.standard_normal((2000, 32)) * 0.02).astype(np.float32)
    codes, sb, _ = mx.quantize_blocks(v)
    scale = 2.0 ** (sb.astype(np.float64) - 127)
    deq = np.array([[mx.e2m1_decode(c) for c in row] for row in codes[:200]]) * scale[:200, None]
    # the element of largest magnitude decodes to 4 or 6 times the scale
    imax = np.argmax(np.abs(v[:200]), axis=1)
    top = np.abs(deq[np.arange(200), imax]) / scale[:200]
    assert set(np.unique(top)) <= {4.0, 6.0}
    # |w - w^| <= half the local grid step * scale, or <= 2 * scale when saturated
    x = np.abs(v[:200].astype(np.float64)) / scale[:200, None]
    step = np.select([x < 2, x < 4], [0.5, 1.0], 2.0)
    err = np.abs(v[:200] - deq) / scale[:200, None]
    assert np.all(err <= np.where(x > 6, 2.0, step / 2) + 1e-12)


def test_idempotent():
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    w[3, :32] = 0
    w[5, 40] = -0.0
    c1, s1, _ = mx.quantize(w)
    w2 = mx.dequantize(c1, s1, 256).astype(np.float32)
    c2, s2, _ = mx.quantize(w2)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_packing_addresses():
    """Element (r, c) lives in byte r*K/2 + c//2, low nibble for even c; scale (r, c//32)."""
    rng = np.random.default_rng(3)
    n, k = 3, 64
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    packed, scales, _ = mx.quantize(w)
    flat = packed.reshape(-1)
    codes, sb, _ = mx.quantize_blocks(w.reshape(-1, 32))
    codes = codes.reshape(n, k)
    for r in range(n):
        for c in range(k):
            byte = int(flat[r * k // 2 + c // 2])
            nib = byte & 0xF if c % 2 == 0 else byte >> 4
            assert nib == codes[r, c]
            assert scales.reshape(-1)[r * (k // 32) + c // 32] == sb[r * (k // 32) + c // 32]
    deq = mx.dequantize(packed, scales, k)
    for r in range(n):
        for c in range(k):
            byte = int(flat[r * k // 2 + c // 2])
            nib = byte & 0xF if c % 2 == 0 else byte >> 4
            s = int(scales.reshape(-1)[r * (k // 32) + c // 32])
            assert deq[r, c] == mx.e2m1_decode(nib) * mx.e8m0_decode(s)


def test_shape_refusal():
    with pytest.raises(ValueError):
        mx.quantize(np.zeros((2, 48), np.float32))
