"""OCP MX-FP4 codec (oracle). Test infrastructure only.

Format, as the Module 11 lecture ("Speculative Decoding and Quantization",
§12 "Microscaled FP4, W4A4, and the role of hardware") states it:

* an E2M1 element has one sign bit, two exponent bits and one fraction bit;
  its magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6, and the two zeros make 16
  encodings for 15 values;
* an E8M0 scale is a bare power of two with no fraction field (bias 127, so
  byte s means 2^(s-127); byte 255 is the NaN encoding);
* 32 elements share one scale, giving (32*4 + 8)/32 = 4.25 bits per value.

Storage follows the MX-FP4 GEMV listing of the news page "Next-Gen Speculative
Decoding and FP4 Quantization Shake Up LLM Inference Economics" (section
"Microscaling FP4 (MX-FP4) Integration"): codes row-major as [N, K/2] bytes
(element (r, c) in byte r*K/2 + c//2) and scales row-major as [N, K/32].
The nibble order inside a byte is not given there; the low nibble holds the
even column.

Quantizer: the pages cite the OCP MX v1.0 specification without restating the
shared-exponent rule; this oracle takes the plain OCP reading: the block
exponent is floor(log2(amax)) minus the E2M1 largest exponent (2, since
6 = 1.5 * 2^2), elements are scaled by 2^-e exactly and rounded to the nearest
E2M1 value with ties to the even encoding, saturating at +-6.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E2M1_EMAX = 2          # 6.0 = 1.5 * 2**2
E8M0_BIAS = 127
E8M0_NAN = 0xFF
FLAG_NONFINITE = 1


def e2m1_decode(code: int) -> float:
    """Value of one 4-bit E2M1 code from its bit fields (sign | 2-bit exponent | 1-bit fraction).

    Exponent field 0 is the subnormal range (value = fraction * 0.5); otherwise
    value = 2^(exponent-1) * (1 + fraction/2). Bias 1.
    """
    if not 0 <= int(code) <= 15:
        raise ValueError("E2M1 code must be in 0..15")
    sign = (code >> 3) & 1
    exp = (code >> 1) & 3
    frac = code & 1
    if exp == 0:
        mag = 0.5 * frac
    else:
        mag = 2.0 ** (exp - 1) * (1.0 + 0.5 * frac)
    return -mag if sign else mag


def e8m0_decode(s: int) -> float:
    """Value of one E8M0 scale byte: 2^(s-127); 0xFF is NaN."""
    if not 0 <= int(s) <= 255:
        raise ValueError("E8M0 byte must be in 0..255")
    if s == E8M0_NAN:
        return float("nan")
    return float(2.0 ** (int(s) - E8M0_BIAS))


# Decode tables built from the bit-field definitions above (oracle-local).
_E2M1 = np.array([e2m1_decode(c) for c in range(16)], dtype=np.float64)
_E8M0 = np.array([e8m0_decode(s) for s in range(256)], dtype=np.float64)


def _magnitude_code(x: np.ndarray) -> np.ndarray:
    """E2M1 magnitude code (0..7) of |x| by round-to-nearest-even with saturation.

    Grid 0, .5, 1, 1.5, 2, 3, 4, 6 (codes 0..7). Midpoints are 0.25, 0.75, 1.25,
    1.75, 2.5, 3.5, 5; a value exactly on a midpoint goes to the even code
    (the one whose fraction bit is 0): 0.25->0, 0.75->1.0, 1.25->1.0,
    1.75->2, 2.5->2, 3.5->4, 5->4. Everything above 5 becomes 6 (saturation).
    """
    a = np.abs(x)
    code = np.zeros(a.shape, dtype=np.uint8)
    code += (a > 0.25)    # tie 0.25 -> code 0 (even)
    code += (a >= 0.75)   # tie 0.75 -> code 2 (even)
    code += (a > 1.25)    # tie 1.25 -> code 2
    code += (a >= 1.75)   # tie 1.75 -> code 4
    code += (a > 2.5)     # tie 2.5  -> code 4
    code += (a >= 3.5)    # tie 3.5  -> code 6
    code += (a > 5.0)     # tie 5    -> code 6; (5, inf) -> code 7 = 6.0
    return code


def quantize_blocks(v: np.ndarray):
    """Quantize fp32 blocks v[nb, 32] -> (codes uint8 [nb, 32] unpacked, scale bytes uint8 [nb], nonfinite bool [nb]).

    Per block, in order:
      1. a block holding a NaN or infinity is refused: scale byte 0xFF (E8M0
         NaN), codes 0, and it is reported;
      2. amax = max |v|;
      3. amax = 0: scale byte 0 (exponent clamped to -127), codes are the
         signed zeros (+0 -> 0x0, -0 -> 0x8);
      4. otherwise e = floor(log2 amax) - 2 from the exact binary exponent
         (frexp), clamped to [-127, 127]; scale byte = e + 127;
      5. x = v * 2^-e (exact in fp64);
      6. magnitude code by round-to-nearest-even on the E2M1 grid, saturating;
      7. sign bit = sign bit of v (so -0 and negative underflows keep 0x8).
    """
    v = np.asarray(v, dtype=np.float32)
    if v.ndim != 2 or v.shape[1] != BLOCK:
        raise ValueError("expected blocks of 32 values")
    v64 = v.astype(np.float64)
    nonfinite = ~np.all(np.isfinite(v64), axis=1)
    amax = np.max(np.abs(np.where(np.isfinite(v64), v64, 0.0)), axis=1)
    _, ex = np.frexp(amax)                 # amax = m * 2^ex, m in [0.5, 1)
    e = ex.astype(np.int64) - 1 - E2M1_EMAX
    e = np.clip(e, -127, 127)
    e = np.where(amax == 0.0, -127, e)
    scale_byte = (e + E8M0_BIAS).astype(np.uint8)
    x = np.ldexp(v64, (-e)[:, None])
    x = np.where(np.isfinite(x), x, 0.0)
    code = _magnitude_code(x)
    sign = np.signbit(v64).astype(np.uint8) << 3
    codes = (code | sign).astype(np.uint8)
    codes[nonfinite] = 0
    scale_byte[nonfinite] = E8M0_NAN
    return codes, scale_byte, nonfinite


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[n, k] codes (0..15) -> [n, k/2] bytes; even column in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    lo = codes[:, 0::2] & 0xF
    hi = codes[:, 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray, k: int) -> np.ndarray:
    """[n, k/2] bytes -> [n, k] codes."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], k), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def quantize(w: np.ndarray):
    """fp32 W[n, k] (k % 32 == 0) -> (codes uint8 [n, k/2], scales uint8 [n, k/32], flags int).

    flags has FLAG_NONFINITE set when any block held a NaN or infinity.
    """
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2 or w.shape[1] % BLOCK:
        raise ValueError("W must be [n, k] with k a multiple of 32")
    n, k = w.shape
    codes, sb, bad = quantize_blocks(w.reshape(-1, BLOCK))
    packed = pack_nibbles(codes.reshape(n, k))
    flags = FLAG_NONFINITE if bool(bad.any()) else 0
    return packed, sb.reshape(n, k // BLOCK), flags


def dequantize(codes: np.ndarray, scales: np.ndarray, k: int) -> np.ndarray:
    """Packed [n, k/2] codes + [n, k/32] scales -> fp64 Ŵ[n, k] = E2M1(code) * 2^(s-127)."""
    c = unpack_nibbles(codes, k)
    val = _E2M1[c]
    sc = _E8M0[np.asarray(scales, dtype=np.uint8)]
    return val * np.repeat(sc, BLOCK, axis=1)


def storage_bits_per_value(n: int, k: int) -> float:
    """Bits per weight of the packed layout: 8*(n*k/2 + n*k/32) / (n*k)."""
    return 8.0 * (n * k // 2 + n * k // BLOCK) / (n * k)


def mx_bytes(n: int, k: int) -> int:
    """Bytes of the packed codes plus scales of an [n, k] matrix."""
    return n * k // 2 + n * k // BLOCK
