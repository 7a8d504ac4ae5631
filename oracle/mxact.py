"""MX-quantized activations for the W4A8 / W4A4 verify GEMM (oracle). Test infrastructure only.

Written from the Module 11 lecture "Speculative Decoding and Quantization":
§11 ("What low-bit quantization actually changes": weight-only quantization
keeps activations and accumulation at higher precision, W8A8 and W4A4 reduce
activations too; the numerals name the widths of weights and activations,
accumulation precision being a separate choice) and §12 ("Microscaled FP4,
W4A4, and the role of hardware": E4M3 is an 8-bit float with 4 exponent and
3 fraction bits; the MX scale is an E8M0 power of two; W4A4 adds activation
quantization), with the MX block of 32 values per E8M0 scale from the news
page "Next-Gen Speculative Decoding and FP4 Quantization Shake Up LLM
Inference Economics" (section "Microscaling FP4 (MX-FP4) Integration").

Readings where the pages leave a detail open:

* A8 is MX-FP8 with E4M3 elements: 32 consecutive values along k share one
  E8M0 scale; E4M3 has bias 7, subnormals m * 2^-9, S.1111.111 = NaN, largest
  finite 448.
* A4 is MX-FP4: the weight codec of oracle.mx applied to the activation rows.
* Shared exponent: the OCP rule used for the weights, e = floor(log2 amax) -
  emax of the element format (8 for E4M3, since 448 = 1.75 * 2^8; 2 for E2M1),
  clamped to [-127, 127]; an all-zero block gets scale byte 0.
* Elements: x = v * 2^-e exactly, then the nearest E4M3 value with ties to the
  even fraction, saturating at +-448 (a block maximum in (448, 512) * 2^e
  saturates); the sign bit of v is kept, so -0 and negative underflows code
  as 0x80.
* A block holding a NaN or an infinity is refused: scale byte 0xFF (NaN),
  codes 0, flag NONFINITE.
* Inputs are bf16 activations (uint16 bit patterns), converted exactly.
* Layout: FP8 codes [m, k] bytes; FP4 codes [m, k/2] as the weights; scales
  [m, k/32] row-major.
* GEMM: Y = deq(Xq) . deq(W)^T in fp64, the exact product of the quantized
  operands.
"""
from __future__ import annotations

import numpy as np

from oracle import mx as omx
from oracle import nvfp4 as onv

BLOCK = 32
E4M3_EMAX = 8          # 448 = 1.75 * 2**8
FMT_FP8 = 0            # activation format tags (the device's element-format numbers)
FMT_FP4 = 4
FLAG_NONFINITE = 1


def bf16_to_f64(xbits) -> np.ndarray:
    return (np.asarray(xbits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3_signed_encode(x) -> np.ndarray:
    """fp64 value(s) -> E4M3 byte(s): magnitude by onv.e4m3_encode (nearest, ties to the even
    fraction, saturating at 448) and the sign bit of x."""
    x = np.asarray(x, dtype=np.float64)
    mag = onv.e4m3_encode(np.abs(x))
    return (mag | (np.signbit(x).astype(np.uint8) << 7)).astype(np.uint8)


def quantize_fp8_blocks(v):
    """fp64 blocks v[nb, 32] -> (E4M3 codes uint8 [nb, 32], scale bytes uint8 [nb], nonfinite [nb])."""
    v = np.asarray(v, dtype=np.float64)
    nonfinite = ~np.all(np.isfinite(v), axis=1)
    amax = np.max(np.abs(np.where(np.isfinite(v), v, 0.0)), axis=1)
    _, ex = np.frexp(amax)                       # amax = f * 2^ex, f in [0.5, 1)
    e = np.clip(ex.astype(np.int64) - 1 - E4M3_EMAX, -127, 127)
    e = np.where(amax == 0.0, -127, e)
    x = np.ldexp(np.where(np.isfinite(v), v, 0.0), (-e)[:, None])
    codes = e4m3_signed_encode(x)
    sb = (e + 127).astype(np.uint8)
    codes[nonfinite] = 0
    sb[nonfinite] = 0xFF
    return codes, sb, nonfinite


def quantize_fp8(xbits):
    """bf16 X[m, k] (uint16 patterns, k % 32 == 0) -> (codes uint8 [m, k], scales uint8 [m, k/32], flags)."""
    x = bf16_to_f64(xbits)
    m, k = x.shape
    if k % BLOCK:
        raise ValueError("k must be a multiple of 32")
    c, s, bad = quantize_fp8_blocks(x.reshape(-1, BLOCK))
    return c.reshape(m, k), s.reshape(m, k // BLOCK), FLAG_NONFINITE if bad.any() else 0


def quantize_fp4(xbits):
    """bf16 X[m, k] -> MX-FP4 (codes [m, k/2], scales [m, k/32], flags): the weight codec."""
    x = bf16_to_f64(xbits).astype(np.float32)    # exact: bf16 values are fp32 values
    return omx.quantize(x)


def quantize(xbits, fmt):
    if fmt == FMT_FP8:
        return quantize_fp8(xbits)
    if fmt == FMT_FP4:
        return quantize_fp4(xbits)
    raise ValueError("activation format must be FMT_FP8 or FMT_FP4")


def dequantize(codes, scales, fmt, k):
    """-> fp64 X^[m, k] = element value * 2^(s-127)."""
    scales = np.asarray(scales, dtype=np.uint8)
    if fmt == FMT_FP4:
        return omx.dequantize(codes, scales, k)
    vals = onv.e4m3_decode(np.asarray(codes, dtype=np.uint8))
    return vals * np.repeat(omx._E8M0[scales], BLOCK, axis=1)


def gemm(w_codes, w_scales, n, k, a_codes, a_scales, fmt, rows=None):
    """fp64 Y[m, n] = deq(activations) . deq(W)^T (optionally only the weight rows `rows`)."""
    w_codes = np.asarray(w_codes)
    w_scales = np.asarray(w_scales)
    if rows is not None:
        w_codes, w_scales = w_codes[rows], w_scales[rows]
    return dequantize(a_codes, a_scales, fmt, k) @ omx.dequantize(w_codes, w_scales, k).T
