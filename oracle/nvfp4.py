"""NVFP4 weight format (oracle). Test infrastructure only.

Written from the Module 11 lecture "Speculative Decoding and Quantization",
§12 ("Microscaled FP4, W4A4, and the role of hardware"): NVFP4 holds E2M1
values with a two-level scale, in the one-dimensional layout one E4M3 scale
per block of 16 values plus one FP32 scale for the whole tensor (4.5 bits per
value counting the block scale); E4M3 is an 8-bit float with 4 exponent bits
and 3 fraction bits.

Readings where the lecture leaves a detail open:

* E4M3 encoding: sign, 4 exponent bits (bias 7), 3 fraction bits; exponent 0
  is subnormal (m * 2^-9); no infinities; S.1111.111 is NaN, so the largest
  finite value is 1.75 * 2^8 = 448 (the 8-bit format of that name in common
  use). Scales are non-negative.
* Global scale g = amax(|W|) / (6 * 448) over the finite entries (fp32), so
  the block with the tensor's largest magnitude gets a block scale near 448;
  g = 1 for an all-zero tensor.
* Block scale: t = amax_block / (6 * g), rounded to E4M3 to nearest with ties
  to the even fraction, saturating at 448 (the block maximum then lands near
  6 on the E2M1 grid, as the MX rule puts it near 4..6).
* Values: x = w / (E4M3(scale) * g), rounded to the E2M1 grid as for MX-FP4
  (nearest, ties to even, saturating at 6, sign kept on zeros). A block whose
  scale rounds to 0 gets +-0 codes.
* Arithmetic of the quantizer: fp32, each operation correctly rounded (the
  divisions and the two products 6 * g and E4M3 * g), so a device quantizer
  doing the same operations gets the same bytes.
* A block holding a NaN or +-inf is refused: scale byte 0x7F (NaN), codes 0,
  flag NONFINITE; non-finite entries are left out of amax.
* Storage: codes [N, K/2] exactly as MX-FP4 (low nibble = even column),
  scales [N, K/16] bytes, one fp32 global scale.

Dequantized value: E2M1(code) * E4M3(scale) * g (fp64 here).
"""
from __future__ import annotations

import numpy as np

from oracle import mx as omx

BLOCK = 16
E4M3_MAX = 448.0
FLAG_NONFINITE = 1


def e2m1_encode(x):
    """fp32 value(s) already divided by the block scale -> E2M1 code(s): the MX-FP4 rounding
    (nearest, ties to the even code, saturating at 6) with the sign bit of x."""
    x = np.asarray(x, dtype=np.float64)
    mag = omx._magnitude_code(np.where(np.isfinite(x), x, 0.0))
    return (mag | (np.signbit(x).astype(np.uint8) << 3)).astype(np.uint8)


def e4m3_decode(byte):
    """E4M3 byte(s) -> fp64 value(s) (NaN for S.1111.111)."""
    b = np.asarray(byte, dtype=np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (8 + m) * 2.0 ** (e - 10))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


E4M3_TABLE = e4m3_decode(np.arange(128))   # non-negative bytes 0x00..0x7F (0x7F = NaN)


def e4m3_encode(t):
    """Non-negative fp32 value(s) -> E4M3 byte(s): nearest finite value, ties to the even
    fraction, saturating at 448. The non-negative encodings increase with the byte, so the
    nearest value is one of the two table entries around t."""
    t = np.asarray(t, dtype=np.float64)
    finite = E4M3_TABLE[:127]
    hi = np.clip(np.searchsorted(finite, t, side="left"), 1, 126)
    lo = hi - 1
    dlo = t - finite[lo]
    dhi = finite[hi] - t
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(t <= 0, 0, pick)
    return np.where(t >= E4M3_MAX, 0x7E, pick).astype(np.uint8)


def e4m3_encode_brute(t):
    """Same rule by scanning all 127 non-negative finite encodings (small inputs; a pin)."""
    t = np.asarray(t, dtype=np.float64)
    finite = E4M3_TABLE[:127]
    d = np.abs(t[..., None] - finite)
    cand = d == d.min(axis=-1, keepdims=True)
    even = (np.arange(127) & 1) == 0
    pick = np.where((cand & even).any(axis=-1), np.argmax(cand & even, axis=-1), np.argmax(cand, axis=-1))
    return np.where(t >= E4M3_MAX, 0x7E, pick).astype(np.uint8)


def global_scale(w) -> np.float32:
    w = np.asarray(w, dtype=np.float32)
    fin = np.isfinite(w)
    amax = np.float32(np.abs(w[fin]).max()) if fin.any() else np.float32(0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / np.float32(6.0 * E4M3_MAX))


def quantize(w):
    """fp32 W[n, k] (k % 16 == 0) -> (codes uint8 [n, k/2], scales uint8 [n, k/16], g fp32, flags)."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if k % BLOCK:
        raise ValueError("k must be a multiple of 16")
    g = global_scale(w)
    blocks = w.reshape(n, k // BLOCK, BLOCK)
    bad = ~np.isfinite(blocks).all(axis=-1)
    amax = np.where(bad, 0.0, np.abs(np.where(np.isfinite(blocks), blocks, 0)).max(axis=-1)).astype(np.float32)
    denom = np.float32(np.float32(6.0) * g)                       # fp32 product
    t = (amax / denom).astype(np.float32)                          # fp32 division
    sbytes = e4m3_encode(t)
    dscale = (e4m3_decode(sbytes).astype(np.float32) * g).astype(np.float32)   # fp32 product
    with np.errstate(divide="ignore", invalid="ignore"):
        x = (blocks / dscale[..., None]).astype(np.float32)          # fp32 division
    zero_scale = dscale == 0
    x = np.where(zero_scale[..., None], np.where(np.signbit(blocks), -0.0, 0.0), x).astype(np.float32)
    codes = e2m1_encode(x)
    codes = np.where(bad[..., None], 0, codes).astype(np.uint8)
    sbytes = np.where(bad, 0x7F, sbytes).astype(np.uint8)
    packed = omx.pack_nibbles(codes.reshape(n, k))
    flags = FLAG_NONFINITE if bad.any() else 0
    return packed, sbytes.reshape(n, k // BLOCK), g, flags


def dequantize(codes, scales, g):
    """-> fp64 Ŵ[n, k] = E2M1(code) * E4M3(scale) * g."""
    codes = np.asarray(codes, dtype=np.uint8)
    k = codes.shape[1] * 2
    vals = omx._E2M1[omx.unpack_nibbles(codes, k)]
    s = e4m3_decode(np.asarray(scales)).repeat(BLOCK, axis=1)
    return vals * s * np.float64(g)


def verify_gemm(codes, scales, g, xbits, rows=None):
    """fp64 Y = X · Ŵᵀ for bf16 activations given as uint16 bit patterns [m, k]."""
    x = (np.asarray(xbits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    codes = np.asarray(codes)
    scales = np.asarray(scales)
    if rows is not None:
        codes, scales = codes[rows], scales[rows]
    return x @ dequantize(codes, scales, g).T
