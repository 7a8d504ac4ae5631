"""Verification GEMM (oracle). Test infrastructure only.

The target model scores all T = K+1 draft positions in one forward pass, so
each weight matrix is read once and applied to T activation rows (Module 11
"Speculative Decoding and Quantization", §4 and §10; weight-streaming limit
Q <= BW/W of §1). With MX-FP4 weights the layer computes

    Y[t, n] = sum_k X[t, k] * Ŵ[n, k],   Ŵ = E2M1(code) * 2^(s - 127),

which is what the news page's MX-FP4 GEMV listing ("Microscaling FP4 (MX-FP4)
Integration") sets out to do with fp32 accumulation, for T = 1. The oracle
computes it exactly up to fp64 rounding: X's bf16 values and Ŵ are both exact
in fp64, and the product is a library fp64 matmul on dequantized row chunks.
"""
from __future__ import annotations

import numpy as np

from . import mx


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> exact fp64 values (a bf16 is the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def verify_gemm(codes: np.ndarray, scales: np.ndarray, n: int, k: int,
                x_bits: np.ndarray, rows: np.ndarray | None = None,
                chunk: int = 2048) -> np.ndarray:
    """fp64 Y[m, n] = X · Ŵᵀ (or Y[m, len(rows)] for a subset of output rows).

    codes [n, k/2] uint8, scales [n, k/32] uint8, x_bits [m, k] uint16 (bf16).
    """
    codes = np.asarray(codes, dtype=np.uint8).reshape(n, k // 2)
    scales = np.asarray(scales, dtype=np.uint8).reshape(n, k // mx.BLOCK)
    x = bf16_bits_to_f64(x_bits).reshape(-1, k)
    idx = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    y = np.empty((x.shape[0], idx.size), dtype=np.float64)
    for lo in range(0, idx.size, chunk):
        sel = idx[lo:lo + chunk]
        w = mx.dequantize(codes[sel], scales[sel], k)
        y[:, lo:lo + sel.size] = x @ w.T
    return y


def abs_bound(codes: np.ndarray, scales: np.ndarray, n: int, k: int,
              x_bits: np.ndarray, rows: np.ndarray | None = None,
              chunk: int = 2048) -> np.ndarray:
    """sum_k |X[t, k] * Ŵ[n, k]| — the scale an fp32 accumulation error is measured against."""
    codes = np.asarray(codes, dtype=np.uint8).reshape(n, k // 2)
    scales = np.asarray(scales, dtype=np.uint8).reshape(n, k // mx.BLOCK)
    x = np.abs(bf16_bits_to_f64(x_bits).reshape(-1, k))
    idx = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    y = np.empty((x.shape[0], idx.size), dtype=np.float64)
    for lo in range(0, idx.size, chunk):
        sel = idx[lo:lo + chunk]
        w = np.abs(mx.dequantize(codes[sel], scales[sel], k))
        y[:, lo:lo + sel.size] = x @ w.T
    return y
