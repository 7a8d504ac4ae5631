"""MX-FP4 KV cache codec (oracle). Test infrastructure only.

The news page "Next-Gen Speculative Decoding and FP4 Quantization Shake Up LLM
Inference Economics" (section "Microscaling FP4 (MX-FP4) Integration") says
MX-FP4 compresses both the weights and the KV cache tensors into 4-bit values
with an E8M0 scale per block of 32 elements; its pipeline figure draws an FP4
KV cache pool beside the verification kernel. The pages fix neither the tensor
layout nor the block axis. The reading taken here:

* the cached tensors are the key and value vectors of every token and KV head,
  [slots, heads, d] (d = 128 for the 8B-class model);
* the 32-element blocks run along d inside one token's one head: a token's
  entry never shares a block with another token, so appending a token codes
  only its own blocks and never revisits earlier entries (blocks along the
  sequence axis would have to be recoded as tokens arrive);
* codes [slots, heads, d/2] (low nibble = even element) and scales
  [slots, heads, d/32]: the weight layout of oracle.mx with row = slot * heads +
  head;
* each block is coded by the weight quantizer of oracle.mx (the OCP rule: block
  exponent floor(log2 amax) - 2, nearest E2M1 value with ties to even,
  saturating, sign of zero kept; a block with a NaN or infinity gets scale
  0xFF, codes 0 and the NONFINITE flag) from the exact fp32 value of the bf16
  input.

Footprint: 4.25 bits per cached value against 16 for bf16, 26.5625% of it.
"""
from __future__ import annotations

import numpy as np

from . import mx

FLAG_NONFINITE = mx.FLAG_NONFINITE
FLAG_SLOT_RANGE = 2  # a slot outside [0, capacity) (the entry is not written)


def bf16_to_f32(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> the same values as fp32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def append(codes: np.ndarray, scales: np.ndarray, kv_bits: np.ndarray, slots) -> int:
    """Code kv_bits [t, heads, d] (bf16 bit patterns) into the cache at rows slots[0..t-1].

    codes [capacity, heads, d/2] uint8 and scales [capacity, heads, d/32] uint8 are updated in
    place; returns the flags (FLAG_NONFINITE for a block with a NaN / infinity, FLAG_SLOT_RANGE
    for a slot outside the cache, whose entry is skipped).
    """
    cap, heads, half = codes.shape
    d = 2 * half
    kv = bf16_to_f32(kv_bits).reshape(-1, heads, d)
    flags = 0
    for i, slot in enumerate(np.asarray(slots, dtype=np.int64)):
        if not 0 <= slot < cap:
            flags |= FLAG_SLOT_RANGE
            continue
        c, s, f = mx.quantize(kv[i])
        codes[slot], scales[slot] = c, s
        flags |= f
    return flags


def read(codes: np.ndarray, scales: np.ndarray, slots) -> np.ndarray:
    """Decoded entries [len(slots), heads, d] in fp64 (exact)."""
    _, heads, half = codes.shape
    d = 2 * half
    sl = np.asarray(slots, dtype=np.int64)
    return np.stack([mx.dequantize(codes[s], scales[s], d) for s in sl]).reshape(len(sl), heads, d)


def footprint_bytes(slots: int, heads: int, d: int) -> int:
    """Bytes of codes plus scales for a cache of `slots` entries (one of K or V)."""
    return slots * heads * (d // 2 + d // mx.BLOCK)
