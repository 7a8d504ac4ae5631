"""Verification attention over an MX-FP4 KV cache (oracle). Test infrastructure only.

The verification pass scores every draft position in one batched target forward ("Module 11.
Speculative Decoding and Quantization", §4: the target pass stays causal, the row predicting
x_i cannot see later proposals; for a tree, a node sees its own path); with the KV cache held
in MX-FP4 (news page "Next-Gen Speculative Decoding and FP4 Quantization Shake Up LLM Inference
Economics", "Microscaling FP4 (MX-FP4) Integration"), each query position attends to the
committed prefix and to the new positions its mask allows, over the decoded keys and values:

    out[t, h] = sum_l softmax_l(scale * q[t, h] . K^[l, h / G]) V^[l, h / G]

over the visible entries l: every prefix entry l < ctx, and new entry ctx + r when bit r of
mask[t] is set (r an ancestor of t or t itself; a lower-triangular mask for a chain). K^ and V^
are the MX-FP4 cache entries decoded exactly (oracle.kvcache layout); G = query heads / KV
heads (grouped-query attention). Everything after the decode is fp64.
"""
from __future__ import annotations

import numpy as np

from . import kvcache


def bf16_to_f64(bits) -> np.ndarray:
    return kvcache.bf16_to_f32(bits).astype(np.float64)


def visible(ctx: int, t: int, masks, length: int) -> np.ndarray:
    """bool [length]: which cache entries query position t sees."""
    vis = np.zeros(length, dtype=bool)
    vis[:ctx] = True
    m = int(masks[t])
    for r in range(length - ctx):
        vis[ctx + r] = bool((m >> r) & 1)
    return vis


def attention(q_bits, k_codes, k_scales, v_codes, v_scales, ctx: int, masks, scale: float) -> np.ndarray:
    """fp64 out [T, Hq, d] for one sequence.

    q_bits [T, Hq, d] bf16 bit patterns; caches [capacity, Hkv, d/2] codes and [capacity, Hkv,
    d/32] scales with the T new entries at ctx .. ctx+T-1; masks [T] ints (bit r: sees new
    position r); scale the score factor (1/sqrt(d) for plain attention).
    """
    q = bf16_to_f64(q_bits)
    t_n, hq, d = q.shape
    hkv = k_codes.shape[1]
    g = hq // hkv
    length = ctx + t_n
    k = kvcache.read(k_codes, k_scales, range(length))  # [length, Hkv, d]
    v = kvcache.read(v_codes, v_scales, range(length))
    out = np.zeros((t_n, hq, d))
    for t in range(t_n):
        vis = visible(ctx, t, masks, length)
        for h in range(hq):
            s = (k[vis, h // g, :] @ q[t, h]) * scale
            p = np.exp(s - s.max())
            p /= p.sum()
            out[t, h] = p @ v[vis, h // g, :]
    return out


def abs_bound(q_bits, k_codes, k_scales, v_codes, v_scales, ctx: int, masks, scale: float) -> np.ndarray:
    """sum_l p_l |V^[l]|: the scale an error of the weighted sum is measured against."""
    q = bf16_to_f64(q_bits)
    t_n, hq, d = q.shape
    hkv = k_codes.shape[1]
    g = hq // hkv
    length = ctx + t_n
    k = kvcache.read(k_codes, k_scales, range(length))
    v = np.abs(kvcache.read(v_codes, v_scales, range(length)))
    out = np.zeros((t_n, hq, d))
    for t in range(t_n):
        vis = visible(ctx, t, masks, length)
        for h in range(hq):
            s = (k[vis, h // g, :] @ q[t, h]) * scale
            p = np.exp(s - s.max())
            p /= p.sum()
            out[t, h] = p @ v[vis, h // g, :]
    return out


def tree_masks(parent) -> list[int]:
    """Masks of the T = N + 1 positions of a tree's verification pass: position 0 is the root's
    input token, position i + 1 draft node i; a position sees itself and its ancestors."""
    n = len(parent)
    masks = [1]
    for i in range(n):
        p = int(parent[i])
        masks.append(masks[p + 1] | (1 << (i + 1)))
    return masks
