"""Pins of the verification-attention oracle (oracle.attention).

* against a library routine: torch's scaled_dot_product_attention in fp64 on the CPU, fed the
  cache entries decoded by oracle.kvcache (itself pinned) and a boolean mask built directly from
  the tree's ancestor sets, on random grouped-query shapes, chains and trees;
* closed forms: one visible entry returns its value row exactly; equal scores return the mean of
  the visible value rows; a chain's masks are lower-triangular; the tree masks are ancestor sets;
* invariance: permuting the prefix entries does not change the output.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import attention as oatt
from oracle import kvcache


def make_cache(cfg, ctx, t, hkv, d, cap=None, sigma=1.0):
    cap = cap or ctx + t
    kc = np.zeros((cap, hkv, d // 2), np.uint8)
    ks = np.zeros((cap, hkv, d // 32), np.uint8)
    vc = np.zeros_like(kc)
    vs = np.zeros_like(ks)
    k = synth.activations(cfg, 1, (ctx + t) * hkv, d, sigma=sigma).reshape(ctx + t, hkv, d)
    v = synth.activations(cfg, 2, (ctx + t) * hkv, d).reshape(ctx + t, hkv, d)
    kvcache.append(kc, ks, k, range(ctx + t))
    kvcache.append(vc, vs, v, range(ctx + t))
    return kc, ks, vc, vs


def ancestors(parent):
    """Direct ancestor sets (self included) of the T = N + 1 positions, by walking up the parents."""
    n = len(parent)
    sets = [{0}]
    for i in range(n):
        s, p = {i + 1}, parent[i]
        while p >= 0:
            s.add(p + 1)
            p = parent[p]
        s.add(0)
        sets.append(s)
    return sets


@pytest.mark.parametrize("ctx,parent,hq,hkv,d", [
    (40, [-1, 0, 1, 2], 8, 2, 128),
    (17, [-1, -1, 0, 0, 1, 1], 4, 1, 64),
    (0, [-1, 0], 2, 2, 32),
    (65, [], 6, 3, 128),
])
def test_matches_torch_sdpa(ctx, parent, hq, hkv, d):
    t = len(parent) + 1
    kc, ks, vc, vs = make_cache(3, ctx, t, hkv, d)
    q = synth.activations(3, 5, t * hq, d).reshape(t, hq, d)
    masks = oatt.tree_masks(parent)
    scale = 1.0 / np.sqrt(d)
    got = oatt.attention(q, kc, ks, vc, vs, ctx, masks, scale)
    k = torch.from_numpy(kvcache.read(kc, ks, range(ctx + t)))
    v = torch.from_numpy(kvcache.read(vc, vs, range(ctx + t)))
    qq = torch.from_numpy(kvcache.bf16_to_f32(q).astype(np.float64))
    allowed = torch.zeros((t, ctx + t), dtype=torch.bool)
    allowed[:, :ctx] = True
    for pos, anc in enumerate(ancestors(parent)):
        for a in anc:
            allowed[pos, ctx + a] = True
    g = hq // hkv
    ref = np.zeros_like(got)
    for h in range(hq):
        o = torch.nn.functional.scaled_dot_product_attention(
            qq[:, h][None], k[:, h // g][None], v[:, h // g][None], attn_mask=allowed[None], scale=scale)
        ref[:, h] = o[0].numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_masks():
    assert oatt.tree_masks([-1, 0, 1, 2]) == [0b1, 0b11, 0b111, 0b1111, 0b11111]
    assert oatt.tree_masks([-1, -1, 0, 1]) == [0b1, 0b11, 0b101, 0b1011, 0b10101]
    for parent in ([-1, -1, 0, 0, 1, 1, 2], [-1, 0, 0, 2, -1]):
        for pos, (m, anc) in enumerate(zip(oatt.tree_masks(parent), ancestors(parent))):
            assert {r for r in range(len(parent) + 1) if (m >> r) & 1} == anc


def test_single_visible_entry_and_equal_scores():
    hkv, d = 1, 32
    kc, ks, vc, vs = make_cache(4, 0, 3, hkv, d)
    q = synth.activations(4, 9, 3, d).reshape(3, 1, d)
    out = oatt.attention(q, kc, ks, vc, vs, 0, [0b1, 0b11, 0b111], 0.25)
    np.testing.assert_array_equal(out[0, 0], kvcache.read(vc, vs, [0])[0, 0])   # position 0 sees only entry 0
    # a zero query gives equal scores: the output is the mean of the visible value rows
    qz = np.zeros((3, 1, d), np.uint16)
    out = oatt.attention(qz, kc, ks, vc, vs, 0, [0b1, 0b11, 0b101], 1.0)
    vv = kvcache.read(vc, vs, range(3))[:, 0]
    np.testing.assert_allclose(out[1, 0], vv[:2].mean(0), rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(out[2, 0], vv[[0, 2]].mean(0), rtol=1e-15, atol=1e-15)


def test_prefix_permutation_invariance():
    ctx, t, hkv, d = 30, 2, 2, 64
    kc, ks, vc, vs = make_cache(6, ctx, t, hkv, d)
    q = synth.activations(6, 3, t * 4, d).reshape(t, 4, d)
    a = oatt.attention(q, kc, ks, vc, vs, ctx, [0b1, 0b11], 0.125)
    perm = np.concatenate([np.random.default_rng(0).permutation(ctx), np.arange(ctx, ctx + t)])
    b = oatt.attention(q, kc[perm], ks[perm], vc[perm], vs[perm], ctx, [0b1, 0b11], 0.125)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)
