"""mxfp4_kv_attention on the GPU vs the fp64 attention oracle over the same MX-FP4 cache.

The caches are coded by the oracle (oracle.kvcache) and uploaded; queries are bf16. The bar is
the verify GEMM's: relative L2 <= 2e-3 over the output, and every element within
1e-4 * sum_l p_l |V^[l]| + 1e-6 (fp32 scores and sums over at most a few thousand entries per
workgroup, probabilities entering the value product as a bf16 pair: errors of order 1e-6 of that
scale). Chains (lower-triangular masks), trees, grouped-query shapes from 1 to 64 query rows per
KV head (one or two 16-row tiles, one or two groups of 32 rows), contexts that end inside a step
of 32 entries, a plain decode step (t = 1) and a refused sequence are covered.
"""
import numpy as np
import pytest
import torch

import mx_fp4_weight_amd as mxs
import synth
from oracle import attention as oatt
from oracle import kvcache
from tests.gpu_util import dev, dev_bf16, host, say

pytestmark = pytest.mark.gpu


def build(cfg, b, ctxs, t, hq, hkv, cap, d=128):
    """Oracle-coded caches [b, cap, hkv, ...] with ctx_s + t entries per sequence, and queries."""
    kc = np.zeros((b, cap, hkv, d // 2), np.uint8)
    ks = np.zeros((b, cap, hkv, d // 32), np.uint8)
    vc, vs = np.zeros_like(kc), np.zeros_like(ks)
    for s in range(b):
        n = ctxs[s] + t
        k = synth.activations(cfg, 10 + s, n * hkv, d, sigma=1.0).reshape(n, hkv, d)
        v = synth.activations(cfg, 20 + s, n * hkv, d).reshape(n, hkv, d)
        kvcache.append(kc[s], ks[s], k, range(n))
        kvcache.append(vc[s], vs[s], v, range(n))
    q = synth.activations(cfg, 30, b * t * hq, d).reshape(b, t, hq, d)
    return kc, ks, vc, vs, q


def run(kc, ks, vc, vs, q, ctxs, masks, max_len=None, flags=None):
    out = mxs.mxfp4_kv_attention(dev_bf16(q).view(q.shape), dev(kc), dev(ks), dev(vc), dev(vs),
                                 dev(np.asarray(ctxs, np.int32)), masks, max_len=max_len, dev_flags=flags)
    torch.cuda.synchronize()
    return host(out).astype(np.float64)


def check(got, kc, ks, vc, vs, q, ctxs, masks, label):
    d = q.shape[-1]
    for s in range(q.shape[0]):
        ref = oatt.attention(q[s], kc[s], ks[s], vc[s], vs[s], ctxs[s], masks, 1.0 / np.sqrt(d))
        bnd = oatt.abs_bound(q[s], kc[s], ks[s], vc[s], vs[s], ctxs[s], masks, 1.0 / np.sqrt(d))
        err = got[s] - ref
        rel = np.linalg.norm(err) / np.linalg.norm(ref)
        assert rel <= 2e-3, (label, s, rel)
        worst = np.max(np.abs(err) - (1e-4 * bnd + 1e-6))
        assert worst <= 0, (label, s, worst, np.unravel_index(np.argmax(np.abs(err) - 1e-4 * bnd), err.shape))
        say(f"  {label} seq {s}: rel L2 {rel:.2e}")


@pytest.mark.parametrize("b,ctxs,t,hq,hkv,masks_of", [
    (1, [4096], 5, 32, 8, "chain"),       # 8B-class: 32 query heads on 8 KV heads, T = 5
    (16, [4096] * 16, 5, 32, 8, "chain"), # the same for 16 sequences (the bench's batched call)
    (2, [1000, 37], 10, 8, 2, "tree"),    # a 3x2 tree (40 query rows per KV head: 4 tiles)
    (3, [0, 5, 130], 3, 4, 4, "chain"),   # one query head per KV head
    (1, [2047], 1, 16, 2, "chain"),       # a plain decode step
    (1, [300], 8, 8, 4, "tree8"),         # 16 query rows: one tile exactly
    (1, [777], 16, 8, 2, "chain"),        # 64 query rows per KV head: two groups of 32
    (1, [60000], 4, 4, 1, "chain"),       # one KV head: 469 entry ranges (merged in batches of 32)
    (2, [63, 200], 64, 2, 2, "chain"),    # T = 64 with one query head per KV head: 64 rows
])
def test_attention_matches_oracle(b, ctxs, t, hq, hkv, masks_of):
    say(f"attention b={b} ctx={ctxs} t={t} hq={hq} hkv={hkv} {masks_of}")
    if masks_of == "chain":
        masks = mxs.chain_masks(t)
    elif masks_of == "tree":
        masks = mxs.tree_masks([-1, -1, -1, 0, 0, 1, 1, 2, 2])
    else:
        masks = mxs.tree_masks([-1, 0, 0, 1, 1, 2, 5])
    assert len(masks) == t
    cap = max(ctxs) + t + 3
    kc, ks, vc, vs, q = build(17, b, ctxs, t, hq, hkv, cap)
    got = run(kc, ks, vc, vs, q, ctxs, masks)
    check(got, kc, ks, vc, vs, q, ctxs, masks, f"{masks_of} t={t}")


def test_long_context_8b():
    """32768 committed entries, T = 5: the split of the cache over many workgroups."""
    say("attention 32768 context")
    ctxs, t, hq, hkv = [32768 - 5], 5, 32, 8
    kc, ks, vc, vs, q = build(18, 1, ctxs, t, hq, hkv, 32768)
    got = run(kc, ks, vc, vs, q, ctxs, mxs.chain_masks(t))
    check(got, kc, ks, vc, vs, q, ctxs, mxs.chain_masks(t), "long")


def test_refused_sequence_and_max_len():
    say("attention refused sequence")
    t, hq, hkv = 2, 4, 2
    ctxs = [10, 60]
    kc, ks, vc, vs, q = build(19, 2, [10, 10], t, hq, hkv, 70)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = run(kc, ks, vc, vs, q, ctxs, mxs.chain_masks(t), max_len=40, flags=flags)
    assert np.all(np.isnan(got[1])) and int(flags.item()) == mxs.FLAG_TOKEN_RANGE
    check(got[:1], kc[:1], ks[:1], vc[:1], vs[:1], q[:1], ctxs[:1], mxs.chain_masks(t), "max_len")


def test_append_then_attend_on_device():
    """The verification pass end to end on the device: the prefix cache is coded by the oracle,
    the T new keys and values are appended by mxfp4_kv_append on the GPU, and the attention reads
    the cache the GPU wrote. The oracle appends the same bf16 rows itself and attends over its own
    cache; the appended bytes must be identical and the outputs within the parity bar."""
    say("attention after a device append")
    b, t, hq, hkv, d = 2, 5, 16, 4, 128
    ctxs = [300, 1023]
    cap = max(ctxs) + t + 8
    kc, ks, vc, vs, q = build(21, b, [c for c in ctxs], 0, hq, hkv, cap)  # prefixes only
    newk = [synth.activations(21, 40 + s, t * hkv, d, sigma=1.0).reshape(t, hkv, d) for s in range(b)]
    newv = [synth.activations(21, 50 + s, t * hkv, d).reshape(t, hkv, d) for s in range(b)]
    q = synth.activations(21, 60, b * t * hq, d).reshape(b, t, hq, d)
    dkc, dks, dvc, dvs = dev(kc), dev(ks), dev(vc), dev(vs)
    for s in range(b):
        slots = dev(np.arange(ctxs[s], ctxs[s] + t, dtype=np.int32))
        mxs.mxfp4_kv_append(dev_bf16(newk[s]).view(t, hkv, d), slots, dkc[s], dks[s])
        mxs.mxfp4_kv_append(dev_bf16(newv[s]).view(t, hkv, d), slots, dvc[s], dvs[s])
        kvcache.append(kc[s], ks[s], newk[s], range(ctxs[s], ctxs[s] + t))
        kvcache.append(vc[s], vs[s], newv[s], range(ctxs[s], ctxs[s] + t))
    torch.cuda.synchronize()
    for dv_, hv in ((dkc, kc), (dks, ks), (dvc, vc), (dvs, vs)):
        assert np.array_equal(host(dv_), hv)
    masks = mxs.chain_masks(t)
    out = mxs.mxfp4_kv_attention(dev_bf16(q).view(q.shape), dkc, dks, dvc, dvs,
                                 dev(np.asarray(ctxs, np.int32)), masks)
    torch.cuda.synchronize()
    check(host(out).astype(np.float64), kc, ks, vc, vs, q, ctxs, masks, "append+attend")
