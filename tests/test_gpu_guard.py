"""Guard bands around every output buffer: no entry point writes outside the outputs it is given.

Each output is a view into a larger device buffer whose bytes before and after it hold a
fixed pattern; after each call the pattern must be intact. Ragged sizes (outputs that end off a
16-byte boundary, partial row blocks, partial tiles, vocabularies off the vector path) and
outputs at offsets that disable the vector stores are covered. This is a plain correctness
test: the calls are valid and no fault is expected.
"""
import numpy as np
import pytest
import torch

import mx_fp4_weight_amd as mxs
import synth
from oracle import mx as omx
from tests.gpu_util import dev, dev_bf16, say

pytestmark = pytest.mark.gpu

GUARD = 4096  # bytes of pattern on each side
PATTERN = 0xC3


class Guarded:
    """A device output of `shape` and `dtype` inside a byte buffer with guard bands (the output
    starts `skew` bytes past the front guard)."""

    def __init__(self, shape, dtype, skew=0):
        self.nbytes = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        self.skew = skew
        self.buf = torch.full((GUARD + skew + self.nbytes + GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.buf[GUARD + skew:GUARD + skew + self.nbytes].view(dtype).view(shape)

    def intact(self):
        torch.cuda.synchronize()
        h = self.buf.cpu().numpy()
        front, back = h[:GUARD + self.skew], h[GUARD + self.skew + self.nbytes:]
        return bool(np.all(front == PATTERN) and np.all(back == PATTERN))


def mx_weights(n, k, idx):
    c, s, _ = omx.quantize(synth.weights(16, idx, n, k))
    return dev(c), dev(s)


@pytest.mark.parametrize("n,k,m,skew", [(1000, 4096, 5, 0), (17, 512, 3, 4), (4100, 4096, 8, 4), (33, 160, 7, 0),
                                        (130, 384, 81, 4), (300, 14336, 5, 4), (9, 1024, 17, 0)])
def test_verify_gemm_outputs(n, k, m, skew):
    say(f"guard: verify gemm n={n} k={k} m={m} skew={skew}")
    dc, ds = mx_weights(n, k, n + k + m)
    x = dev_bf16(synth.activations(16, n + m, m, k))
    y = Guarded((m, n), torch.float32, skew)
    mxs.mxfp4_verify_gemm(dc, ds, x, y=y.t)
    assert y.intact()
    if k % 128 == 0:
        yt = Guarded((m, n), torch.float32, skew)
        mxs.mxfp4_verify_gemm_tiled(mxs.mxfp4_tile_codes(dc), mxs.mxfp4_tile_scales(ds), n, k, x, y=yt.t)
        assert yt.intact()


def test_grouped_and_nvfp4_outputs():
    say("guard: grouped / NVFP4")
    k, m = 1024, 5
    shapes = [1000, 130, 17, 9]
    items, ys, tiled, yts = [], [], [], []
    for i, n in enumerate(shapes):
        dc, ds = mx_weights(n, k, 50 + i)
        x = dev_bf16(synth.activations(16, 50 + i, m, k))
        items.append((dc, ds, x))
        tiled.append((mxs.mxfp4_tile_codes(dc), mxs.mxfp4_tile_scales(ds), n, x))
        ys.append(Guarded((m, n), torch.float32, 4 * (i % 2)))
        yts.append(Guarded((m, n), torch.float32, 4 * ((i + 1) % 2)))
    mxs.mxfp4_verify_gemm_grouped(items, ys=[g.t for g in ys])
    mxs.mxfp4_verify_gemm_grouped_tiled(tiled, ys=[g.t for g in yts])
    assert all(g.intact() for g in ys + yts)
    w = dev(synth.weights(16, 60, 300, 512))
    codes, scales = Guarded((300, 256), torch.uint8), Guarded((300, 32), torch.uint8)
    gs = Guarded((1,), torch.float32)
    mxs.nvfp4_quantize(w, codes=codes.t, scales=scales.t, global_scale=gs.t)
    y = Guarded((5, 300), torch.float32, 4)
    mxs.nvfp4_verify_gemm(codes.t, scales.t, gs.t, dev_bf16(synth.activations(16, 61, 5, 512)), y=y.t)
    assert codes.intact() and scales.intact() and gs.intact() and y.intact()


def test_quantize_outputs():
    say("guard: quantizers")
    w = dev(synth.weights(16, 70, 37, 96))
    codes, scales = Guarded((37, 48), torch.uint8), Guarded((37, 3), torch.uint8, 1)
    mxs.mxfp4_quantize(w, codes=codes.t, scales=scales.t)
    x = dev_bf16(synth.activations(16, 71, 7, 160))
    ac, asc = Guarded((7, 80), torch.uint8), Guarded((7, 5), torch.uint8, 3)
    mxs.mx_quantize_act(x, mxs.ACT_FP4, codes=ac.t, scales=asc.t)
    assert codes.intact() and scales.intact() and ac.intact() and asc.intact()


@pytest.mark.parametrize("b,kd,v", [(3, 4, 1000), (1, 4, 128256), (5, 0, 4097), (64, 4, 8192)])
def test_accept_outputs(b, kd, v):
    say(f"guard: spec_accept b={b} K={kd} V={v}")
    tgt, dft, tok, u = synth.accept_batch(16, b, kd, v, 3.0, 1.0, seq0=b + v)
    ot, on = Guarded((b, kd + 1), torch.int32, 4), Guarded((b,), torch.int32, 8)
    args = (dev(tgt), dev(dft) if kd else None, dev(tok) if kd else None, dev(u))
    mxs.spec_accept(*args, out_tokens=ot.t, out_num=on.t)
    assert ot.intact() and on.intact()
    ot2, on2 = Guarded((b, kd + 1), torch.int32), Guarded((b,), torch.int32, 4)
    mxs.spec_accept_noalloc(*args, ot2.t, on2.t)
    assert ot2.intact() and on2.intact() and torch.equal(ot2.t, ot.t)
    ot3, on3 = Guarded((b, kd + 1), torch.int32, 4), Guarded((b,), torch.int32)
    mxs.spec_accept_sampled(*args, 0.9, 20, 0.95, None, out_tokens=ot3.t, out_num=on3.t)
    assert ot3.intact() and on3.intact()


def test_tree_and_kv_outputs():
    say("guard: tree / kv append")
    parent = [-1, -1, 0, 0, 1, 2]
    b, v = 7, 4097
    tgt, dft, tok, u = synth.tree_batch(16, b, parent, v, 3.0, 1.0)
    d = mxs.tree_depth(parent)
    ot, on, onum = Guarded((b, d + 1), torch.int32, 4), Guarded((b, d), torch.int32), Guarded((b,), torch.int32, 8)
    mxs.spec_accept_tree(parent, dev(tgt), dev(dft), dev(tok), dev(u), out_tokens=ot.t, out_nodes=on.t,
                         out_num=onum.t)
    assert ot.intact() and on.intact() and onum.intact()
    heads, dd, cap = 8, 128, 10
    kv = dev_bf16(synth.activations(16, 80, 3 * heads, dd)).view(3, heads, dd)
    codes, scales = Guarded((cap, heads, dd // 2), torch.uint8), Guarded((cap, heads, dd // 32), torch.uint8, 4)
    mxs.mxfp4_kv_append(kv, dev(np.array([0, cap - 1, 4], np.int32)), codes.t, scales.t)
    assert codes.intact() and scales.intact()
