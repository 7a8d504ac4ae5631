"""mxfp4_kv_append on the GPU vs the KV cache oracle (oracle.kvcache.append): codes and scales
bit-exact, entries at other slots untouched, slots outside the cache flagged and skipped."""
import numpy as np
import pytest
import torch

import mx_fp4_weight_amd as mxs
import synth
from oracle import kvcache as okv
from tests.gpu_util import dev, dev_bf16, host, say

pytestmark = pytest.mark.gpu


def run_append(kv_bits, slots, cap, heads, d, fill=0x5A):
    t = len(slots)
    codes = torch.full((cap, heads, d // 2), fill, dtype=torch.uint8, device="cuda")
    scales = torch.full((cap, heads, d // 32), fill, dtype=torch.uint8, device="cuda")
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    mxs.mxfp4_kv_append(dev_bf16(kv_bits.reshape(t, heads, d)).view(t, heads, d), dev(np.asarray(slots, np.int32)),
                        codes, scales, dev_flags=flags)
    torch.cuda.synchronize()
    ref_c = np.full((cap, heads, d // 2), fill, np.uint8)
    ref_s = np.full((cap, heads, d // 32), fill, np.uint8)
    ref_f = okv.append(ref_c, ref_s, kv_bits.reshape(t, heads, d), slots)
    return host(codes), host(scales), int(flags.item()), ref_c, ref_s, ref_f


@pytest.mark.parametrize("t,heads,d,cap", [(5, 8, 128, 64), (1, 1, 32, 1), (16, 8, 128, 4096), (33, 2, 96, 50)])
def test_append_matches_oracle(t, heads, d, cap):
    say(f"kv append t={t} heads={heads} d={d} cap={cap}")
    rng = np.random.default_rng(t * 7 + cap)
    slots = rng.choice(cap, size=t, replace=False).astype(np.int32)
    kv = synth.activations(13, t + heads, t * heads, d, sigma=2.5)
    c, s, f, rc, rs, rf = run_append(kv, slots, cap, heads, d)
    assert np.array_equal(c, rc) and np.array_equal(s, rs) and f == rf == 0


def test_prefill_8b_layer():
    """A 4096-token prefill of one layer's K (8 KV heads of 128) into a 8192-entry cache."""
    say("kv append prefill 4096 x 8 x 128")
    t, heads, d, cap = 4096, 8, 128, 8192
    slots = np.arange(100, 100 + t, dtype=np.int32)
    kv = synth.activations(14, 0, t * heads, d)
    c, s, f, rc, rs, rf = run_append(kv, slots, cap, heads, d)
    assert np.array_equal(c, rc) and np.array_equal(s, rs) and f == rf == 0


def test_out_of_range_slots_and_special_values():
    say("kv append edge cases")
    heads, d, cap = 2, 64, 6
    kv = synth.activations(15, 1, 4 * heads, d).reshape(4, heads, d).copy()
    kv[0, 0, :32] = 0x0000                       # all-zero block
    kv[0, 1, :32] = 0x8000                       # -0 block
    kv[1, 0, 3] = 0x7FC0                         # NaN
    kv[1, 1, 40] = 0xFF80                        # -inf
    kv[2, 0, :32] = 0x0001                       # subnormal bf16 values
    slots = np.array([4, 0, 7, -1], np.int32)    # the last two are outside the cache
    c, s, f, rc, rs, rf = run_append(kv, slots, cap, heads, d)
    assert np.array_equal(c, rc) and np.array_equal(s, rs)
    assert f == rf == okv.FLAG_NONFINITE | okv.FLAG_SLOT_RANGE
