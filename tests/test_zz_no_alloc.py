"""spec_accept_noalloc (the built-in workspace) against spec_accept (a caller workspace).

Two calls in a row on the same GPU, the second with a smaller input, so the second
runs on the built-in array as the first left it; outputs, accepted counts and device
flags must equal spec_accept's bit for bit. (Sizes past the built-in array are refused
before any HIP call; tests/test_abi_cpu.py checks that without a GPU.)
"""
import numpy as np
import pytest
import torch

import mx_fp4_weight_amd as mxs
import synth
from tests.gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


def _both(tgt, dft, tok, u):
    b, kd1, _ = tgt.shape
    kd = kd1 - 1
    args = (dev(tgt), dev(dft) if kd else None, dev(tok) if kd else None, dev(u))
    f_ref = torch.zeros(1, dtype=torch.int32, device="cuda")
    ref_tok, ref_n = mxs.spec_accept(*args, dev_flags=f_ref)
    f_na = torch.zeros(1, dtype=torch.int32, device="cuda")
    out_tok = torch.full((b, kd + 1), -7, dtype=torch.int32, device="cuda")
    out_n = torch.full((b,), -7, dtype=torch.int32, device="cuda")
    mxs.spec_accept_noalloc(*args, out_tok, out_n, dev_flags=f_na)
    torch.cuda.synchronize()
    return (host(ref_tok), host(ref_n), int(f_ref.item())), (host(out_tok), host(out_n), int(f_na.item()))


@pytest.mark.parametrize("first,second", [
    ((64, 4, 128256), (3, 2, 4097)),   # batched call, then a small one with a vocab off the vector path
    ((2, 4, 128256), (1, 0, 1000)),    # one sequence, then no drafts at all
])
def test_noalloc_matches_spec_accept(first, second):
    for call, (b, kd, v) in enumerate((first, second)):
        say(f"noalloc: call {call} b={b} K={kd} V={v}")
        tgt, dft, tok, u = synth.accept_batch(8, b, kd, v, 3.0, 1.0, seq0=31 * call + b)
        (rt, rn, rf), (nt, nn, nf) = _both(tgt, dft, tok, u)
        assert np.array_equal(nt, rt) and np.array_equal(nn, rn) and nf == rf, (call, b, kd, v)
