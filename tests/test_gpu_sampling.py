"""spec_accept_sampled on the GPU vs the oracle's transformed-law cycle.

Same bar as the plain cycle: accepted counts and emitted tokens bit-exact for
every sequence the oracle does not flag (a decision or the final draw within
1e-6 of u, or a top-p boundary within 1e-9 of a tie); device flags equal the
OR of the oracle's. Draft tokens are drawn from the oracle's transformed draft
laws (Gumbel-max with the shared seeded noise), as a caller sampling from the
filtered proposal would.
"""
import numpy as np
import pytest
import torch

import mx_fp4_weight_amd as mxs
import synth
from oracle import accept as oacc
from oracle import sampling as osm
from tests.gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


def transformed_draft_tokens(dft, tau, k, p, mask, config, seq0):
    b, kd, v = dft.shape
    tok = np.zeros((b, kd), np.int32)
    for s in range(b):
        g = synth.rng(config, synth.ROLE_DRAFT, seq0 + s).gumbel(size=(kd, v))
        for i in range(kd):
            q, _ = osm.transformed_law(dft[s, i], tau, k, p, None if mask is None else mask[s, i])
            if q is None:
                continue
            with np.errstate(divide="ignore"):
                tok[s, i] = int(np.argmax(np.log(q) + g[i]))
    return tok


def run_sampled(tgt, dft, tok, u, tau, k, p, mask, workspace=None):
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    kd = tgt.shape[1] - 1
    m = None if mask is None else dev(synth.pack_mask(mask).view(np.int32))
    out, n = mxs.spec_accept_sampled(dev(tgt), dev(dft) if kd else None, dev(tok) if kd else None, dev(u),
                                     tau, k, p, m, workspace=workspace, dev_flags=flags)
    torch.cuda.synchronize()
    return host(out), host(n), int(flags.item())


def compare(tgt, dft, tok, u, tau, k, p, mask, label):
    out, n, f = run_sampled(tgt, dft, tok, u, tau, k, p, mask)
    ref = osm.step_sampled_batch(tgt, dft, tok, u, tau, k, p, mask)
    differ = (n != ref["n"]) | np.any(out != ref["out_tokens"], axis=1)
    bad = np.nonzero(~ref["flagged"] & differ)[0]
    assert bad.size == 0, (label, bad[:5], n[bad[:5]], ref["n"][bad[:5]], out[bad[:5]], ref["out_tokens"][bad[:5]])
    assert f == int(np.bitwise_or.reduce(ref["flags"])), (label, f, ref["flags"])
    say(f"  {label}: {len(n)} sequences, {int(ref['flagged'].sum())} flagged, mean accepted {n.mean():.2f}")
    return ref


def inputs(config, b, kd, v, base_sigma, noise_sigma, tau, k, p, keep, seq0=0):
    tgt, dft, _, u = synth.accept_batch(config, b, kd, v, base_sigma, noise_sigma, seq0=seq0)
    mask = None
    if keep is not None:
        mask = np.stack([synth.token_mask(config, seq0 + s, kd + 1, v, keep) for s in range(b)])
    tok = transformed_draft_tokens(dft, tau, k, p, mask, config, seq0)
    return tgt, dft, tok, u, mask


SETTINGS = [  # (temperature, top_k, top_p, mask keep fraction)
    (0.7, 0, 1.0, None),
    (1.0, 50, 1.0, None),
    (1.0, 0, 0.9, None),
    (0.8, 40, 0.8, None),
    (1.3, 0, 0.95, 0.7),
    (1.0, 1, 1.0, None),
    (0.5, 5, 0.5, 0.5),
    (2.0, 300, 0.99, 0.9),
]


@pytest.mark.parametrize("tau,k,p,keep", SETTINGS)
def test_small_vocab_many_sequences(tau, k, p, keep):
    say(f"sampled: V=1024 K=4 tau={tau} k={k} p={p} keep={keep}")
    tgt, dft, tok, u, mask = inputs(21, 160, 4, 1024, 2.0, 0.5, tau, k, p, keep, seq0=int(tau * 100) + k)
    compare(tgt, dft, tok, u, tau, k, p, mask, f"tau={tau} k={k} p={p}")


@pytest.mark.parametrize("tau,k,p,keep", [(0.8, 50, 0.9, None), (1.0, 0, 0.95, None),
                                          (1.2, 1000, 1.0, 0.6), (1.0, 0, 0.6, 0.3),
                                          (0.9, 100, 0.8, None), (1.0, 128, 1.0, 0.9)])
def test_8b_vocab(tau, k, p, keep):
    say(f"sampled: V=128256 K=4 tau={tau} k={k} p={p} keep={keep}")
    tgt, dft, tok, u, mask = inputs(22, 3, 4, 128256, 3.0, 1.0, tau, k, p, keep, seq0=k)
    compare(tgt, dft, tok, u, tau, k, p, mask, f"8b tau={tau} k={k} p={p}")


@pytest.mark.parametrize("v", [5, 4095, 4097, 12289])
def test_vocab_edges(v):
    """Chunk edges and vocabularies without vector loads."""
    say(f"sampled: V={v}")
    tgt, dft, tok, u, mask = inputs(23, 60, 3, v, 2.0, 1.0, 0.9, 7, 0.85, 0.8, seq0=v)
    compare(tgt, dft, tok, u, 0.9, 7, 0.85, mask, f"v={v}")


@pytest.mark.parametrize("kd", [0, 1, 6])
def test_draft_lengths(kd):
    say(f"sampled: K={kd}")
    tgt, dft, tok, u, mask = inputs(24, 40, kd, 8192, 2.0, 0.7, 0.9, 100, 0.9, 0.8, seq0=kd)
    compare(tgt, dft, tok, u, 0.9, 100, 0.9, mask, f"kd={kd}")


def test_ties_in_logits():
    """Integer logits: many ties at the top-k and top-p boundaries (all tied tokens stay)."""
    say("sampled: tied logits")
    b, kd, v = 60, 3, 512
    r = synth.rng(25, 3)
    tgt = r.integers(-3, 4, size=(b, kd + 1, v)).astype(np.float32)
    dft = tgt[:, :kd] + r.integers(-1, 2, size=(b, kd, v)).astype(np.float32)
    u = r.random((b, kd + 1), dtype=np.float32)
    for tau, k, p in [(1.0, 10, 1.0), (1.0, 0, 0.7), (0.7, 30, 0.5), (1.0, 1, 1.0)]:
        tok = transformed_draft_tokens(dft, tau, k, p, None, 25, 0)
        compare(tgt, dft, tok, u, tau, k, p, None, f"ties tau={tau} k={k} p={p}")


def test_defaults_equal_plain_spec_accept():
    say("sampled: defaults == spec_accept")
    tgt, dft, tok, u = synth.accept_batch(26, 8, 4, 128256, 3.0, 1.0)
    out_s, n_s, f_s = run_sampled(tgt, dft, tok, u, 1.0, 0, 1.0, None)
    out, n = mxs.spec_accept(dev(tgt), dev(dft), dev(tok), dev(u))
    torch.cuda.synchronize()
    assert np.array_equal(out_s, host(out)) and np.array_equal(n_s, host(n)) and f_s == 0
    ref = oacc.step_batch(tgt, dft, tok, u)
    keep = ~ref["flagged"]
    assert np.array_equal(out_s[keep], ref["out_tokens"][keep])


def test_mask_edge_cases():
    """The mask removes the proposed draft token (q = 0: rejected and flagged), and removes every
    token of one row (the sequence is refused)."""
    say("sampled: mask edge cases")
    b, kd, v = 4, 2, 256
    tgt, dft, _, u = synth.accept_batch(27, b, kd, v, 2.0, 0.5)
    mask = np.ones((b, kd + 1, v), bool)
    tok = np.array([[3, 7], [10, 11], [20, 21], [30, 31]], np.int32)
    mask[0, 0, 3] = False          # draft token 0 of sequence 0 removed: Q_ZERO at position 0
    mask[1, 1, :] = False          # position 1 of sequence 1 has no allowed token: refused
    mask[2, 2, :] = False
    mask[2, 2, 5] = True           # bonus row of sequence 2 keeps one token
    out, n, f = run_sampled(tgt, dft, tok, u, 1.0, 0, 1.0, mask)
    ref = osm.step_sampled_batch(tgt, dft, tok, u, 1.0, 0, 1.0, mask)
    assert np.array_equal(out, ref["out_tokens"]) and np.array_equal(n, ref["n"])
    assert f == int(np.bitwise_or.reduce(ref["flags"]))
    assert f & mxs.FLAG_Q_ZERO and f & mxs.FLAG_NONFINITE
    assert ref["n"][0] == 0 and list(out[1]) == [-1, -1, -1]


def test_workspace_reused_across_settings():
    """One garbage-filled workspace serves calls with different transforms in a row."""
    say("sampled: one workspace, several settings")
    b, kd, v = 3, 4, 128256
    ws = torch.full((mxs.spec_accept_sampled_workspace_bytes(b, kd, v),), 0xAB, dtype=torch.uint8,
                    device="cuda")
    for i, (tau, k, p, keep) in enumerate([(1.0, 0, 0.9, None), (0.8, 64, 1.0, 0.7), (1.0, 20, 0.8, None)]):
        tgt, dft, tok, u, mask = inputs(28, b, kd, v, 3.0, 1.0, tau, k, p, keep, seq0=100 * i)
        out, n, f = run_sampled(tgt, dft, tok, u, tau, k, p, mask, workspace=ws)
        ref = osm.step_sampled_batch(tgt, dft, tok, u, tau, k, p, mask)
        keep_rows = ~ref["flagged"]
        assert np.array_equal(out[keep_rows], ref["out_tokens"][keep_rows]), i
        assert f == int(np.bitwise_or.reduce(ref["flags"]))


def test_nonfinite_rows_under_top_k():
    """A NaN or +inf logit anywhere in a row refuses its sequence also when top-k / top-p leave
    it out of the kept set (the selection then leaves that row's statistics to the stats pass);
    the other sequences keep their tokens."""
    say("sampled: non-finite logits under top-k")
    b, kd, v = 6, 3, 8192
    tgt, dft, _, u = synth.accept_batch(29, b, kd, v, 2.0, 0.7)
    tgt[1, 0, 17] = np.nan      # target row 0 of sequence 1
    dft[2, 1, 4000] = np.inf    # draft row 1 of sequence 2
    tgt[3, kd, 5] = np.nan      # bonus row of sequence 3
    for tau, k, p in [(1.0, 20, 1.0), (0.8, 50, 0.9)]:
        tok = transformed_draft_tokens(np.nan_to_num(dft, nan=0.0, posinf=0.0), tau, k, p, None, 29, 0)
        ref = compare(tgt, dft, tok, u, tau, k, p, None, f"nonfinite tau={tau} k={k} p={p}")
        assert all(ref["n"][i] == 0 for i in (1, 2, 3)) and ref["flags"][1] & mxs.FLAG_NONFINITE


@pytest.mark.parametrize("tau,k,p,keep", [(0.8, 50, 0.9, 0.9), (1.0, 0, 0.95, None)])
def test_batch_64_full_vocab(tau, k, p, keep):
    """The batched configuration the bench times: B = 64, K = 4, V = 128256 (576 rows; the counting
    pass then takes 8 chunks per workgroup)."""
    say(f"sampled: B=64 V=128256 K=4 tau={tau} k={k} p={p} keep={keep}")
    tgt, dft, tok, u, mask = inputs(30, 64, 4, 128256, 3.0, 1.0, tau, k, p, keep, seq0=1000 + k)
    compare(tgt, dft, tok, u, tau, k, p, mask, f"B=64 tau={tau} k={k} p={p}")
