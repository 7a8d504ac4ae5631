"""spec_accept on the GPU vs the scalar oracle loop.

Accepted counts and emitted tokens must be bit-exact for every sequence the
oracle does not flag (a decision or the final draw within 1e-6 of u). Both
sides compute probabilities and prefix sums in fp64, so flagged sequences are
compared as well unless their margin is below 1e-12 (stronger than the 1e-6
contract). With V = 128256 the residual spreads over ~1e5 tokens and the 1e-6
band around the final draw's interval ends is hit in several percent of
sequences, so no cap is put on the flagged fraction. Device flags must equal
the OR of the oracle's per-sequence flags.
"""
import numpy as np
import pytest
import torch

import mx_fp4_weight_amd as mxs
import synth
from oracle import accept as oacc
from tests.gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


def run_accept(target, draft, tokens, u, workspace=None):
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    kd = target.shape[1] - 1
    out, n = mxs.spec_accept(dev(target), dev(draft) if kd else None, dev(tokens) if kd else None,
                             dev(u), workspace=workspace, dev_flags=flags)
    torch.cuda.synchronize()
    return host(out), host(n), int(flags.item())


STRICT_MARGIN = 1e-12


def compare(target, draft, tokens, u, label, workspace=None):
    out, n, f = run_accept(target, draft, tokens, u, workspace)
    ref = oacc.step_batch(target, draft, tokens, u)
    differ = (n != ref["n"]) | np.any(out != ref["out_tokens"], axis=1)
    bad = np.nonzero(~ref["flagged"] & differ)[0]
    assert bad.size == 0, (label, bad[:5], n[bad[:5]], ref["n"][bad[:5]], out[bad[:5]], ref["out_tokens"][bad[:5]])
    bad = np.nonzero((ref["margin"] >= STRICT_MARGIN) & differ)[0]
    assert bad.size == 0, (label, "flagged but fp64-resolvable", bad[:5], ref["margin"][bad[:5]])
    assert f == int(np.bitwise_or.reduce(ref["flags"])), (label, f, ref["flags"])
    say(f"  {label}: {len(n)} sequences, {int(ref['flagged'].sum())} flagged, mean accepted {n.mean():.2f}")
    return ref


def test_tiny_config_many_sequences():
    say("accept: tiny V=1024 K=4, 2000 sequences")
    tgt, dft, tok, u = synth.accept_batch(1, 2000, 4, 1024, 2.0, 0.5)
    ref = compare(tgt, dft, tok, u, "tiny")
    assert 0 < ref["n"].mean() < 4


@pytest.mark.parametrize("sigma", [0.25, 1.0, 2.0])
def test_8b_vocab(sigma):
    say(f"accept: V=128256 K=4 sigma={sigma}")
    tgt, dft, tok, u = synth.accept_batch(2, 24, 4, 128256, 3.0, sigma, seq0=int(sigma * 1000))
    compare(tgt, dft, tok, u, f"8b sigma={sigma}")


def test_batched_64():
    say("accept: batched B=64 K=4 V=128256")
    tgt, dft, tok, u = synth.accept_batch(4, 64, 4, 128256, 3.0, 1.0)
    compare(tgt, dft, tok, u, "batched")


@pytest.mark.parametrize("kd", [0, 1, 2, 3, 5, 6, 7])
def test_draft_length_sweep(kd):
    say(f"accept: K={kd}")
    tgt, dft, tok, u = synth.accept_batch(2, 6, kd, 128256, 3.0, 0.5, seq0=100 + kd)
    compare(tgt, dft, tok, u, f"kd={kd}")


@pytest.mark.parametrize("v", [2, 5, 4095, 4096, 4097, 8192, 12289])
def test_vocab_edges(v):
    """Chunk boundaries (4096 logits per chunk) and vocabularies that disable vector loads."""
    say(f"accept: V={v}")
    tgt, dft, tok, u = synth.accept_batch(5, 300, 3, v, 2.0, 1.0, seq0=v)
    compare(tgt, dft, tok, u, f"v={v}")


# Small calls (few workgroups per launch, all candidate rows prefetched by decide)
# at vocabulary sizes on and off the 4096-logit chunk grid.
@pytest.mark.parametrize("b,kd,v", [(1, 4, 128256), (2, 3, 128256), (4, 4, 128256), (3, 0, 128256),
                                    (128, 4, 4096), (64, 2, 8192), (40, 1, 12288), (5, 4, 8),
                                    (4, 4, 131072), (2, 4, 262144)])
def test_small_calls_share_one_workspace(b, kd, v):
    """Three calls in a row on one workspace filled with garbage first: each must
    match the oracle, so nothing a call reads from the workspace survives from an
    earlier one."""
    say(f"accept: small calls b={b} K={kd} V={v}")
    ws = torch.full((mxs.spec_accept_workspace_bytes(b, kd, v),), 0xAB, dtype=torch.uint8, device="cuda")
    for rep in range(3):
        tgt, dft, tok, u = synth.accept_batch(6, b, kd, v, 3.0, 1.0, seq0=1000 * rep + b)
        compare(tgt, dft, tok, u, f"b={b} kd={kd} v={v} call {rep}", workspace=ws)


def test_workspace_shared_by_calls_of_different_sizes():
    """One workspace sized for the largest call serves smaller ones in any order
    (b = 64 runs decide without the row prefetch, b <= 4 with it)."""
    say("accept: one workspace, b = 4, 1, 64, 2, 4")
    ws = torch.full((mxs.spec_accept_workspace_bytes(64, 4, 128256),), 0xAB, dtype=torch.uint8, device="cuda")
    for b in (4, 1, 64, 2, 4):
        tgt, dft, tok, u = synth.accept_batch(6, b, 4, 128256, 3.0, 0.5, seq0=77 + b)
        compare(tgt, dft, tok, u, f"b={b}", workspace=ws)


def _logits(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, np.float64)).astype(np.float32)


def test_hand_worked_cycles():
    """Same hand-worked cycle as the oracle pin: reject at 1, residual draw lands on token 2."""
    say("accept: hand-worked")
    p0 = [0.25] * 4
    p1 = [0.375, 0.125, 0.375, 0.125]
    q1 = [0.125, 0.25, 0.125, 0.5]
    p2 = [1.0, 0.0, 0.0, 0.0]
    tgt = np.stack([_logits(p0), _logits(p1), _logits(p2)])[None]
    dft = np.stack([_logits(p0), _logits(q1)])[None]
    tok = np.array([[2, 1]], np.int32)
    out, n, f = run_accept(tgt, dft, tok, np.array([[0.3, 0.9, 0.6]], np.float32))
    assert n[0] == 1 and list(out[0]) == [2, 2, -1] and f == 0
    out, n, f = run_accept(tgt, dft, tok, np.array([[0.3, 0.2, 0.6]], np.float32))
    assert n[0] == 2 and list(out[0]) == [2, 1, 0]


@pytest.mark.parametrize("v", [6, 8])
def test_edge_cases_and_flags(v):
    """V = 6 takes the scalar-load path, V = 8 the 16-byte vector loads."""
    say(f"accept: edge cases V={v}")
    z = np.random.default_rng(1).standard_normal((4, v)).astype(np.float32)
    cases = []
    # 0: p = q never rejects
    cases.append((z[:3], z[:2], [1, 4], [0.999, 0.5, 0.3]))
    # 1: zero draw on a zero-acceptance proposal (p(x) = 0 under a -inf target logit)
    t = z[:3].copy()
    t[0, 2] = -np.inf
    cases.append((t, z[:2], [2, 0], [0.0, 0.5, 0.0]))
    # 2: draft masks the proposed token: q(x) = 0 -> rejected and flagged
    d = z[:2].copy()
    d[1, 3] = -np.inf
    cases.append((z[:3], d, [0, 3], [0.1, 0.1, 0.5]))
    # 3: token out of range
    cases.append((z[:3], z[:2], [0, 9], [0.1, 0.2, 0.5]))
    # 4: NaN logit -> refused
    t = z[:3].copy()
    t[2, 1] = np.nan
    cases.append((t, z[:2], [0, 1], [0.1, 0.2, 0.5]))
    # 5: a draft row that is all -inf -> refused
    d = z[:2].copy()
    d[0] = -np.inf
    cases.append((z[:3], d, [0, 1], [0.1, 0.2, 0.5]))
    # 6: final uniform at the top of [0, 1)
    cases.append((z[:3] * 3, z[:2], [0, 1], [0.9, 0.9, np.float32(0.99999994)]))
    for i, (t, d, tk, uu) in enumerate(cases):
        tgt = np.asarray(t, np.float32)[None]
        dft = np.asarray(d, np.float32)[None]
        tok = np.asarray(tk, np.int32)[None]
        u = np.asarray(uu, np.float32)[None]
        out, n, f = run_accept(tgt, dft, tok, u)
        ref = oacc.step(tgt[0], dft[0], tok[0], u[0])
        assert not ref["flagged"] or i in (1, 6), i   # 1: u = a = 0; 6: u at the top of the last interval
        assert n[0] == ref["n"] and list(out[0]) == list(ref["out_tokens"]), (i, out, ref)
        assert f == ref["flags"], (i, f, ref["flags"])
    # case-specific expectations from the rule itself
    assert run_accept(np.asarray(cases[2][0])[None], np.asarray(cases[2][1])[None],
                      np.array([[0, 3]], np.int32), np.array([[0.1, 0.1, 0.5]], np.float32))[2] & mxs.FLAG_Q_ZERO


def test_residual_zero_fallback():
    """u >= 1 forces a rejection of an a = 1 proposal with p = q: zero residual, draw from p."""
    say("accept: zero residual")
    z = _logits([0.5, 0.5])
    tgt = np.stack([z, z])[None]
    dft = z[None, None]
    out, n, f = run_accept(tgt, dft, np.array([[0]], np.int32), np.array([[1.0, 0.75]], np.float32))
    ref = oacc.step(tgt[0], dft[0], [0], np.array([1.0, 0.75], np.float32))
    assert n[0] == ref["n"] == 0 and out[0, 0] == ref["out_tokens"][0] == 1
    assert f == ref["flags"] and f & mxs.FLAG_RESIDUAL_ZERO


@pytest.mark.parametrize("v", [6, 4097, 128256])
def test_equal_rows_forced_rejection(v):
    """Target row == draft row and an out-of-range draft token: the residual is exactly zero
    (no FMA residue), so the draw falls back to p and RESIDUAL_ZERO is raised."""
    say(f"accept: equal rows, forced rejection, V={v}")
    z = synth.rng(9, 3, v).standard_normal((3, v)).astype(np.float32) * np.float32(3.0)
    tgt = z[None]
    dft = z[None, :2].copy()
    tok = np.array([[0, v + 5]], np.int32)
    for uk in [0.0, 0.3, 0.77]:
        u = np.array([[0.5, 0.5, uk]], np.float32)
        out, n, f = run_accept(tgt, dft, tok, u)
        ref = oacc.step(tgt[0], dft[0], tok[0], u[0])
        assert ref["flags"] == (mxs.FLAG_TOKEN_RANGE | mxs.FLAG_RESIDUAL_ZERO)
        assert f == ref["flags"], (v, uk, f)
        if ref["margin"] >= 1e-12:
            assert n[0] == ref["n"] == 1 and list(out[0]) == list(ref["out_tokens"]), (v, uk)
