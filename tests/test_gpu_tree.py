"""spec_accept_tree on the GPU vs the tree oracle (oracle.tree.step_batch).

Accepted counts, accepted node paths and emitted tokens must be bit-exact for every sequence
whose smallest decision or draw margin is at least 1e-12 (both sides compute the laws and
prefix sums in fp64; the contract flags margins below 1e-6). Device flags must equal the OR
of the oracle's per-sequence flags.
"""
import numpy as np
import pytest
import torch

import mx_fp4_weight_amd as mxs
import synth
from oracle import tree as otree
from tests.gpu_util import dev, host, say

pytestmark = pytest.mark.gpu

TREES = {
    "chain4": [-1, 0, 1, 2],
    "3x2": [-1, -1, -1, 0, 0, 1, 1, 2, 2],
    "binary3": [-1, -1, 0, 0, 1, 1, 2, 2, 3, 3, 4, 4, 5, 5],
    "star8": [-1] * 8,
    "single": [-1],
    "ragged": [-1, 0, -1, 1, 1, 2, 4, 4, 4, 0],
}


def run_tree(parent, tgt, dft, tok, u, workspace=None):
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, nodes, n = mxs.spec_accept_tree(parent, dev(tgt), dev(dft), dev(tok) if len(parent) else None, dev(u),
                                         workspace=workspace, dev_flags=flags)
    torch.cuda.synchronize()
    return host(out), host(nodes), host(n), int(flags.item())


def compare(parent, tgt, dft, tok, u, label, workspace=None):
    out, nodes, n, f = run_tree(parent, tgt, dft, tok, u, workspace)
    ref = otree.step_batch(parent, tgt, dft, tok, u)
    differ = (n != ref["n"]) | np.any(out != ref["out_tokens"], axis=1) | np.any(nodes != ref["nodes"], axis=1)
    bad = np.nonzero((ref["margin"] >= 1e-12) & differ)[0]
    assert bad.size == 0, (label, bad[:5], n[bad[:5]], ref["n"][bad[:5]], out[bad[:5]], ref["out_tokens"][bad[:5]])
    assert f == int(np.bitwise_or.reduce(ref["flags"])) if len(ref["flags"]) else f == 0, (label, f)
    say(f"  {label}: {len(n)} sequences, {int(ref['flagged'].sum())} flagged, mean accepted {n.mean():.2f}")
    return ref


@pytest.mark.parametrize("name", list(TREES))
@pytest.mark.parametrize("v,sigma", [(1024, 0.5), (128256, 1.0), (4097, 2.0)])
def test_trees_match_oracle(name, v, sigma):
    parent = TREES[name]
    b = 48 if v <= 4097 else 6
    say(f"tree: {name} V={v} sigma={sigma}")
    tgt, dft, tok, u = synth.tree_batch(9, b, parent, v, 3.0, sigma, seq0=len(parent) * 100 + v % 97)
    compare(parent, tgt, dft, tok, u, f"{name} v={v}")


@pytest.mark.parametrize("name", ["chain4", "3x2", "binary3"])
def test_batched_64(name):
    """B = 64 at V = 128256: the batched calls the bench times (large-grid passes)."""
    parent = TREES[name]
    say(f"tree: {name} B=64 V=128256")
    tgt, dft, tok, u = synth.tree_batch(10, 64, parent, 128256, 3.0, 0.5)
    compare(parent, tgt, dft, tok, u, f"{name} b=64")


def test_no_drafts_is_a_bonus_draw():
    say("tree: no nodes")
    tgt, dft, tok, u = synth.tree_batch(11, 20, [], 1024, 2.0, 1.0)
    compare([], tgt, dft, tok, u, "empty tree")


def test_edge_cases_and_shared_dirty_workspace():
    """q(x) = 0, a token out of range, a NaN row (refused), u = 0 and u at the top of [0, 1),
    duplicate siblings; three calls on one workspace filled with garbage first."""
    parent = TREES["3x2"]
    v = 64
    tgt, dft, tok, u = synth.tree_batch(12, 12, parent, v, 2.0, 1.0)
    dft[0, 0, tok[0, 0]] = -np.inf                  # q(x) = 0 for the root's first child
    tok[1, 0] = v + 3                               # out of range (the root's first child: always tried)
    tgt[2, 4, 7] = np.nan                           # refused sequence
    u[3, :] = 0.0
    u[4, :] = np.float32(1.0) - np.float32(2.0 ** -24)
    tok[5, 1] = tok[5, 0]                           # duplicate siblings at the root
    tok[6, 2] = tok[6, 1] = tok[6, 0]
    need = mxs.spec_accept_tree_workspace_bytes(parent, 12, v)
    ws = torch.full((need,), 0xAB, dtype=torch.uint8, device="cuda")
    for rep in range(3):
        ref = compare(parent, tgt, dft, tok, u, f"edges call {rep}", workspace=ws)
    assert ref["flags"][0] & otree.FLAG_Q_ZERO and ref["flags"][1] & otree.FLAG_TOKEN_RANGE
    assert ref["flags"][2] == otree.FLAG_NONFINITE


@pytest.mark.parametrize("name", ["3x2", "binary3", "chain4"])
def test_zero_residual_at_an_inner_node(name):
    """Identical target and draft rows at the root, its first child's token at -inf in both: the
    child is refused (q(x) = 0), the residual (p - q)+ has no mass, and the final token is drawn
    from p at the root, an inner node (R8's rule at a tree node)."""
    parent = TREES[name]
    say(f"tree: zero residual at the root, {name}")
    for v, b in [(1024, 16), (128256, 4)]:
        tgt, dft, tok, u = synth.tree_batch(13, b, parent, v, 3.0, 1.0, seq0=7 * len(parent))
        dft[:, 0] = tgt[:, 0]
        for s in range(b):
            x = tok[s, 0]
            tgt[s, 0, x] = dft[s, 0, x] = -np.inf
        ref = compare(parent, tgt, dft, tok, u, f"{name} v={v}")
        assert np.all(ref["n"] == 0)
        assert np.all(ref["flags"] & otree.FLAG_RESIDUAL_ZERO) and np.all(ref["flags"] & otree.FLAG_Q_ZERO)
