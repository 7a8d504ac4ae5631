"""Verification of a tree of draft tokens (oracle). Test infrastructure only.

The pages give the exact rule for one chain of drafts (Module 11 lecture
"Speculative Decoding and Quantization", §4: accept x with probability
min(1, p(x)/q(x)), at the first rejection replace it by a draw from
r = norm((p - q)+), a bonus draw from the next law when all survive; the
mass-balance identity min(p, q) + (1 - alpha) r = p makes the emitted token
follow p). For a tree they only say that Medusa-style trees with typical
acceptance lack that guarantee (§8) and that tree verification needs its own
argument (§4). The reading taken here is the plainest one that keeps §4's
guarantee with nothing but §4's identity:

* a node's children are independent draws from the draft law q of the node's
  history (with replacement, so two children may carry the same token);
* the children are tried in index order: child j is accepted with probability
  min(1, p_j(x_j)/q(x_j)), where p_1 is the target law p of the node's history
  and, after a rejection, p_{j+1} = norm((p_j - q)+), §4's residual taken
  against the current law; an accepted child becomes the next node;
* when every child is rejected, or the node is a leaf, the final token is
  drawn from the current law (the last residual, or p itself at a leaf: the
  bonus draw).

Each try is §4's cycle with target p_j and proposal q, so by the identity the
token a node emits follows p_j before the try, hence p at the node; a chain
(one child per node) is exactly §4's rule. As in §4, a residual with no mass
left (possible only through rounding) is reported and the draw falls back to
the law before the failed try, and no further child is tried.

Layout: parent[i] in {-1 (the root), 0 .. i-1} for the N draft nodes (parents
precede children); target and draft logit rows 0 .. N, row 0 for the root's
history and row i + 1 for the history ending in node i (a node's children are
drawn from its draft row); tokens[i] the draft token of node i; uniforms u[i]
for node i's test and u[N] for the one final draw (a convention, as the
lecture notes equality in law fixes no consumption order).
"""
from __future__ import annotations

import numpy as np

from . import accept

FLAG_NONFINITE = accept.FLAG_NONFINITE
FLAG_TOKEN_RANGE = accept.FLAG_TOKEN_RANGE
FLAG_Q_ZERO = accept.FLAG_Q_ZERO
FLAG_RESIDUAL_ZERO = accept.FLAG_RESIDUAL_ZERO
MARGIN = accept.MARGIN


def children_of(parent) -> list[list[int]]:
    """children[v + 1] = the nodes whose parent is v (v = -1 for the root), ascending."""
    parent = [int(x) for x in parent]
    n = len(parent)
    for i, p in enumerate(parent):
        if not -1 <= p < i:
            raise ValueError("parent[i] must be -1 or a node before i")
    ch = [[] for _ in range(n + 1)]
    for i, p in enumerate(parent):
        ch[p + 1].append(i)
    return ch


def depth(parent) -> int:
    """Number of nodes on the longest root-to-leaf path (0 for an empty tree)."""
    d = []
    for i, p in enumerate(parent):
        d.append(1 if p < 0 else d[p] + 1)
    return max(d, default=0)


def next_law(w: np.ndarray, q: np.ndarray):
    """The law a node tries its next child against after a rejection: norm((w - q)+), or None
    when the positive part has no mass."""
    r = accept.residual_weights(w, q)
    z = r.sum()
    return r / z if z > 0.0 else None


def step(parent, target: np.ndarray, draft: np.ndarray, tokens, u) -> dict:
    """One verification cycle of one sequence over a token tree.

    target, draft [N+1, V] fp32 logits; tokens [N]; u [N+1] fp32. Returns out_tokens [D+1]
    (the accepted path's tokens, then the final token, then -1; D = depth), nodes [D] (the
    accepted path's node indices, then -1), n (accepted drafts), flags, flagged (a decision
    or the final draw within MARGIN of its uniform) and the smallest such margin.
    """
    ch = children_of(parent)
    n_nodes = len(ch) - 1
    target = np.asarray(target, dtype=np.float32)
    draft = np.asarray(draft, dtype=np.float32)
    if target.shape[0] != n_nodes + 1 or draft.shape != target.shape or len(tokens) != n_nodes \
            or len(u) != n_nodes + 1:
        raise ValueError("shape mismatch")
    d = depth(parent)
    out = np.full(d + 1, -1, dtype=np.int32)
    nodes = np.full(d, -1, dtype=np.int32)
    # every law of the tree is examined up front, as the batched verification pass scores
    # every node at once: a malformed row refuses the whole sequence
    p_rows = [accept.softmax(target[i]) for i in range(n_nodes + 1)]
    q_rows = [accept.softmax(draft[i]) for i in range(n_nodes + 1)]
    if any(r is None for r in p_rows + q_rows):
        return dict(out_tokens=out, nodes=nodes, n=0, flags=FLAG_NONFINITE, flagged=False, margin=np.inf)

    flags = 0
    margin_min = np.inf
    v = -1      # current node (-1: the root)
    n = 0
    while True:
        w = p_rows[v + 1]
        q = q_rows[v + 1]
        moved = False
        for c in ch[v + 1]:
            a, f = accept.acceptance(w, q, int(tokens[c]))
            flags |= f
            uc = float(u[c])
            margin_min = min(margin_min, abs(uc - a))
            if uc < a:
                out[n] = int(tokens[c])
                nodes[n] = c
                n += 1
                v = c
                moved = True
                break
            nxt = next_law(w, q)
            if nxt is None:  # no residual mass (rounding): draw from w, try no further child
                flags |= FLAG_RESIDUAL_ZERO
                break
            w = nxt
        if not moved:
            break
    t, margin = accept.inverse_cdf(w, float(u[n_nodes]))
    margin_min = min(margin_min, margin)
    out[n] = t
    return dict(out_tokens=out, nodes=nodes, n=n, flags=flags, flagged=bool(margin_min < MARGIN),
                margin=margin_min)


def step_batch(parent, target, draft, tokens, u) -> dict:
    """step() for b sequences sharing one tree: target, draft [b, N+1, V], tokens [b, N], u [b, N+1]."""
    b = target.shape[0]
    d = depth(parent)
    out = np.full((b, d + 1), -1, dtype=np.int32)
    nodes = np.full((b, d), -1, dtype=np.int32)
    n = np.zeros(b, dtype=np.int32)
    flags = np.zeros(b, dtype=np.int32)
    flagged = np.zeros(b, dtype=bool)
    margin = np.zeros(b)
    for s in range(b):
        r = step(parent, target[s], draft[s], tokens[s], u[s])
        out[s], nodes[s], n[s], flags[s], flagged[s], margin[s] = (r["out_tokens"], r["nodes"], r["n"], r["flags"],
                                                                  r["flagged"], r["margin"])
    return dict(out_tokens=out, nodes=nodes, n=n, flags=flags, flagged=flagged, margin=margin)
