"""Pins of the tree-verification oracle (oracle.tree).

* a chain (one child per node) is the linear rule: oracle.tree.step equals oracle.accept.step
  token for token, with the same uniforms, on random laws, rejections, bonus draws and flags;
* law preservation by brute force: over many cycles with siblings drawn independently from
  their parent's draft law, the first emitted token follows the root's target law and, on
  the cycles whose path enters node c, the next token follows node c's target law (Pearson
  chi-square at every such node); a planted mistake (later siblings tried against p instead of
  the residual) fails it;
* hand-built cases: a leaf gives the bonus draw from its own law; duplicate siblings (the
  second try of a rejected token has acceptance 0); q(x) = 0 and out-of-range tokens are
  flagged and rejected; u = 0 takes the first positive token of the final law.
"""
import numpy as np
import pytest
from scipy import stats

from oracle import accept, tree

V = 5


def logits_of(p):
    p = np.asarray(p, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return np.log(p).astype(np.float32)


def test_children_and_depth():
    parent = [-1, -1, 0, 0, 2, -1]
    assert tree.children_of(parent) == [[0, 1, 5], [2, 3], [], [4], [], [], []]
    assert tree.depth(parent) == 3
    with pytest.raises(ValueError):
        tree.children_of([0])
    with pytest.raises(ValueError):
        tree.children_of([-1, 2, 1])


@pytest.mark.parametrize("kd", [0, 1, 2, 4, 6])
def test_chain_is_the_linear_rule(kd):
    rng = np.random.default_rng(kd)
    parent = [-1] + list(range(kd - 1)) if kd else []
    for trial in range(300):
        v = int(rng.integers(2, 9))
        tgt = (rng.standard_normal((kd + 1, v)) * 1.5).astype(np.float32)
        dft = tgt + (rng.standard_normal((kd + 1, v)) * rng.choice([0.0, 0.5, 2.0])).astype(np.float32)
        if trial % 7 == 3 and kd:
            dft[0, 0] = -np.inf          # a draft law with a zero
        tok = rng.integers(0, v + (1 if trial % 11 == 5 else 0), kd).astype(np.int32)
        u = rng.random(kd + 1).astype(np.float32)
        if trial % 13 == 0:
            u[:] = 0.0
        lin = accept.step(tgt, dft[:kd], tok, u)
        tr = tree.step(parent, tgt, dft, tok, u)
        assert tr["n"] == lin["n"] and tr["flags"] == lin["flags"], trial
        assert np.array_equal(tr["out_tokens"], lin["out_tokens"]), trial
        assert list(tr["nodes"][:tr["n"]]) == list(range(tr["n"])) and np.all(tr["nodes"][tr["n"]:] == -1)


# a tree with a three-way root, a two-way child and a chain below another child
PARENT = [-1, -1, -1, 0, 0, 1, 5]


def laws(seed):
    rng = np.random.default_rng(seed)
    n = len(PARENT)
    p = rng.dirichlet(np.ones(V) * 0.8, n + 1)
    q = rng.dirichlet(np.ones(V) * 0.8, n + 1)
    return p, q


def run_cycles(p, q, cycles, seed):
    """Brute-force cycles: siblings drawn from their parent's draft law, fresh uniforms."""
    rng = np.random.default_rng(seed)
    n = len(PARENT)
    tgt = np.stack([logits_of(r) for r in p])
    dft = np.stack([logits_of(r) for r in q])
    first = np.zeros(V, np.int64)
    nxt = {c: np.zeros(V, np.int64) for c in range(n)}
    cq = np.cumsum(q, axis=1)
    for _ in range(cycles):
        tok = np.array([min(V - 1, int(np.searchsorted(cq[PARENT[c] + 1], rng.random(), side="right")))
                        for c in range(n)], np.int32)
        u = rng.random(n + 1).astype(np.float32)
        r = tree.step(PARENT, tgt, dft, tok, u)
        first[r["out_tokens"][0]] += 1
        for i in range(r["n"]):
            nxt[int(r["nodes"][i])][r["out_tokens"][i + 1]] += 1
    return first, nxt


def chi2_p(counts, law):
    tot = counts.sum()
    exp = law * tot
    keep = exp > 0
    assert counts[~keep].sum() == 0
    return stats.chisquare(counts[keep], exp[keep]).pvalue


@pytest.mark.slow
def test_tree_preserves_the_target_law():
    p, q = laws(3)
    first, nxt = run_cycles(p, q, 60000, 11)
    assert chi2_p(first, p[0]) > 1e-4
    checked = 0
    for c, cnt in nxt.items():
        if cnt.sum() >= 2000:
            assert chi2_p(cnt, p[c + 1]) > 1e-4, c
            checked += 1
    assert checked >= 3


def test_planted_mistake_is_caught(monkeypatch):
    """Later siblings tried against p instead of the residual: the first token is biased."""
    p, q = laws(3)
    monkeypatch.setattr(tree, "next_law", lambda w, q_: w)
    first, _ = run_cycles(p, q, 20000, 12)
    assert chi2_p(first, p[0]) < 1e-6


def test_leaf_bonus_and_duplicate_siblings():
    # root with two children carrying the same token 1; p(1) < q(1), so a rejection of the
    # first leaves residual weight 0 at token 1 and the second try cannot accept
    p0 = np.array([0.5, 0.1, 0.4])
    q0 = np.array([0.2, 0.6, 0.2])
    tgt = np.stack([logits_of(p0), logits_of([0.2, 0.3, 0.5]), logits_of([0.6, 0.2, 0.2])])
    dft = np.stack([logits_of(q0), logits_of([1 / 3] * 3), logits_of([1 / 3] * 3)])
    parent = [-1, -1]
    a1 = 0.1 / 0.6
    r = tree.step(parent, tgt, dft, [1, 1], np.array([a1 + 0.01, 0.0, 0.3], np.float32))
    assert r["n"] == 0
    w = accept.residual_weights(p0, q0) / accept.residual_weights(p0, q0).sum()  # (0.3, 0, 0.2)/0.5
    assert w[1] == 0.0
    t, _ = accept.inverse_cdf(w, np.float32(0.3))
    assert r["out_tokens"][0] == t == 0
    # acceptance of the first child: the path moves to node 0, a leaf: bonus draw from row 1
    r = tree.step(parent, tgt, dft, [1, 1], np.array([a1 - 0.01, 0.9, 0.7], np.float32))
    assert r["n"] == 1 and r["out_tokens"][0] == 1 and list(r["nodes"]) == [0]
    t, _ = accept.inverse_cdf(np.array([0.2, 0.3, 0.5]), np.float32(0.7))
    assert r["out_tokens"][1] == t == 2


def test_flags_and_zero_draw():
    tgt = np.stack([logits_of([0.25, 0.25, 0.5]), logits_of([0.5, 0.5, 0.0])])
    dft = np.stack([logits_of([0.0, 0.5, 0.5]), logits_of([0.5, 0.5, 0.0])])
    # q(0) = 0: acceptance 0, flagged, rejected even at u = 0; the draw then uses the residual
    r = tree.step([-1], tgt, dft, [0], np.zeros(2, np.float32))
    assert r["n"] == 0 and r["flags"] == tree.FLAG_Q_ZERO
    w = accept.residual_weights(np.array([0.25, 0.25, 0.5]), np.array([0.0, 0.5, 0.5]))
    assert r["out_tokens"][0] == int(np.nonzero(w > 0)[0][0]) == 0   # u = 0: first positive token
    r = tree.step([-1], tgt, dft, [7], np.zeros(2, np.float32))
    assert r["n"] == 0 and r["flags"] == tree.FLAG_TOKEN_RANGE
    bad = tgt.copy()
    bad[1, 2] = np.nan
    r = tree.step([-1], bad, dft, [1], np.zeros(2, np.float32))
    assert r["flags"] == tree.FLAG_NONFINITE and r["n"] == 0 and np.all(r["out_tokens"] == -1)
