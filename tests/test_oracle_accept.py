"""Pins of the oracle's acceptance step.

* worked example A: overlap 0.85, TV 0.15, residual e_0, exact balance;
* the B18 edge cases: p = q never rejects, q(t) = 0 never evaluates p/q, a tiny
  residual stays a law, a zero draw rejects a zero-acceptance proposal;
* hand-worked cycles that fix the uniform-consumption convention and the
  inverse-CDF rule (including zero weights and u = 0);
* law preservation: exact piecewise quadrature over (u_0, u_K) and a Pearson
  chi-square on brute-force cycles at every position, bonus row included;
* expected tokens per cycle against the closed form (Monte Carlo, 4 s.e.).
"""
import numpy as np
import pytest
from scipy import stats

from oracle import accept, expect
from tests.conftest import golden


def logits_of(p):
    """fp32 logits whose softmax is p (log p; -inf where p = 0)."""
    p = np.asarray(p, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return np.log(p).astype(np.float32)


def test_worked_example_a():
    g = golden("worked_example_a.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    assert accept.overlap_mass(p, q) == pytest.approx(g["alpha"], abs=1e-15)
    assert 0.5 * np.abs(p - q).sum() == pytest.approx(g["tv"], abs=1e-15)
    assert 1 - accept.overlap_mass(p, q) == pytest.approx(g["tv"], abs=1e-15)
    r = accept.residual_law(p, q)
    assert np.array_equal(r, np.array(g["residual"], float))
    rho = accept.residual_weights(p, q).sum()
    assert rho == pytest.approx(g["rejection_mass"], abs=1e-15)
    balance = np.minimum(p, q) + (1 - accept.overlap_mass(p, q)) * r
    np.testing.assert_allclose(balance, p, rtol=0, atol=1e-12)
    # acceptance probabilities min(1, p/q) token by token
    a = [accept.acceptance(p, q, t)[0] for t in range(5)]
    np.testing.assert_allclose(a, [1, 0.3 / 0.35, 0.75, 1, 0.5], rtol=1e-15)


def test_p_equals_q_never_rejects():
    rng = np.random.default_rng(0)
    z = rng.standard_normal((4, 16)).astype(np.float32)
    for _ in range(200):
        u = rng.random(4, dtype=np.float32)
        tok = rng.integers(0, 16, 3)
        r = accept.step(z, z[:3], tok, u)
        assert r["n"] == 3 and list(r["out_tokens"][:3]) == list(tok)


def test_q_zero_never_divides():
    p = np.array([0.5, 0.5, 0.0])
    q = np.array([0.0, 0.5, 0.5])
    with np.errstate(all="raise"):
        a, f = accept.acceptance(p, q, 0)
    assert a == 0.0 and f == accept.FLAG_Q_ZERO
    # the missing mass comes back through the residual
    r = accept.residual_law(p, q)
    np.testing.assert_array_equal(r, [1.0, 0.0, 0.0])


def test_tiny_residual_stays_a_law():
    g = golden("b18_edge_cases.json")["tiny_residual"]
    p, q = np.array(g["p"]), np.array(g["q"])
    r = accept.residual_law(p, q)
    np.testing.assert_allclose(r, g["residual"], rtol=0, atol=g["atol"])
    bal = np.minimum(p, q) + accept.residual_weights(p, q).sum() * r
    np.testing.assert_allclose(bal, p, rtol=0, atol=g["atol"])


def test_zero_draw_rejects():
    g = golden("b18_edge_cases.json")["zero_draw"]
    target = np.stack([logits_of(g["p"]), logits_of(g["p"])])
    draft = logits_of(g["q"])[None]
    r = accept.step(target, draft, [g["proposal"]], np.array([g["u"], 0.0], np.float32))
    assert r["n"] == 0 and r["out_tokens"][0] == g["token"]
    assert (r["n"] > 0) == g["accepted"]


def test_uniform_consumption_convention():
    """Hand-worked: position 0 always accepts (p_0 = q_0), position 1 has a = 0.5.

    u = [0.3, 0.9, 0.6]: u_1 = 0.9 >= 0.5 rejects at 1; the residual at 1 is
    (p_1 - q_1)_+ = (0.25, 0, 0.25, 0), Z = 0.5, so u_2 * Z = 0.3 first falls
    below C = (0.25, 0.25, 0.5, 0.5) at t = 2. With u_1 = 0.2 the draft
    survives and the bonus row (1, 0, 0, 0) gives token 0.
    """
    p0 = [0.25, 0.25, 0.25, 0.25]
    q0 = [0.25, 0.25, 0.25, 0.25]
    p1 = [0.375, 0.125, 0.375, 0.125]
    q1 = [0.125, 0.25, 0.125, 0.5]      # x_1 = 1: a = 0.125 / 0.25 = 0.5
    p2 = [1.0, 0.0, 0.0, 0.0]
    target = np.stack([logits_of(p0), logits_of(p1), logits_of(p2)])
    draft = np.stack([logits_of(q0), logits_of(q1)])
    r = accept.step(target, draft, [2, 1], np.array([0.3, 0.9, 0.6], np.float32))
    assert r["n"] == 1 and list(r["out_tokens"]) == [2, 2, -1]
    assert r["a"][1] == pytest.approx(0.5, rel=1e-6)
    r = accept.step(target, draft, [2, 1], np.array([0.3, 0.2, 0.6], np.float32))
    assert r["n"] == 2 and list(r["out_tokens"]) == [2, 1, 0]
    # the final draw uses u[K], not u[0]: u_0 = 0 would pick token 0 of the residual
    r = accept.step(target, draft, [2, 1], np.array([0.0, 0.9, 0.6], np.float32))
    assert list(r["out_tokens"]) == [2, 2, -1]


def test_inverse_cdf_rule():
    w = np.array([0.0, 0.25, 0.0, 0.5, 0.25])          # dyadic: prefix sums are exact
    assert accept.inverse_cdf(w, 0.0)[0] == 1          # first positive weight
    assert accept.inverse_cdf(w, 0.2499)[0] == 1
    assert accept.inverse_cdf(w, 0.25)[0] == 3         # a boundary belongs to the next token
    assert accept.inverse_cdf(w, 0.7499)[0] == 3
    assert accept.inverse_cdf(w, 0.75)[0] == 4
    assert accept.inverse_cdf(w, 0.99999994)[0] == 4
    assert accept.inverse_cdf(w, 1.0)[0] == 4          # no crossing: last positive weight
    w2 = np.array([0.25, 0.75, 0.0, 0.0])
    assert accept.inverse_cdf(w2, 1.0)[0] == 1         # never a zero-weight token
    t, m = accept.inverse_cdf(w, 0.5)
    assert t == 3 and m == 0.25
    t, m = accept.inverse_cdf(2 * w, 0.5)              # unnormalised weights, same answer
    assert t == 3 and m == 0.25


def test_flags_and_invalid_rows():
    z = np.zeros((2, 4), np.float32)
    r = accept.step(z, z[:1], [7], np.array([0.5, 0.5], np.float32))
    assert r["flags"] & accept.FLAG_TOKEN_RANGE and r["n"] == 0
    bad = z.copy()
    bad[1, 2] = np.nan
    r = accept.step(bad, z[:1], [0], np.array([0.5, 0.5], np.float32))
    assert r["flags"] == accept.FLAG_NONFINITE and list(r["out_tokens"]) == [-1, -1]
    masked = np.full((1, 4), -np.inf, np.float32)
    r = accept.step(z, masked, [0], np.array([0.5, 0.5], np.float32))
    assert r["flags"] == accept.FLAG_NONFINITE
    # -inf logits are legal masks; a proposal the draft masks out is flagged and rejected
    dm = z[:1].copy()
    dm[0, 1] = -np.inf
    r = accept.step(z, dm, [1], np.array([0.0, 0.5], np.float32))
    assert r["flags"] & accept.FLAG_Q_ZERO and r["n"] == 0


def test_residual_zero_falls_back_to_p():
    """Rejection with no positive residual (only possible through rounding) draws from p."""
    p = np.array([0.5, 0.5])
    w = accept.residual_weights(p, p)
    assert w.sum() == 0
    target = np.stack([logits_of(p), logits_of(p)])
    # a = 1 for equal laws; u >= 1 is outside [0, 1) and forces the rejection branch
    r = accept.step(target, target[:1], [0], np.array([1.0, 0.75], np.float32))
    assert r["flags"] & accept.FLAG_RESIDUAL_ZERO
    assert r["out_tokens"][0] == 1


# ------------------------------------------------------------ law preservation
def _exact_position_law(p0, q0, p1):
    """Exact law of the token emitted at position 0 of a K=1 cycle, by piecewise quadrature.

    The cycle is piecewise constant in (u_0, u_1); breakpoints are a(x) for u_0
    and the normalised CDF of the final weights for u_1, computed here from
    p and q directly. Each cell is evaluated once at its midpoint by the oracle.
    """
    v = len(p0)
    law0 = np.zeros(v)
    target = np.stack([logits_of(p0), logits_of(p1)])
    draft = logits_of(q0)[None]
    res = np.maximum(np.asarray(p0) - np.asarray(q0), 0)
    for x in range(v):
        if q0[x] == 0:
            continue
        a = min(1.0, p0[x] / q0[x])
        for lo0, hi0 in [(0.0, a), (a, 1.0)]:
            if hi0 <= lo0:
                continue
            u0 = 0.5 * (lo0 + hi0)
            w = res if u0 >= a else np.asarray(p1)
            cdf = np.concatenate([[0.0], np.cumsum(w) / w.sum()])
            for j in range(v):
                lo1, hi1 = cdf[j], cdf[j + 1]
                if hi1 <= lo1:
                    continue
                u1 = 0.5 * (lo1 + hi1)
                r = accept.step(target, draft, [x], np.array([u0, u1], np.float32))
                law0[r["out_tokens"][0]] += q0[x] * (hi0 - lo0) * (hi1 - lo1)
    return law0


def test_exact_quadrature_preserves_p():
    g = golden("worked_example_a.json")
    p, q = g["p"], g["q"]
    law = _exact_position_law(p, q, p)
    np.testing.assert_allclose(law, p, rtol=0, atol=1e-6)
    rng = np.random.default_rng(42)
    for _ in range(3):
        p0 = rng.dirichlet(np.ones(6))
        q0 = rng.dirichlet(np.ones(6))
        q0[2] = 0.0
        q0 /= q0.sum()
        law = _exact_position_law(p0, q0, p0)
        np.testing.assert_allclose(law, p0, rtol=0, atol=1e-6)


@pytest.mark.parametrize("case", ["example_a", "random_v8"])
def test_chi_square_every_position(case):
    kd = 3
    rng = np.random.default_rng(2024 if case == "example_a" else 2025)
    if case == "example_a":
        g = golden("worked_example_a.json")
        P = [np.array(g["p"])] * (kd + 1)
        Q = [np.array(g["q"])] * kd
    else:
        P = [rng.dirichlet(np.ones(8) * 0.7) for _ in range(kd + 1)]
        Q = [rng.dirichlet(np.ones(8) * 0.7) for _ in range(kd)]
    v = len(P[0])
    target = np.stack([logits_of(p) for p in P])
    draft = np.stack([logits_of(q) for q in Q])
    # the laws the oracle actually sees after the fp32 logit round trip
    Pe = [accept.softmax(r) for r in target]
    Qe = [accept.softmax(r) for r in draft]
    trials = 40000
    counts = np.zeros((kd + 1, v))
    toks = np.stack([rng.choice(v, size=trials, p=Qe[i]) for i in range(kd)], axis=1)
    us = rng.random((trials, kd + 1), dtype=np.float32)
    for j in range(trials):
        r = accept.step(target, draft, toks[j], us[j])
        for i in range(r["n"] + 1):
            counts[i, r["out_tokens"][i]] += 1
    for i in range(kd + 1):
        reached = counts[i].sum()
        assert reached > 1000
        exp_counts = reached * Pe[i]
        keep = exp_counts > 0
        chi2 = (((counts[i] - exp_counts)[keep]) ** 2 / exp_counts[keep]).sum()
        pval = stats.chi2.sf(chi2, keep.sum() - 1)
        assert pval > 1e-4, (i, chi2, pval)


def test_expected_tokens_closed_form_monte_carlo():
    """Same law pair at every position -> i.i.d. acceptance alpha -> E = (1 - a^(K+1)) / (1 - a)."""
    g = golden("worked_example_a.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    kd = 4
    target = np.stack([logits_of(p)] * (kd + 1))
    draft = np.stack([logits_of(q)] * kd)
    pe, qe = accept.softmax(target[0]), accept.softmax(draft[0])
    alpha = accept.overlap_mass(pe, qe)
    rng = np.random.default_rng(77)
    trials = 20000
    emitted = np.empty(trials)
    toks = rng.choice(5, size=(trials, kd), p=qe)
    us = rng.random((trials, kd + 1), dtype=np.float32)
    for j in range(trials):
        r = accept.step(target, draft, toks[j], us[j])
        emitted[j] = r["n"] + 1
    e_closed = expect.expected_tokens(alpha, kd)
    se = emitted.std(ddof=1) / np.sqrt(trials)
    assert abs(emitted.mean() - e_closed) < 4 * se
    assert e_closed == pytest.approx(expect.expected_tokens_tail([alpha] * kd), rel=1e-14)


def test_softmax_shift_invariance_large_logits():
    """softmax(z + c) = softmax(z): logits near 800 must not overflow exp."""
    rng = np.random.default_rng(8)
    z = rng.standard_normal(50).astype(np.float32)
    p = accept.softmax(z)
    p_shift = accept.softmax(z + np.float32(800.0))
    assert np.isfinite(p_shift).all()
    np.testing.assert_allclose(p_shift, p, rtol=1e-4)   # fp32 rounding of z + 800
    np.testing.assert_allclose(accept.softmax(np.array([800.0, 800.0], np.float32)), [0.5, 0.5], rtol=0)
