"""Pins of the sampling-transform oracle (oracle/sampling.py) against things it does not compute
itself: closed forms, direct enumeration, hand-worked cases, and the law the accept loop must
preserve once the transforms are on."""
import numpy as np
import pytest

import synth
from oracle import accept as oacc
from oracle import sampling as osm


def _logits(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, np.float64)).astype(np.float32)


def test_defaults_are_the_plain_softmax():
    z = synth.rng(11, 3).standard_normal(300).astype(np.float32) * np.float32(2.5)
    law, margin = osm.transformed_law(z)
    assert np.array_equal(law, oacc.softmax(z)) and margin == np.inf


@pytest.mark.parametrize("tau", [0.25, 0.7, 1.0, 1.6, 4.0])
def test_temperature_closed_form(tau):
    """softmax(z / tau) = p^(1/tau) / sum p^(1/tau) with p = softmax(z)."""
    z = synth.rng(12, 3).standard_normal(500).astype(np.float32) * np.float32(2.0)
    p = oacc.softmax(z)
    want = p ** (1.0 / np.float64(np.float32(tau)))   # tau is an fp32 argument
    want /= want.sum()
    law, _ = osm.transformed_law(z, temperature=tau)
    np.testing.assert_allclose(law, want, rtol=1e-10, atol=1e-300)


def test_low_temperature_concentrates_on_the_argmax():
    z = synth.rng(13, 3).standard_normal(64).astype(np.float32)
    law, _ = osm.transformed_law(z, temperature=1e-3)
    assert law[np.argmax(z)] > 1 - 1e-12


@pytest.mark.parametrize("seed", range(6))
def test_top_k_matches_enumeration_with_ties(seed):
    """Integer logits make ties; the kept set must equal the count-of-strictly-larger rule."""
    r = synth.rng(14, 3, seed)
    z = r.integers(-4, 5, size=23).astype(np.float32)
    allowed = r.random(23) < 0.8
    for k in [1, 2, 3, 5, 8, 22, 23, 40]:
        law, _ = osm.transformed_law(z, top_k=k, allowed=allowed)
        kept = sorted(np.nonzero(law > 0)[0].tolist())
        assert kept == osm.kept_set_brute(z, top_k=k, allowed=allowed), (seed, k)
        assert np.nonzero(osm.kept_set(z, top_k=k, allowed=allowed)[0])[0].tolist() == kept
        # ties included: at least min(k, allowed) tokens, and every kept token beats every dropped one
        assert len(kept) >= min(k, int(allowed.sum()))
        dropped = [t for t in range(23) if allowed[t] and t not in kept]
        if dropped and kept:
            assert z[kept].min() > z[dropped].max()


def test_kept_set_keeps_tokens_whose_weight_underflows():
    """top-k keeps a token whose e_t underflows to 0 (logits 2000 apart): it is in the kept set
    (so a sampler's support and a threshold include it) though the law gives it 0."""
    z = np.array([0.0, -2000.0, -3000.0, 5.0], np.float32)
    keep, e, _ = osm.kept_set(z, top_k=3)
    assert np.nonzero(keep)[0].tolist() == osm.kept_set_brute(z, top_k=3) == [0, 1, 3]
    assert e[1] == 0.0 and e[3] == 1.0
    law, _ = osm.transformed_law(z, top_k=3)
    assert law[1] == 0.0


def test_top_k_without_ties_keeps_exactly_k():
    z = synth.rng(15, 3).permutation(100).astype(np.float32)
    for k in [1, 7, 50, 99]:
        law, _ = osm.transformed_law(z, top_k=k)
        assert np.count_nonzero(law) == k
        assert set(np.argsort(-z)[:k].tolist()) == set(np.nonzero(law)[0].tolist())


def test_top_p_hand_worked():
    """p = (0.5, 0.3, 0.1, 0.1): the mass strictly above each token is 0, 0.5, 0.8, 0.8."""
    z = _logits([0.5, 0.3, 0.1, 0.1])
    cases = {0.45: [1.0, 0.0, 0.0, 0.0],           # 0.5 >= 0.45: token 1 dropped
             0.75: [0.625, 0.375, 0.0, 0.0],      # 0.8 >= 0.75: both tied tokens dropped
             0.85: [0.5, 0.3, 0.1, 0.1]}          # 0.8 < 0.85: both tied tokens kept
    for P, want in cases.items():
        law, margin = osm.transformed_law(z, top_p=P)
        np.testing.assert_allclose(law, want, rtol=1e-6, atol=1e-7)
        assert margin > 1e-3


def test_top_p_acts_on_the_top_k_law():
    """p = (0.4, 0.3, 0.2, 0.1), k = 2, P = 0.5: after top-k the law is (4/7, 3/7), the mass above
    token 1 is 4/7 >= 0.5, so only token 0 survives; on the untruncated law token 1 would stay
    (0.4 < 0.5). Pins the order top-k -> renormalise -> top-p."""
    z = _logits([0.4, 0.3, 0.2, 0.1])
    law, _ = osm.transformed_law(z, top_k=2, top_p=0.5)
    np.testing.assert_allclose(law, [1.0, 0.0, 0.0, 0.0])
    law, _ = osm.transformed_law(z, top_p=0.5)
    np.testing.assert_allclose(law, [4 / 7, 3 / 7, 0.0, 0.0], rtol=1e-6)


@pytest.mark.parametrize("seed", range(6))
def test_top_p_matches_enumeration(seed):
    r = synth.rng(16, 3, seed)
    z = (r.integers(-6, 7, size=31) * 0.5).astype(np.float32)
    allowed = r.random(31) < 0.9
    for tau in [0.6, 1.0, 1.7]:
        for k in [0, 4, 12]:
            for P in [0.05, 0.3, 0.6, 0.9, 0.999]:
                law, margin = osm.transformed_law(z, temperature=tau, top_k=k, top_p=P, allowed=allowed)
                if margin < 1e-9:
                    continue
                kept = sorted(np.nonzero(law > 0)[0].tolist())
                assert kept == osm.kept_set_brute(z, top_k=k, top_p=P, allowed=allowed, temperature=tau), \
                    (seed, tau, k, P)
                keep = osm.kept_set(z, temperature=tau, top_k=k, top_p=P, allowed=allowed)[0]
                assert np.nonzero(keep)[0].tolist() == kept


def test_top_p_kept_mass_reaches_p_minimally():
    """Without ties: the kept set is the shortest most-probable prefix with mass >= P."""
    z = synth.rng(17, 3).standard_normal(400).astype(np.float32) * np.float32(2.0)
    p = oacc.softmax(z)
    for P in [0.1, 0.5, 0.9, 0.99]:
        law, _ = osm.transformed_law(z, top_p=P)
        kept = np.nonzero(law)[0]
        order = np.argsort(-p)
        c = np.cumsum(p[order])
        n_min = int(np.searchsorted(c, np.float32(P), side="left")) + 1
        assert kept.size == n_min
        assert set(kept.tolist()) == set(order[:n_min].tolist())


def test_mask_is_renormalised_softmax_over_allowed():
    z = synth.rng(18, 3).standard_normal(200).astype(np.float32)
    allowed = synth.token_mask(18, 0, 1, 200, 0.3)[0]
    law, _ = osm.transformed_law(z, allowed=allowed)
    want = np.where(allowed, np.exp(z.astype(np.float64) - z[allowed].max()), 0.0)
    np.testing.assert_allclose(law, want / want.sum(), rtol=1e-12, atol=1e-300)
    assert osm.transformed_law(z, allowed=np.zeros(200, bool))[0] is None


def test_invalid_rows():
    z = np.zeros(8, np.float32)
    z[3] = np.nan
    assert osm.transformed_law(z)[0] is None
    z[3] = np.inf
    assert osm.transformed_law(z)[0] is None


def _gumbel_draw(law, g):
    with np.errstate(divide="ignore"):
        return int(np.argmax(np.log(law) + g))


def _cycles(n_cycles, transformed_acceptance, seed=19):
    """Emitted token at position 0 over many cycles with tokens drawn from the transformed
    draft law. transformed_acceptance=False runs the acceptance on the raw laws instead."""
    v, kd = 8, 2
    tau, k, P = 0.7, 5, 0.8
    r = synth.rng(seed, 3)
    base = r.standard_normal((kd + 1, v)).astype(np.float32) * np.float32(1.5)
    target = (base + r.standard_normal((kd + 1, v)).astype(np.float32)).astype(np.float32)
    draft = base[:kd].copy()
    mask = np.ones((kd + 1, v), bool)
    mask[0, 6] = False
    mask[1, 2] = False
    q = [osm.transformed_law(draft[i], tau, k, P, mask[i])[0] for i in range(kd)]
    p0 = osm.transformed_law(target[0], tau, k, P, mask[0])[0]
    counts = np.zeros(v)
    rr = synth.rng(seed, 6)
    for _ in range(n_cycles):
        g = rr.gumbel(size=(kd, v))
        tok = np.array([_gumbel_draw(q[i], g[i]) for i in range(kd)], np.int32)
        u = rr.random(kd + 1).astype(np.float32)
        if transformed_acceptance:
            res = osm.step_sampled(target, draft, tok, u, tau, k, P, mask)
        else:
            res = oacc.step(target, draft, tok, u)
        counts[res["out_tokens"][0]] += 1
    return counts, p0


def _chi2_pvalue(counts, law):
    from scipy.stats import chi2
    n = counts.sum()
    live = law > 0
    exp = law[live] * n
    stat = ((counts[live] - exp) ** 2 / exp).sum() + (np.inf if counts[~live].sum() else 0.0)
    return float(chi2.sf(stat, live.sum() - 1))


def test_transformed_laws_are_preserved_chi_square():
    """Position 0's emitted token follows the transformed target law p_0 (including tokens the
    transforms remove, which must never appear)."""
    counts, p0 = _cycles(30000, True)
    assert _chi2_pvalue(counts, p0) > 1e-4


def test_raw_laws_break_the_guarantee():
    """Negative control: accepting with the raw laws while the draft samples from the
    transformed one does not reproduce p_0 (the lecture's warning); the test above is not vacuous."""
    counts, p0 = _cycles(30000, False)
    assert _chi2_pvalue(counts, p0) < 1e-6


def test_pack_mask_layout():
    m = np.zeros(40, bool)
    m[[0, 5, 31, 32, 39]] = True
    assert synth.pack_mask(m).tolist() == [1 + 32 + 2 ** 31, 1 + 128]
