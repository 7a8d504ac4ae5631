"""Sampling transforms of the speculative acceptance step (oracle). Test infrastructure only.

Written from the Module 11 lecture "Speculative Decoding and Quantization",
§4 (the laws p_i and q_i are the distributions tokens are actually sampled
from): temperature rescales the logits, top-k keeps the most probable tokens,
top-p keeps a smallest most-probable set whose mass reaches a chosen level,
and a grammar mask removes forbidden continuations. All of them are applied
to the target law and to the draft law alike (each law its own top-k / top-p
set, one mask per position shared by both), and the acceptance rule then uses
the transformed laws; with raw laws the exactness argument fails.

Readings where the lecture leaves a detail open (the plainest ones it
supports):

* Order: temperature, then top-k, then top-p (the order the lecture names),
  the mask first of all (a removed token is not a candidate for anything).
* Temperature tau > 0 (an fp32 number) divides the logits: y = z / tau (fp64).
* top-k (k >= 1; 0 = off) keeps token t iff fewer than k allowed tokens have
  a strictly larger logit: ties at the k-th value are all kept.
* top-p (0 < P < 1; P >= 1 = off) acts on the law left by top-k: with
  e_t = exp(y_t - max y) over the kept tokens and S = sum e, token t is kept
  iff the mass of kept tokens with a strictly larger logit is below P * S.
  Without ties this is the smallest most-probable prefix whose mass reaches
  P; tied tokens at the boundary are all kept.
* The resulting law is e_t / sum over the kept tokens, zero elsewhere.

Where floating point decides membership (the top-p comparison) the oracle
reports the distance of the boundary sum to P * S, relative to S, so a
comparison can set aside rows within rounding of a tie.

Floating point: logits are fp32 inputs, everything after is fp64.
"""
from __future__ import annotations

import numpy as np

from oracle import accept as acc

TOP_P_MARGIN = 1e-9   # top-p boundaries this close (relative to S) are "flagged", not compared


def transformed_law(z, temperature: float = 1.0, top_k: int = 0, top_p: float = 1.0, allowed=None):
    """(law, top_p_margin) of one fp32 logit row under the transforms; law is None if invalid.

    allowed: bool row (True = the mask keeps the token) or None. A NaN or +inf
    logit anywhere, or no allowed finite logit, makes the row invalid.
    """
    z = np.asarray(z, dtype=np.float32)
    if np.isnan(z).any() or np.isposinf(z).any():
        return None, np.inf
    keep, e, margin = kept_set(z, temperature, top_k, top_p, allowed)
    if not keep.any():
        return None, np.inf
    return e / e.sum(), margin


def kept_set(z, temperature: float = 1.0, top_k: int = 0, top_p: float = 1.0, allowed=None):
    """(keep, e, top_p_margin): the tokens the transforms keep (bool row), their weights
    e_t = exp(y_t - max y) (0 elsewhere) and the top-p margin, for a row whose finite logits
    are the candidates (non-finite logits are never kept)."""
    z = np.asarray(z, dtype=np.float32)
    keep = np.isfinite(z)
    if allowed is not None:
        keep &= np.asarray(allowed, dtype=bool)
    if not keep.any():
        return keep, np.zeros(z.shape, np.float64), np.inf
    zk = z.astype(np.float64)

    # top-k on the logits (dividing by tau > 0 keeps their order)
    if top_k > 0:
        vals = zk[keep]
        srt = np.sort(vals)[::-1]
        if top_k < srt.size:
            kth = srt[top_k - 1]
            # strictly larger count < k  <=>  value >= the k-th largest value
            keep &= zk >= kth

    y = zk / np.float64(np.float32(temperature))   # the temperature is an fp32 argument
    m = y[keep].max()
    e = np.where(keep, np.exp(np.where(keep, y - m, 0.0)), 0.0)

    margin = np.inf
    if top_p < 1.0:
        s1 = e.sum()
        bound = np.float64(np.float32(top_p)) * s1
        # mass strictly above each distinct kept value, summed from the top down
        idx = np.nonzero(keep)[0]
        order = idx[np.argsort(-zk[idx], kind="stable")]
        vals = zk[order]
        starts = np.r_[0, np.nonzero(vals[1:] != vals[:-1])[0] + 1]
        group_mass = np.add.reduceat(e[order], starts)
        above = np.r_[0.0, np.cumsum(group_mass)[:-1]]
        margin = float(np.min(np.abs(above - bound)) / s1)
        kept_vals = vals[starts][above < bound]
        keep &= np.isin(zk, kept_vals)
        e = np.where(keep, e, 0.0)

    return keep, e, margin


def kept_set_brute(z, top_k: int = 0, top_p: float = 1.0, allowed=None, temperature: float = 1.0):
    """The kept token set by direct enumeration (tiny rows): for each token, count and sum over
    every other token. Independent of transformed_law's sorting, for pinning it."""
    z = np.asarray(z, dtype=np.float32).astype(np.float64)
    v = z.size
    ok = np.isfinite(z) & (np.ones(v, bool) if allowed is None else np.asarray(allowed, bool))
    kept = []
    for t in range(v):
        if not ok[t]:
            continue
        larger = sum(1 for u in range(v) if ok[u] and z[u] > z[t])
        if top_k > 0 and larger >= top_k:
            continue
        kept.append(t)
    if top_p < 1.0:
        y = z / np.float64(np.float32(temperature))
        m = max(y[t] for t in kept)
        e = {t: np.exp(y[t] - m) for t in kept}
        s = sum(e.values())
        kept = [t for t in kept if sum(e[u] for u in kept if z[u] > z[t]) < np.float64(np.float32(top_p)) * s]
    return kept


def step_sampled(target, draft, tokens, u, temperature: float = 1.0, top_k: int = 0,
                 top_p: float = 1.0, mask=None) -> dict:
    """One verification cycle with transformed laws (acc.step's rule and uniform convention).

    mask: bool [K+1, V] or None; row i serves target row i and draft row i, row K the bonus row.
    The result is flagged when a decision or the final draw is within acc.MARGIN of u, or a
    top-p boundary of any evaluated row is within TOP_P_MARGIN of its tie.
    """
    target = np.asarray(target, dtype=np.float32)
    draft = np.asarray(draft, dtype=np.float32)
    kd = draft.shape[0]
    allow = (lambda i: None) if mask is None else (lambda i: np.asarray(mask)[i])
    p_rows, q_rows, margins = [], [], []
    for i in range(kd + 1):
        p, mg = transformed_law(target[i], temperature, top_k, top_p, allow(i))
        p_rows.append(p)
        margins.append(mg)
    for i in range(kd):
        q, mg = transformed_law(draft[i], temperature, top_k, top_p, allow(i))
        q_rows.append(q)
        margins.append(mg)
    r = acc.step_laws(p_rows, q_rows, tokens, u)
    top_margin = min(margins) if margins else np.inf
    r["top_p_margin"] = top_margin
    r["flagged"] = bool(r["flagged"] or top_margin < TOP_P_MARGIN)
    return r


def step_sampled_batch(target, draft, tokens, u, temperature=1.0, top_k=0, top_p=1.0, mask=None) -> dict:
    """step_sampled for b sequences; mask bool [b, K+1, V] or None."""
    b = target.shape[0]
    kd = draft.shape[1]
    out = np.full((b, kd + 1), -1, dtype=np.int32)
    n = np.zeros(b, dtype=np.int32)
    flags = np.zeros(b, dtype=np.int32)
    flagged = np.zeros(b, dtype=bool)
    margin = np.zeros(b)
    for s in range(b):
        r = step_sampled(target[s], draft[s], tokens[s], u[s], temperature, top_k, top_p,
                         None if mask is None else mask[s])
        out[s], n[s], flags[s], flagged[s], margin[s] = (r["out_tokens"], r["n"], r["flags"],
                                                         r["flagged"], r["margin"])
    return dict(out_tokens=out, n=n, flags=flags, flagged=flagged, margin=margin)
