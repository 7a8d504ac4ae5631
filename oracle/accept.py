"""Speculative acceptance step (oracle). Test infrastructure only.

Written from the Module 11 lecture "Speculative Decoding and Quantization":

* §4 "The exact propose–verify–correct cycle": p_i and q_i are the laws the
  tokens are sampled from (here the softmax of the given logits, temperature 1,
  no filtering); draft token x_i is accepted with probability
  a(x_i) = min(1, p_i(x_i)/q_i(x_i)); positions are checked left to right; at
  the first rejection the rest of the draft is dropped and one token is drawn
  from r = norm((p - q)_+) at that position; if every draft token survives,
  one bonus token is drawn from the next-position target law.
* §5 and its B18 bridge: a token with q(t) = 0 never has p/q evaluated (its
  acceptance is 0); a draw u is accepted only when u < a (strictly), so u = 0
  still rejects a zero-acceptance proposal; a tiny residual stays a proper law.
* §13: malformed inputs are refused and reported, never repaired.

Random numbers are supplied, not drawn: u[i] (i < K) is the acceptance draw
of position i and u[K] is the single draw of the final token, taken by
inverse CDF: t* = min{t : u * Z < C_t} with C the inclusive prefix sums of
the (unnormalised) final weights w and Z = sum(w). If rounding leaves no such
t, the last token with w > 0 is taken. This consumption order is a convention
(the lecture notes that equality in law does not fix how random numbers are
used), so bit-exact comparison is against this oracle.

Floating point: logits are fp32 inputs; everything after is fp64.
"""
from __future__ import annotations

import numpy as np

FLAG_NONFINITE = 1       # a NaN/+inf logit, or a row with no finite logit
FLAG_TOKEN_RANGE = 2     # a draft token outside [0, V)
FLAG_Q_ZERO = 4          # a draft token the draft law gives probability 0
FLAG_RESIDUAL_ZERO = 8   # rejection with zero residual mass (rounding); drew from p instead

MARGIN = 1e-6            # decisions this close to u are "flagged", not compared


def softmax(z: np.ndarray):
    """Law of one logit row in fp64: exp(z - max z) / sum. None if the row is invalid.

    -inf logits are allowed (masked tokens get probability 0). A NaN or +inf
    logit, or a row whose largest logit is -inf, is invalid.
    """
    z = np.asarray(z, dtype=np.float32).astype(np.float64)
    if np.isnan(z).any() or np.isposinf(z).any():
        return None
    m = z.max()
    if m == -np.inf:
        return None
    e = np.exp(z - m)
    return e / e.sum()


def acceptance(p: np.ndarray, q: np.ndarray, x: int) -> tuple[float, int]:
    """a(x) = min(1, p(x)/q(x)) and any flags; a = 0 where q(x) = 0 or x is out of range."""
    if not 0 <= x < p.size:
        return 0.0, FLAG_TOKEN_RANGE
    if q[x] == 0.0:
        return 0.0, FLAG_Q_ZERO
    return min(1.0, p[x] / q[x]), 0


def residual_weights(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Unnormalised residual (p - q)_+ ."""
    return np.maximum(p - q, 0.0)


def overlap_mass(p: np.ndarray, q: np.ndarray) -> float:
    """alpha = sum_t min(p_t, q_t), the expected acceptance probability at a position."""
    return float(np.minimum(p, q).sum())


def inverse_cdf(w: np.ndarray, u: float) -> tuple[int, float]:
    """(t*, margin) for weights w >= 0 with sum Z > 0 and one uniform u.

    t* = min{t : u*Z < C_t}; if none, the last t with w_t > 0. The margin is
    the distance of u*Z to the nearest boundary of t*'s interval, over Z.
    """
    c = np.cumsum(w)
    z = c[-1]
    uz = float(u) * z
    hit = np.nonzero(uz < c)[0]
    if hit.size == 0:
        pos = np.nonzero(w > 0)[0]
        return int(pos[-1]), 0.0
    t = int(hit[0])
    below = c[t - 1] if t > 0 else 0.0
    margin = min(uz - below, c[t] - uz) / z
    return t, float(margin)


def step(target: np.ndarray, draft: np.ndarray, tokens: np.ndarray, u: np.ndarray) -> dict:
    """One verification cycle of one sequence.

    target [K+1, V] and draft [K, V] fp32 logits, tokens [K] int draft tokens
    (drawn from the draft laws by the caller), u [K+1] fp32 uniforms.

    Returns out_tokens [K+1] (first n+1 valid, rest -1), n (accepted drafts),
    flags, flagged (a decision or the final draw was within MARGIN of u), the
    smallest such distance (margin) and the per-position acceptance
    probabilities that were evaluated.
    """
    target = np.asarray(target, dtype=np.float32)
    draft = np.asarray(draft, dtype=np.float32)
    kd = draft.shape[0]
    v = target.shape[1]
    if target.shape != (kd + 1, v) or draft.shape != (kd, v) or len(tokens) != kd or len(u) != kd + 1:
        raise ValueError("shape mismatch")
    p_rows = [softmax(target[i]) for i in range(kd + 1)]
    q_rows = [softmax(draft[i]) for i in range(kd)]
    return step_laws(p_rows, q_rows, tokens, u)


def step_laws(p_rows, q_rows, tokens, u) -> dict:
    """The cycle of step() on given laws: p_rows [K+1] target laws, q_rows [K] draft laws
    (fp64 rows over one vocabulary, or None for an invalid row)."""
    kd = len(q_rows)
    if len(p_rows) != kd + 1 or len(tokens) != kd or len(u) != kd + 1:
        raise ValueError("shape mismatch")
    out = np.full(kd + 1, -1, dtype=np.int32)
    if any(r is None for r in p_rows + q_rows):
        return dict(out_tokens=out, n=0, flags=FLAG_NONFINITE, flagged=False, margin=np.inf, a=[])

    flags = 0
    margin_min = np.inf
    a_seen = []
    n = kd
    for i in range(kd):
        x = int(tokens[i])
        a, f = acceptance(p_rows[i], q_rows[i], x)
        flags |= f
        a_seen.append(a)
        ui = float(u[i])
        margin_min = min(margin_min, abs(ui - a))
        if ui < a:
            out[i] = x
            continue
        n = i
        break

    if n < kd:
        w = residual_weights(p_rows[n], q_rows[n])
        if not w.sum() > 0.0:
            flags |= FLAG_RESIDUAL_ZERO
            w = p_rows[n]
    else:
        w = p_rows[kd]
    t, margin = inverse_cdf(w, float(u[kd]))
    margin_min = min(margin_min, margin)
    out[n] = t
    return dict(out_tokens=out, n=n, flags=flags, flagged=bool(margin_min < MARGIN),
                margin=margin_min, a=a_seen)


def step_batch(target: np.ndarray, draft: np.ndarray, tokens: np.ndarray, u: np.ndarray) -> dict:
    """step() for b independent sequences: target [b, K+1, V], draft [b, K, V], tokens [b, K], u [b, K+1]."""
    b = target.shape[0]
    kd = draft.shape[1]
    out = np.full((b, kd + 1), -1, dtype=np.int32)
    n = np.zeros(b, dtype=np.int32)
    flags = np.zeros(b, dtype=np.int32)
    flagged = np.zeros(b, dtype=bool)
    margin = np.zeros(b)
    for s in range(b):
        r = step(target[s], draft[s], tokens[s], u[s])
        out[s], n[s], flags[s], flagged[s], margin[s] = (r["out_tokens"], r["n"], r["flags"],
                                                         r["flagged"], r["margin"])
    return dict(out_tokens=out, n=n, flags=flags, flagged=flagged, margin=margin)


def residual_law(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """norm((p - q)_+); a zero vector when there is no positive part (then rejection cannot occur)."""
    w = residual_weights(p, q)
    z = w.sum()
    return w / z if z > 0 else np.zeros_like(w)
