"""Seeded synthetic inputs shared by the oracle-side tests and the GPU side.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic: no E2M1/E8M0 coding, no softmax, no acceptance rule. The
oracle and the HIP path both take their inputs from here and from nowhere else.

Every stream comes from ``numpy.random.default_rng([config, role, index, sub])``
so any piece (one matrix, one row chunk, one sequence) can be regenerated alone.

Workload shapes and distributions follow the verification-step workloads
(weights N(0, 0.02) as a standard deviation, bf16 activations N(0, 1), logits
N(0, sigma) with a target = draft + N(0, sigma') perturbation).
"""
from __future__ import annotations

import numpy as np

# role ids of the seed tuple
ROLE_W = 0          # fp32 weights
ROLE_X = 1          # activations
ROLE_OUTLIER = 2    # choice of outlier input channels
ROLE_BASE = 3       # base (draft) logits
ROLE_NOISE = 4      # target = base + noise
ROLE_DRAFT = 5      # draft-token sampling noise (Gumbel)
ROLE_U = 6          # uniforms handed to the acceptance kernel
ROLE_MASK = 7       # token masks (grammar-mask stand-in)

W_CHUNK_ROWS = 256  # weights are drawn in row chunks so any row range regenerates alone


def rng(config: int, role: int, index: int = 0, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(config), int(role), int(index), int(sub)])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest even) and return the uint16 bit patterns.

    Input preparation only: activations are defined as bf16 numbers, so the
    generator draws fp32 normals and stores their nearest bf16 values. NaN is
    not expected from a normal draw and is not special-cased.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def outlier_columns(config: int, index: int, k: int, frac: float) -> np.ndarray:
    """Sorted input-channel indices scaled as outliers (1% of K for the 70B-class set)."""
    count = int(round(k * frac))
    if count == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(rng(config, ROLE_OUTLIER, index).choice(k, size=count, replace=False))


def weights(config: int, index: int, n: int, k: int, sigma: float = 0.02,
            outlier_frac: float = 0.0, outlier_mul: float = 20.0,
            row_start: int = 0, row_stop: int | None = None) -> np.ndarray:
    """fp32 W[row_start:row_stop, :k] of an [n, k] weight matrix ~ N(0, sigma).

    Rows are drawn in chunks of W_CHUNK_ROWS with their own seed, so a row range
    regenerates identically whatever range it is requested in. With
    outlier_frac > 0 the chosen input channels (columns) are multiplied by
    outlier_mul in every row.
    """
    row_stop = n if row_stop is None else row_stop
    if not (0 <= row_start <= row_stop <= n):
        raise ValueError("bad row range")
    out = np.empty((row_stop - row_start, k), dtype=np.float32)
    c0 = row_start // W_CHUNK_ROWS
    c1 = (row_stop + W_CHUNK_ROWS - 1) // W_CHUNK_ROWS
    for c in range(c0, c1):
        lo = c * W_CHUNK_ROWS
        hi = min(n, lo + W_CHUNK_ROWS)
        blk = rng(config, ROLE_W, index, c).standard_normal((hi - lo, k), dtype=np.float32)
        blk *= np.float32(sigma)
        a, b = max(lo, row_start), min(hi, row_stop)
        out[a - row_start:b - row_start] = blk[a - lo:b - lo]
    if outlier_frac > 0:
        cols = outlier_columns(config, index, k, outlier_frac)
        out[:, cols] *= np.float32(outlier_mul)
    return out


def activations(config: int, index: int, m: int, k: int, sigma: float = 1.0) -> np.ndarray:
    """bf16 activations X[m, k] ~ N(0, sigma), returned as uint16 bit patterns."""
    x = rng(config, ROLE_X, index).standard_normal((m, k), dtype=np.float32) * np.float32(sigma)
    return f32_to_bf16_bits(x)


def logits(config: int, seq: int, kd: int, v: int, base_sigma: float, noise_sigma: float):
    """(target [kd+1, v], draft [kd, v]) fp32 logits for one sequence.

    Base logits are drawn for all kd+1 positions; the draft uses rows 0..kd-1
    of the base and the target is base + N(0, noise_sigma) on every row, so
    target row kd is the next-position (bonus) law.
    """
    base = rng(config, ROLE_BASE, seq).standard_normal((kd + 1, v), dtype=np.float32)
    base *= np.float32(base_sigma)
    noise = rng(config, ROLE_NOISE, seq).standard_normal((kd + 1, v), dtype=np.float32)
    target = base + noise * np.float32(noise_sigma)
    draft = base[:kd].copy()
    return target.astype(np.float32), draft.astype(np.float32)


def gumbel_tokens(config: int, seq: int, draft: np.ndarray) -> np.ndarray:
    """Draft tokens x_i drawn from each draft row's law by the Gumbel-max trick.

    argmax(z + G) with G i.i.d. standard Gumbel is a draw from the softmax of z,
    so the proposer's sampling needs no probability computation here. Rows that
    are entirely -inf have no law; they get token 0.
    """
    kd, v = draft.shape
    if kd == 0:
        return np.zeros(0, dtype=np.int32)
    g = rng(config, ROLE_DRAFT, seq).gumbel(size=(kd, v))
    z = draft.astype(np.float64) + g
    return np.argmax(z, axis=1).astype(np.int32)


def uniforms(config: int, seq: int, kd: int) -> np.ndarray:
    """kd+1 fp32 uniforms in [0, 1): u[i < kd] for the acceptance tests, u[kd] for the one final draw."""
    return rng(config, ROLE_U, seq).random(kd + 1, dtype=np.float32)


def accept_batch(config: int, b: int, kd: int, v: int, base_sigma: float, noise_sigma: float,
                 seq0: int = 0):
    """Stacked inputs for b sequences (per-sequence seeds seq0..seq0+b-1).

    Returns target [b, kd+1, v], draft [b, kd, v], tokens [b, kd] int32, u [b, kd+1] fp32.
    """
    tgt = np.empty((b, kd + 1, v), dtype=np.float32)
    dft = np.empty((b, kd, v), dtype=np.float32)
    tok = np.empty((b, kd), dtype=np.int32)
    uni = np.empty((b, kd + 1), dtype=np.float32)
    for i in range(b):
        t, d = logits(config, seq0 + i, kd, v, base_sigma, noise_sigma)
        tgt[i], dft[i] = t, d
        tok[i] = gumbel_tokens(config, seq0 + i, d)
        uni[i] = uniforms(config, seq0 + i, kd)
    return tgt, dft, tok, uni


def token_mask(config: int, seq: int, rows: int, v: int, keep_frac: float) -> np.ndarray:
    """bool [rows, v]: each token allowed independently with probability keep_frac."""
    return rng(config, ROLE_MASK, seq).random((rows, v)) < keep_frac


def pack_mask(mask) -> np.ndarray:
    """bool [..., V] -> uint32 [..., ceil(V/32)] in the library's mask layout: token t is
    bit t % 32 of word t // 32 (1 = allowed)."""
    mask = np.asarray(mask, dtype=bool)
    v = mask.shape[-1]
    w = (v + 31) // 32
    pad = np.zeros(mask.shape[:-1] + (w * 32,), dtype=bool)
    pad[..., :v] = mask
    bits = pad.reshape(mask.shape[:-1] + (w, 32)).astype(np.uint64)
    return (bits << np.arange(32, dtype=np.uint64)).sum(axis=-1).astype(np.uint32)


def tree_batch(config: int, b: int, parent, v: int, base_sigma: float, noise_sigma: float, seq0: int = 0):
    """Inputs of b verification cycles over one tree of N = len(parent) draft nodes.

    Rows 0..N of each sequence are the laws of the root's history (row 0) and of the history
    ending in node i (row i + 1). Base logits are drawn for every row; the draft rows are the
    base and the target rows base + N(0, noise_sigma). Node i's token is drawn from the draft
    row of its parent (row parent[i] + 1) by the Gumbel-max trick, independently for every
    node (siblings are independent draws, with replacement).

    Returns target, draft [b, N+1, v] fp32, tokens [b, N] int32, u [b, N+1] fp32.
    """
    parent = [int(p) for p in parent]
    n = len(parent)
    tgt = np.empty((b, n + 1, v), dtype=np.float32)
    dft = np.empty((b, n + 1, v), dtype=np.float32)
    tok = np.empty((b, n), dtype=np.int32)
    uni = np.empty((b, n + 1), dtype=np.float32)
    for i in range(b):
        s = seq0 + i
        base = rng(config, ROLE_BASE, s).standard_normal((n + 1, v), dtype=np.float32) * np.float32(base_sigma)
        noise = rng(config, ROLE_NOISE, s).standard_normal((n + 1, v), dtype=np.float32)
        tgt[i] = base + noise * np.float32(noise_sigma)
        dft[i] = base
        if n:
            g = rng(config, ROLE_DRAFT, s).gumbel(size=(n, v))
            for c in range(n):
                tok[i, c] = int(np.argmax(base[parent[c] + 1].astype(np.float64) + g[c]))
        uni[i] = rng(config, ROLE_U, s).random(n + 1, dtype=np.float32)
    return tgt, dft, tok, uni
