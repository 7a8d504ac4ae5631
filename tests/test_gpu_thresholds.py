"""spec_sampling_thresholds on the GPU vs the oracle's kept sets.

A row's kept set on the device is {t : allowed, finite, key(z_t) >= threshold}; it must
equal oracle.sampling.kept_set token for token, except on rows whose top-p boundary lies
within 1e-9 of a tie (the oracle's margin), which are set aside. The inputs steer every
route of the selection: candidates collected after the first digit (top-k, top-p, both),
candidate lists too long for the workgroup (k = 9000; every logit in one bucket), top-k that
keeps every token under top-p, logit ranges where exp(z / tau) against 0 would leave fp64's
range, ties, vocabularies with ragged chunks or without vector loads, and rows with nothing
allowed.
"""
import numpy as np
import pytest
import torch

import mx_fp4_weight_amd as mxs
import synth
from oracle import sampling as osm
from tests.gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


def order_keys(z):
    """uint32 keys with the logits' order (-0 as +0): bits | 2^31 for z >= 0, ~bits below."""
    z = np.asarray(z, np.float32).copy()
    z[z == 0] = 0.0
    b = z.view(np.uint32)
    return np.where(b & np.uint32(0x80000000), ~b, b | np.uint32(0x80000000)).astype(np.uint32)


def device_thresholds(z, tau, k, p, allowed):
    m = None if allowed is None else dev(synth.pack_mask(allowed).view(np.int32))
    out = mxs.spec_sampling_thresholds(dev(z), tau, k, p, m)
    torch.cuda.synchronize()
    return host(out).view(np.uint32)


def compare(z, tau, k, p, allowed, label):
    thr = device_thresholds(z, tau, k, p, allowed)
    again = device_thresholds(z, tau, k, p, allowed)
    assert np.array_equal(thr, again), (label, "thresholds differ between two calls")
    keys = order_keys(z)
    flagged = 0
    for r in range(z.shape[0]):
        al = None if allowed is None else allowed[r]
        keep, _, margin = osm.kept_set(z[r], tau, k, p, al)
        if margin < osm.TOP_P_MARGIN:
            flagged += 1
            continue
        ok = np.isfinite(z[r]) & (np.ones(z.shape[1], bool) if al is None else al)
        got = ok & (keys[r] >= thr[r])
        if not np.array_equal(got, keep):
            diff = np.nonzero(got != keep)[0]
            raise AssertionError((label, r, int(thr[r]), int(got.sum()), int(keep.sum()), diff[:8].tolist()))
    say(f"  {label}: {z.shape[0]} rows, {flagged} set aside")


def normal_rows(seed, rows, v, sigma=3.0, mu=0.0):
    return (mu + sigma * synth.rng(31, synth.ROLE_BASE, seed).standard_normal((rows, v))).astype(np.float32)


SETTINGS_8B = [  # (temperature, top_k, top_p, mask keep fraction)
    (0.8, 50, 0.9, 0.9),
    (1.0, 0, 0.95, None),
    (1.0, 50, 1.0, None),
    (0.7, 0, 0.5, 0.7),
    (1.0, 1, 1.0, None),
    (0.05, 0, 0.9, None),     # sharp law: masses against 0 up to e^~300
    (2.0, 300, 0.99, 0.9),
    (1.0, 2000, 0.9, None),   # a few thousand candidates: radix passes over the list, both selections
    (1.0, 8000, 1.0, None),   # ~8000 candidates: the list or the radix passes
    (1.0, 9000, 1.0, None),   # more candidates than the list holds
    (1.0, 9000, 0.8, None),
]


@pytest.mark.parametrize("tau,k,p,keep", SETTINGS_8B)
def test_8b_vocab(tau, k, p, keep):
    say(f"thresholds: V=128256 tau={tau} k={k} p={p} keep={keep}")
    rows, v = 12, 128256
    z = normal_rows(k + int(100 * tau), rows, v)
    allowed = None if keep is None else synth.token_mask(31, k, rows, v, keep)
    compare(z, tau, k, p, allowed, f"8b tau={tau} k={k} p={p}")


@pytest.mark.parametrize("tau,k,p", [(1.0, 0, 0.9), (1.0, 50, 1.0), (1.0, 50, 0.5), (0.3, 0, 0.3)])
def test_one_crowded_bucket(tau, k, p):
    """Every logit in [1, 1.1): one first-digit bucket holds the whole row (radix passes)."""
    say(f"thresholds: one bucket tau={tau} k={k} p={p}")
    rows, v = 6, 128256
    z = (1.0 + 0.1 * synth.rng(32, synth.ROLE_BASE, k).random((rows, v))).astype(np.float32)
    compare(z, tau, k, p, None, f"bucket tau={tau} k={k} p={p}")


def test_top_k_keeps_every_token_then_top_p():
    say("thresholds: top-k above the allowed count, then top-p")
    rows, v = 16, 1024
    z = normal_rows(3, rows, v, sigma=2.0)
    allowed = synth.token_mask(33, 0, rows, v, 0.3)
    compare(z, 1.0, 500, 0.9, allowed, "k=500 of ~300 allowed, p=0.9")
    compare(z, 1.0, 500, 1.0, allowed, "k=500 of ~300 allowed")


@pytest.mark.parametrize("mu,tau", [(1000.0, 1.0), (-1000.0, 1.0), (0.0, 0.01)])
def test_logit_ranges_outside_the_reference(mu, tau):
    """max / tau above 690 or below -650: top-p masses against the row maximum only."""
    say(f"thresholds: mu={mu} tau={tau}")
    rows, v = 6, 20000
    z = normal_rows(4, rows, v, sigma=1.0 if mu else 3.0, mu=mu)
    compare(z, tau, 0, 0.9, None, f"mu={mu} tau={tau} p=0.9")
    compare(z, tau, 40, 0.7, None, f"mu={mu} tau={tau} k=40 p=0.7")


def test_ties():
    say("thresholds: integer logits")
    rows, v = 24, 4096
    z = synth.rng(34, 3).integers(-3, 4, size=(rows, v)).astype(np.float32)
    for tau, k, p in [(1.0, 10, 1.0), (1.0, 0, 0.7), (0.7, 30, 0.5), (1.0, 1, 1.0), (1.0, 4000, 0.99)]:
        compare(z, tau, k, p, None, f"ties tau={tau} k={k} p={p}")


@pytest.mark.parametrize("v", [2, 5, 4095, 4097, 12289])
def test_vocab_edges(v):
    say(f"thresholds: V={v}")
    rows = 20
    z = normal_rows(v, rows, v, sigma=2.0)
    allowed = synth.token_mask(35, v, rows, v, 0.8)
    compare(z, 0.9, 7, 0.85, allowed, f"v={v}")
    compare(z, 1.1, 0, 0.6, None, f"v={v} top-p")


def test_empty_and_nonfinite_rows():
    """Rows with nothing allowed, only -inf, and NaN / +inf entries (never kept)."""
    say("thresholds: empty and non-finite rows")
    rows, v = 6, 4096
    z = normal_rows(5, rows, v)
    allowed = np.ones((rows, v), bool)
    allowed[0] = False
    z[1] = -np.inf
    z[2, ::7] = np.nan
    z[3, ::11] = np.inf
    z[4, :4000] = -np.inf
    for tau, k, p in [(1.0, 20, 0.9), (1.0, 0, 0.8), (1.0, 20, 1.0)]:
        compare(z, tau, k, p, allowed, f"edge rows tau={tau} k={k} p={p}")


def test_both_off_is_zero():
    z = normal_rows(6, 4, 1000)
    assert not device_thresholds(z, 1.0, 0, 1.0, None).any()
    assert not device_thresholds(z, 1.0, 1000, 1.0, None).any()


@pytest.mark.parametrize("rows", [300, 576])
def test_many_rows_several_chunks_per_workgroup(rows):
    """Batches large enough that each counting workgroup takes several 4096-logit chunks of its row
    (rows x 32 chunks >= 4096: 4 and 8 chunks per workgroup), as spec_accept_sampled at B = 64."""
    say(f"thresholds: {rows} rows of V=128256")
    v = 128256
    z = normal_rows(rows, rows, v)
    for tau, k, p in [(0.8, 50, 0.9), (1.0, 0, 0.95), (1.0, 300, 1.0)]:
        compare(z, tau, k, p, None, f"{rows} rows tau={tau} k={k} p={p}")


def test_random_settings():
    """A seeded sweep of 40 random settings: vocabulary 2..20000, 1..40 rows, logit spreads from
    0.01 to 30 around offsets 0, 5 or -50 (or small integers: ties), temperature 0.05..3, top-k off /
    1 / up to v, top-p off or 0.05..0.999, masks keeping 5% to 95% of tokens or none."""
    r = synth.rng(36, 0)
    for case in range(40):
        v = int(r.integers(2, 20001))
        rows = int(r.integers(1, 41))
        if r.random() < 0.2:
            z = r.integers(-3, 4, size=(rows, v)).astype(np.float32)
        else:
            sigma = float(r.choice([0.01, 0.3, 3.0, 30.0]))
            mu = float(r.choice([0.0, 5.0, -50.0]))
            z = (mu + sigma * r.standard_normal((rows, v))).astype(np.float32)
        tau = float(np.float32(r.uniform(0.05, 3.0)))
        kc = r.random()
        k = 0 if kc < 0.3 else (1 if kc < 0.4 else int(r.integers(1, v + 1)))
        p = 1.0 if r.random() < 0.3 else float(np.float32(r.uniform(0.05, 0.999)))
        keep = None if r.random() < 0.5 else float(r.choice([0.05, 0.5, 0.95]))
        allowed = None if keep is None else r.random((rows, v)) < keep
        compare(z, tau, k, p, allowed, f"case {case}: v={v} rows={rows} tau={tau:.3f} k={k} p={p:.3f} keep={keep}")


def test_top_k_chunk_route_branches():
    """The per-chunk top-k route (k <= 128 at V = 128256) down each of its branches:
    integer logits (every chunk holds ~590 keys tied at the top, more than its 256 list slots:
    radix passes over the row); continuous logits with ~200 copies of the row maximum per chunk
    (the chunks fit, but ~6400 candidates survive every cut: radix passes over the list);
    k = 100 and 128 (the cut set holds more than 64 keys: the block sort instead of one wave)."""
    rows, v = 6, 128256
    ints = synth.rng(37, 0).integers(-3, 4, size=(rows, v)).astype(np.float32)
    for k, p in [(10, 1.0), (50, 0.9), (128, 1.0)]:
        say(f"thresholds: integer logits V={v} k={k} p={p}")
        compare(ints, 1.0, k, p, None, f"ints k={k} p={p}")
    dup = normal_rows(38, rows, v)
    top = synth.rng(38, 1).random((rows, v)) < 200.0 / 4096
    dup[top] = 20.0
    for k, p in [(50, 1.0), (50, 0.9)]:
        say(f"thresholds: tied maximum V={v} k={k} p={p}")
        compare(dup, 1.0, k, p, None, f"tied max k={k} p={p}")
    z = normal_rows(39, rows, v)
    for k, p in [(100, 1.0), (100, 0.8), (128, 0.95)]:
        say(f"thresholds: V={v} k={k} p={p}")
        compare(z, 0.9, k, p, None, f"k={k} p={p}")
