"""Parity on every launch the benchmark times, and on the full-step chain.

The tiled entry points (mxfp4_verify_gemm_tiled / _grouped_tiled) are what the
benchmark runs. Here they run at the benchmark's own shapes and launch
groupings and are checked bit for bit against the row layout (same kernel,
same sums) and, on sampled or full rows, against the fp64 oracle:

* 70B-class launches at k = 8192 (one phase, one workgroup per CU) with 1% of
  the input channels x20: q | k | v grouped, o, gate | up grouped;
* both lm_heads, 128256 x 8192 (outliers) and 128256 x 4096;
* the four 8B-class launch types at every T = 1..8;
* the full-step chain at reduced depth (two decoder layers, then the
  128256 x 4096 lm_head, then the acceptance step on logits of that law with
  draft rows tuned to a target acceptance), checked three ways:
  the GEMM outputs against the oracle GEMM; spec_accept on the oracle's own
  lm_head logits against the oracle's acceptance loop (bit-exact); and the
  device-resident chain (spec_accept reading the GPU lm_head output) against
  the closed form E = (1 - a^(K+1)) / (1 - a) ("Module 11. Speculative
  Decoding and Quantization", §6).

The oracle never takes a value computed on the GPU: its codes come from its own
quantizer on the seeded fp32 weights, its logits from its own GEMM.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import mx_fp4_weight_amd as mxs
import synth
from oracle import accept as oacc
from oracle import gemm as ogemm
from oracle import mx as omx
from tests.gpu_util import check_gemm, dev, dev_bf16, host, say

pytestmark = pytest.mark.gpu

T = 5
KD = 4
CHUNK = 4096  # weight rows generated / quantized per host job


def _row_ranges(n, step=CHUNK):
    return [(r0, min(n, r0 + step)) for r0 in range(0, n, step)]


def gpu_quantized(config, index, n, k, outlier_frac=0.0):
    """Seeded fp32 W[n, k] (drawn on the host in row chunks, threads in parallel) quantized by
    mxfp4_quantize into device codes / scales (the weights never sit on the host whole)."""
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n, k // 32), dtype=torch.uint8, device="cuda")

    def draw(rr):
        return synth.weights(config, index, n, k, outlier_frac=outlier_frac, row_start=rr[0], row_stop=rr[1])

    with ThreadPoolExecutor(8) as ex:
        for (r0, r1), w in zip(_row_ranges(n), ex.map(draw, _row_ranges(n))):
            mxs.mxfp4_quantize(dev(w), codes=codes[r0:r1], scales=scales[r0:r1])
    torch.cuda.synchronize()
    return codes, scales


def oracle_quantized(config, index, n, k, outlier_frac=0.0):
    """The oracle's codes / scales of the same seeded W (row chunks quantized on host threads)."""
    def job(rr):
        w = synth.weights(config, index, n, k, outlier_frac=outlier_frac, row_start=rr[0], row_stop=rr[1])
        c, s, _ = omx.quantize(w)
        return c, s

    with ThreadPoolExecutor(8) as ex:
        parts = list(ex.map(job, _row_ranges(n)))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def sample_rows(n, seed, count=254):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([rng.choice(n, size=min(count, n), replace=False), [0, n - 1]]))


def check_sampled(config, index, n, k, outlier_frac, dcodes, dscales, x, y, label):
    """Codes of sampled rows bit-exact against the oracle quantizer, outputs of those rows
    against the oracle GEMM."""
    rows = sample_rows(n, config * 1000 + index)
    w_rows = np.concatenate([synth.weights(config, index, n, k, outlier_frac=outlier_frac, row_start=r, row_stop=r + 1)
                             for r in rows])
    rc, rs, _ = omx.quantize(w_rows)
    ridx = torch.from_numpy(rows).cuda()
    assert np.array_equal(host(dcodes[ridx]), rc) and np.array_equal(host(dscales[ridx]), rs), label
    sub_c = np.zeros((n, k // 2), np.uint8)
    sub_s = np.zeros((n, k // 32), np.uint8)
    sub_c[rows], sub_s[rows] = rc, rs
    check_gemm(sub_c, sub_s, n, k, x, host(y)[:, rows], rows=rows, label=label)


def tiled(dc, ds):
    return mxs.mxfp4_tile_codes(dc), mxs.mxfp4_tile_scales(ds)


# ----------------------------------------------------------------------------- 70B-class, k = 8192

@pytest.mark.parametrize("name,shapes", [
    ("qkv", [8192, 1024, 1024]),
    ("o", [8192]),
    ("gate_up", [28672, 28672]),
])
def test_70b_k8192_launches_tiled(name, shapes):
    """The 70B-class launches at k = 8192 and T = 5 as the benchmark groups them, on tiled
    weights with 1% outlier input channels x20: bit-identical to the row layout, sampled rows
    against the oracle."""
    k = 8192
    say(f"bench launches: 70B {name} {shapes} k={k} T={T}")
    mats = []
    for i, n in enumerate(shapes):
        idx = 700 + 10 * len(shapes) + i
        dc, ds = gpu_quantized(3, idx, n, k, outlier_frac=0.01)
        x = synth.activations(3, idx, T, k)
        mats.append((idx, n, dc, ds, x, dev_bf16(x)))
    if len(mats) == 1:
        idx, n, dc, ds, x, dx = mats[0]
        y_row = [mxs.mxfp4_verify_gemm(dc, ds, dx)]
        y_t = [mxs.mxfp4_verify_gemm_tiled(*tiled(dc, ds), n, k, dx)]
    else:
        y_row = mxs.mxfp4_verify_gemm_grouped([(dc, ds, dx) for (_, _, dc, ds, _, dx) in mats])
        y_t = mxs.mxfp4_verify_gemm_grouped_tiled([(*tiled(dc, ds), n, dx) for (_, n, dc, ds, _, dx) in mats])
    torch.cuda.synchronize()
    for (idx, n, dc, ds, x, _), yr, yt in zip(mats, y_row, y_t):
        assert torch.equal(yt, yr), (name, n)
        check_sampled(3, idx, n, k, 0.01, dc, ds, x, yt, f"70B {name} n={n}")


# ----------------------------------------------------------------------------- lm_heads

@pytest.mark.parametrize("k,outlier_frac", [(8192, 0.01), (4096, 0.0)])
def test_lm_head_tiled(k, outlier_frac):
    """lm_head 128256 x k at T = 5 (70B-class with outliers; the full 8B-class step's): the tiled
    launch bit-identical to the row layout, sampled rows against the oracle."""
    n = 128256
    idx = 900 + k // 1024
    say(f"bench launches: lm_head {n}x{k} T={T}")
    dc, ds = gpu_quantized(3, idx, n, k, outlier_frac=outlier_frac)
    x = synth.activations(3, idx, T, k)
    dx = dev_bf16(x)
    y_row = mxs.mxfp4_verify_gemm(dc, ds, dx)
    tc, ts = tiled(dc, ds)
    y_t = mxs.mxfp4_verify_gemm_tiled(tc, ts, n, k, dx)
    torch.cuda.synchronize()
    assert torch.equal(y_t, y_row)
    check_sampled(3, idx, n, k, outlier_frac, dc, ds, x, y_t, f"lm_head {n}x{k}")


# ----------------------------------------------------------------------------- 8B-class, T = 1..8

LAYER_8B = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
            ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336)]
LAUNCHES_8B = [("qkv", (0, 1, 2)), ("o", (3,)), ("gate_up", (4, 5)), ("down", (6,))]


def run_launch(items, ys, layout):
    """One benchmark launch: items [(codes, scales, tiled codes, tiled scales, n, x)]."""
    if layout == "tiled":
        if len(items) == 1:
            _, _, tc, ts, n, x = items[0]
            mxs.mxfp4_verify_gemm_tiled(tc, ts, n, x.shape[1], x, y=ys[0])
        else:
            mxs.mxfp4_verify_gemm_grouped_tiled([(tc, ts, n, x) for (_, _, tc, ts, n, x) in items], ys=ys)
    else:
        if len(items) == 1:
            dc, ds, _, _, _, x = items[0]
            mxs.mxfp4_verify_gemm(dc, ds, x, y=ys[0])
        else:
            mxs.mxfp4_verify_gemm_grouped([(dc, ds, x) for (dc, ds, _, _, _, x) in items], ys=ys)


@pytest.mark.parametrize("launch", [name for name, _ in LAUNCHES_8B])
def test_8b_launch_types_t_sweep_tiled(launch):
    """Each 8B-class launch type at T = 1..8 as the benchmark runs it (grouped where the
    benchmark groups): tiled outputs against the oracle (full rows) and bit-identical to the
    row-layout call."""
    idxs = dict(LAUNCHES_8B)[launch]
    say(f"bench launches: 8B {launch} T=1..8")
    mats = []
    for i in idxs:
        _, n, k = LAYER_8B[i]
        c, s = oracle_quantized(2, 300 + i, n, k)
        x8 = synth.activations(2, 300 + i, 8, k)
        ref = ogemm.verify_gemm(c, s, n, k, x8)
        bound = ogemm.abs_bound(c, s, n, k, x8)
        dc, ds = dev(c), dev(s)
        mats.append((n, k, dc, ds, *tiled(dc, ds), x8, ref, bound))
    for t in range(1, 9):
        items = [(dc, ds, tc, ts, n, dev_bf16(x8[:t])) for (n, k, dc, ds, tc, ts, x8, _, _) in mats]
        ys_t = [torch.empty((t, m[0]), dtype=torch.float32, device="cuda") for m in mats]
        ys_r = [torch.empty((t, m[0]), dtype=torch.float32, device="cuda") for m in mats]
        run_launch(items, ys_t, "tiled")
        run_launch(items, ys_r, "row")
        torch.cuda.synchronize()
        for (n, k, _, _, _, _, _, ref, bound), yt, yr in zip(mats, ys_t, ys_r):
            assert torch.equal(yt, yr), (launch, n, t)
            err = host(yt).astype(np.float64) - ref[:t]
            assert np.linalg.norm(err) / np.linalg.norm(ref[:t]) <= 2e-3, (launch, n, t)
            assert np.all(np.abs(err) <= 1e-4 * bound[:t]), (launch, n, t)


# ----------------------------------------------------------------------------- full-step chain

def _overlap(p, q):
    return float(np.minimum(p, q).sum())


def tune_draft_rows(tgt_rows, noise, alpha):
    """Draft logit rows tgt_i + lam_i * noise_i (fp32), with lam_i bisected in fp64 so that the
    overlap sum_x min(p_i, q_i) of row i is alpha (input preparation on the oracle's logits)."""
    lams = []
    for i in range(noise.shape[0]):
        p = oacc.softmax(tgt_rows[i])
        lo, hi = 0.0, 64.0
        for _ in range(50):
            mid = 0.5 * (lo + hi)
            q = oacc.softmax((tgt_rows[i] + np.float32(mid) * noise[i]).astype(np.float32))
            if _overlap(p, q) > alpha:
                lo = mid
            else:
                hi = mid
        lams.append(np.float32(0.5 * (lo + hi)))
    return np.stack([(tgt_rows[i] + lams[i] * noise[i]).astype(np.float32) for i in range(noise.shape[0])]), lams


def test_full_step_chain_reduced():
    """Two 8B-class decoder layers and the 128256 x 4096 lm_head at T = 5 on tiled weights, then
    the acceptance step on logits of the lm_head's law (K = 4, draft rows tuned to a = 0.6, 0.8,
    0.9)."""
    V, k = 128256, 4096
    cfg = 5
    say("bench launches: chain, 2 layers + lm_head 128256x4096 + spec_accept")
    # two layers in the benchmark's four launches, outputs against the oracle on sampled rows
    for layer in range(2):
        mats = []
        for j, (_, n, kk) in enumerate(LAYER_8B):
            idx = 10 * layer + j
            c, s = oracle_quantized(cfg, idx, n, kk)
            x = synth.activations(cfg, idx, T, kk)
            dc, ds = dev(c), dev(s)
            mats.append((c, s, n, kk, x, (dc, ds, *tiled(dc, ds), n, dev_bf16(x))))
        ys = [torch.empty((T, n), dtype=torch.float32, device="cuda") for (_, n, _) in LAYER_8B]
        for _, idxs in LAUNCHES_8B:
            run_launch([mats[i][5] for i in idxs], [ys[i] for i in idxs], "tiled")
        torch.cuda.synchronize()
        for (c, s, n, kk, x, _), y in zip(mats, ys):
            rows = sample_rows(n, 17 * layer + n)
            check_gemm(c[rows], s[rows], len(rows), kk, x, host(y)[:, rows], label=f"chain layer {layer} n={n}")
    # lm_head: oracle codes (host threads) feed both sides; the full output against the oracle
    lm_idx = 99
    c, s = oracle_quantized(cfg, lm_idx, V, k)
    x = synth.activations(cfg, lm_idx, T, k)
    dc, ds = dev(c), dev(s)
    tc, ts = tiled(dc, ds)
    y_lm = mxs.mxfp4_verify_gemm_tiled(tc, ts, V, k, dev_bf16(x))
    torch.cuda.synchronize()
    del dc, ds
    ref = ogemm.verify_gemm(c, s, V, k, x)
    bound = ogemm.abs_bound(c, s, V, k, x)
    got = host(y_lm).astype(np.float64)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) <= 2e-3
    assert np.all(np.abs(got - ref) <= 1e-4 * bound)
    # the oracle's logits of the step: its GEMM output rounded to the fp32 the GEMM returns
    tgt_rows = ref.astype(np.float32)
    eps = float(np.max(np.abs(got - tgt_rows.astype(np.float64))))
    say(f"  lm_head logits: max |GPU - oracle| = {eps:.3g}")
    noise = synth.rng(cfg, synth.ROLE_NOISE, 0).standard_normal((KD, V), dtype=np.float32)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    for alpha in (0.6, 0.8, 0.9):
        dft_rows, lams = tune_draft_rows(tgt_rows, noise, alpha)
        alphas = [_overlap(oacc.softmax(tgt_rows[i]), oacc.softmax(dft_rows[i])) for i in range(KD)]
        assert max(abs(a - alpha) for a in alphas) < 1e-4, alphas
        # (1) spec_accept on the oracle's logits: bit-exact against the oracle loop
        b = 64
        tgt_b = np.broadcast_to(tgt_rows, (b, KD + 1, V)).copy()
        dft_b = np.broadcast_to(dft_rows, (b, KD, V)).copy()
        tok = np.stack([synth.gumbel_tokens(cfg, 1000 * int(alpha * 10) + s_, dft_rows) for s_ in range(b)])
        u = np.stack([synth.uniforms(cfg, 1000 * int(alpha * 10) + s_, KD) for s_ in range(b)])
        out, nacc = mxs.spec_accept(dev(tgt_b), dev(dft_b), dev(tok), dev(u))
        torch.cuda.synchronize()
        out, nacc = host(out), host(nacc)
        r = oacc.step_batch(tgt_b, dft_b, tok, u)
        differ = (nacc != r["n"]) | np.any(out != r["out_tokens"], axis=1)
        bad = np.nonzero((r["margin"] >= 1e-12) & differ)[0]
        assert bad.size == 0, (alpha, bad[:5], nacc[bad[:5]], r["n"][bad[:5]])
        # (2) the device-resident chain: spec_accept reads the GPU lm_head output and draft rows
        # built from it (same lam_i and noise); over 4096 cycles the emitted tokens per step
        # match the closed form within 4 standard errors
        lam = torch.tensor(np.array(lams), device="cuda").unsqueeze(1)
        dft_gpu = (y_lm[:KD] + lam * dev(noise)).contiguous()
        trials, bt = 4096, 512
        tgt_g = y_lm.unsqueeze(0).expand(bt, KD + 1, V).contiguous()
        dft_g = dft_gpu.unsqueeze(0).expand(bt, KD, V).contiguous()
        qd = torch.softmax(dft_gpu.double(), -1)
        emitted = []
        for _ in range(trials // bt):
            tk = torch.multinomial(qd, bt, replacement=True, generator=gen).t().contiguous().to(torch.int32)
            ub = torch.rand((bt, KD + 1), generator=gen, device="cuda", dtype=torch.float32)
            _, nb = mxs.spec_accept(tgt_g, dft_g, tk, ub)
            emitted.append((nb + 1).double())
        em = torch.cat(emitted)
        e_closed = (1 - alpha ** (KD + 1)) / (1 - alpha)
        e_meas, se = float(em.mean()), float(em.std()) / np.sqrt(em.numel())
        say(f"  alpha={alpha}: {int(r['flagged'].sum())}/{b} flagged; E measured {e_meas:.4f} vs closed "
            f"form {e_closed:.4f} (s.e. {se:.4f})")
        assert abs(e_meas - e_closed) <= 4 * se, (alpha, e_meas, e_closed, se)
        del tgt_g, dft_g
