"""NVFP4 weights on the GPU vs the oracle (oracle/nvfp4.py).

nvfp4_quantize: codes, E4M3 block scales, the fp32 tensor scale and the flags
bit-exact (every step is one correctly rounded fp32 operation on both sides).
nvfp4_verify_gemm: relative L2 <= 2e-3 against the fp64 product and each
element within 1e-4 of sum_k |x_k w_k|; one-hot activations return the
dequantized column rounded once to fp32.
"""
import numpy as np
import pytest
import torch

import mx_fp4_weight_amd as mxs
import synth
from oracle import nvfp4 as nv
from tests.gpu_util import ELEM, REL_L2, dev, dev_bf16, host, say

pytestmark = pytest.mark.gpu


def gpu_quantize(w: np.ndarray):
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    codes, scales, g = mxs.nvfp4_quantize(dev(w), dev_flags=flags)
    torch.cuda.synchronize()
    return host(codes), host(scales), host(g)[0], int(flags.item())


def check_quantize(w, label):
    c, s, g, f = gpu_quantize(w)
    rc, rs, rg, rf = nv.quantize(w)
    assert np.float32(g).view(np.uint32) == np.float32(rg).view(np.uint32), (label, g, rg)
    assert np.array_equal(s, rs), (label, np.argwhere(s != rs)[:5])
    assert np.array_equal(c, rc), (label, np.argwhere(c != rc)[:5])
    assert f == rf, (label, f, rf)
    return rc, rs, rg


def run_gemm(codes, scales, g, xbits, dc=None, ds=None):
    y = mxs.nvfp4_verify_gemm(dev(codes) if dc is None else dc, dev(scales) if ds is None else ds,
                              torch.tensor([g], dtype=torch.float32, device="cuda"), dev_bf16(xbits))
    torch.cuda.synchronize()
    return host(y)


def check_gemm(codes, scales, g, xbits, y_gpu, rows=None, label=""):
    if rows is not None:
        codes, scales = codes[rows], scales[rows]
    wq = nv.dequantize(codes, scales, g)
    ref = nv.verify_gemm(codes, scales, g, xbits)
    x = (np.asarray(xbits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    bound = np.abs(x) @ np.abs(wq).T
    got = np.asarray(y_gpu, np.float64)
    assert got.shape == ref.shape, (label, got.shape, ref.shape)
    assert np.isfinite(got).all(), label
    err = got - ref
    rel = np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300)
    assert rel <= REL_L2, (label, rel)
    worst = np.max(np.abs(err) - ELEM * bound)
    assert worst <= 1e-30, (label, worst)


# ------------------------------------------------------------------ quantizer

def test_quantize_small_bit_exact():
    say("nvfp4 quantize: 1024x1024")
    check_quantize(synth.weights(1, 0, 1024, 1024), "1024x1024")


def test_quantize_hand_built_edges():
    """Global amax 2688 makes g = 1 exactly: block amax 6·t puts t on chosen E4M3 values,
    midpoints (ties to the even fraction), the subnormal range and the saturation point;
    the values inside each block sit on the E2M1 midpoints of their block scale."""
    say("nvfp4 quantize: edge blocks")
    table = nv.E4M3_TABLE[:127]
    mids = (table[:-1] + table[1:]) / 2
    targets = np.concatenate([table[1:], mids, [2.0 ** -10, 3 * 2.0 ** -11, 447.0, 448.0]])
    e2m1_ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -1.75, -5.0, 0.0, -0.0, 1.0, 4.0])
    rows = []
    for t in targets:
        blk = np.zeros(16, np.float64)
        blk[0] = 6.0 * t
        s = nv.e4m3_decode(nv.e4m3_encode(np.float32(6.0 * t / 6.0)))
        blk[1:15] = e2m1_ties * s
        blk[15] = -6.0 * t * 0.999
        rows.append(blk)
    while len(rows) % 4:
        rows.append(np.zeros(16))
    w = np.stack(rows).astype(np.float32).reshape(-1, 64)
    w[0, 0] = 2688.0
    assert nv.global_scale(w) == 1.0
    check_quantize(w, "edges")


@pytest.mark.parametrize("gmag", [1e-30, 1e-3, 1.0, 3e4, 1e30])
def test_quantize_block_ranges(gmag):
    """Blocks 2^0 .. 2^-30 below the tensor maximum (normal, subnormal and zero E4M3 scales)
    at several tensor magnitudes."""
    say(f"nvfp4 quantize: block ranges at {gmag}")
    r = synth.rng(51, 0, int(np.log10(gmag) + 40))
    n, k = 64, 512
    w = r.standard_normal((n, k))
    w *= (2.0 ** -r.integers(0, 31, (n, k // 16))).repeat(16, axis=1)
    w = (w * gmag).astype(np.float32)
    w[5] = 0.0
    w[6, :16] = -0.0
    _, rs, _ = check_quantize(w, f"ranges {gmag}")
    assert (rs == 0).any() and ((rs > 0) & (rs < 8)).any() and (rs >= 8).any()


def test_quantize_nonfinite_and_zero():
    say("nvfp4 quantize: non-finite blocks, zero tensor")
    w = synth.weights(52, 0, 8, 128)
    w[1, 3] = np.nan
    w[4, 127] = np.inf
    w[7, 64] = -np.inf
    check_quantize(w, "nonfinite")
    z = np.zeros((3, 64), np.float32)
    z[1, 5] = -0.0
    check_quantize(z, "zeros")
    # a single non-zero value: every other block gets scale 0 and signed-zero codes
    z[2, 40] = -3e-3
    check_quantize(z, "one value")


def test_quantize_8b_shape_full():
    say("nvfp4 quantize: 4096x14336 full compare")
    check_quantize(synth.weights(53, 0, 4096, 14336, outlier_frac=0.01), "4096x14336")


# ------------------------------------------------------------------ GEMM

def test_gemm_one_hot_exact():
    say("nvfp4 gemm: one-hot")
    n, k = 80, 1024
    codes, scales, g, _ = nv.quantize(synth.weights(54, 0, n, k, sigma=0.7))
    cols = [0, 1, 15, 16, 31, 32, 127, 128, 511, 512, 1023]
    x = np.zeros((len(cols), k), np.float32)
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    y = run_gemm(codes, scales, g, synth.f32_to_bf16_bits(x))
    wq = nv.dequantize(codes, scales, g)
    for i, c in enumerate(cols):
        assert np.array_equal(y[i], wq[:, c].astype(np.float32)), c


@pytest.mark.parametrize("n,k,m", [
    (1, 512, 1), (17, 512, 5), (16, 1024, 3), (1000, 4096, 5), (300, 1536, 16), (4100, 512, 9),
    (64, 512, 17), (33, 2048, 40), (3, 11776, 8), (70000, 512, 2),
    # activations of all of k do not fit in LDS: k walked in phases
    (300, 14336, 8), (100, 28672, 5), (70, 28672, 16), (257, 28672, 13), (17, 16384, 11),
])
def test_gemm_ragged_shapes(n, k, m):
    say(f"nvfp4 gemm: n={n} k={k} m={m}")
    idx = n + 3 * k + m
    codes, scales, g, _ = nv.quantize(synth.weights(55, idx, n, k))
    x = synth.activations(55, idx, m, k)
    check_gemm(codes, scales, g, x, run_gemm(codes, scales, g, x), label=f"{n}x{k}x{m}")


@pytest.mark.parametrize("gmag", [1e-25, 1e25])
def test_gemm_tensor_scale_extremes(gmag):
    """The tensor scale is applied once per output: tiny and huge g with mixed block scales."""
    say(f"nvfp4 gemm: tensor magnitude {gmag}")
    r = synth.rng(56, 0, int(gmag > 1))
    n, k = 48, 1024
    w = r.standard_normal((n, k)) * (2.0 ** -r.integers(0, 12, (n, k // 16))).repeat(16, axis=1)
    w = (w * gmag).astype(np.float32)
    codes, scales, g, _ = nv.quantize(w)
    x = synth.activations(56, int(gmag > 1), 5, k)
    check_gemm(codes, scales, g, x, run_gemm(codes, scales, g, x), label=f"g {g}")


def test_gemm_nan_block_propagates():
    """A refused block (scale NaN) turns its row's outputs into NaN; other rows are unaffected."""
    say("nvfp4 gemm: NaN block")
    n, k = 40, 512
    w = synth.weights(57, 0, n, k)
    w[9, 100] = np.nan
    codes, scales, g, flags = nv.quantize(w)
    assert flags == nv.FLAG_NONFINITE
    x = synth.activations(57, 0, 4, k)
    y = run_gemm(codes, scales, g, x)
    assert np.isnan(y[:, 9]).all()
    keep = np.array([i for i in range(n) if i != 9])
    check_gemm(codes, scales, g, x, y[:, keep], rows=keep, label="nan block")


@pytest.mark.parametrize("n,k", [(4096, 4096), (14336, 4096), (4096, 14336)])
def test_gemm_8b_shapes_t_sweep(n, k):
    """8B-class layer shapes at T = 1..8, weights quantized on the GPU, full outputs."""
    say(f"nvfp4 gemm: 8B {n}x{k} T=1..8")
    w = synth.weights(58, n + k, n, k)
    dc, ds, dg = mxs.nvfp4_quantize(dev(w))
    torch.cuda.synchronize()
    codes, scales, g = host(dc), host(ds), host(dg)[0]
    x8 = synth.activations(58, n + k, 8, k)
    ref = nv.verify_gemm(codes, scales, g, x8)
    wq = nv.dequantize(codes, scales, g)
    xf = (x8.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    bound = np.abs(xf) @ np.abs(wq).T
    for t in range(1, 9):
        y = mxs.nvfp4_verify_gemm(dc, ds, dg, dev_bf16(x8[:t]))
        torch.cuda.synchronize()
        err = host(y).astype(np.float64) - ref[:t]
        rel = np.linalg.norm(err) / np.linalg.norm(ref[:t])
        assert rel <= REL_L2, (t, rel)
        assert np.all(np.abs(err) <= ELEM * bound[:t]), t


@pytest.mark.parametrize("n,k", [(8192, 8192), (28672, 8192), (8192, 28672)])
def test_gemm_70b_shapes_sampled(n, k):
    """70B-class shapes at T = 5 with 1% outlier input channels x20: quantized on the GPU;
    the tensor scale and the sampled rows' codes and scales bit-exact (the tensor scale is
    checked against the oracle's amax rule over the whole matrix), sampled outputs."""
    say(f"nvfp4 gemm: 70B {n}x{k} T=5")
    idx = 7 * n + k
    w = synth.weights(59, idx, n, k, outlier_frac=0.01)
    dc, ds, dg = mxs.nvfp4_quantize(dev(w))
    x = synth.activations(59, idx, 5, k)
    y = mxs.nvfp4_verify_gemm(dc, ds, dg, dev_bf16(x))
    torch.cuda.synchronize()
    g = nv.global_scale(w)
    assert host(dg)[0] == g
    rows = np.unique(np.concatenate([synth.rng(59, 1, idx).choice(n, 126, replace=False), [0, n - 1]]))
    # the oracle's rows under the whole matrix's tensor scale: quantize [the rows + one
    # extra row that carries the matrix amax], so global_scale() gives the same g
    amax_row = np.zeros((1, k), np.float32)
    amax_row[0, 0] = np.abs(w).max()
    rc, rs, rg, _ = nv.quantize(np.concatenate([w[rows], amax_row]))
    assert rg == g
    rc, rs = rc[:-1], rs[:-1]
    assert np.array_equal(host(dc)[rows], rc) and np.array_equal(host(ds)[rows], rs)
    check_gemm(rc, rs, g, x, host(y)[:, rows], label=f"70B {n}x{k}")


def test_reused_outputs_and_inputs():
    """Two products in a row into the same output buffer, the second with fewer positions."""
    say("nvfp4 gemm: reuse")
    n, k = 512, 2048
    codes, scales, g, _ = nv.quantize(synth.weights(60, 0, n, k))
    dc, ds = dev(codes), dev(scales)
    dg = torch.tensor([g], dtype=torch.float32, device="cuda")
    ybuf = torch.full((8, n), float("nan"), dtype=torch.float32, device="cuda")
    for m in (8, 3):
        x = synth.activations(60, m, m, k)
        y = mxs.nvfp4_verify_gemm(dc, ds, dg, dev_bf16(x), y=ybuf[:m])
        torch.cuda.synchronize()
        check_gemm(codes, scales, g, x, host(y), label=f"reuse m={m}")


@pytest.mark.parametrize("shapes,k,m", [
    ([4096 // 8, 1024 // 8, 1024 // 8], 4096, 5),        # q | k | v shapes, scaled down
    ([300, 17, 1000, 64, 129, 5, 77, 256, 33, 500], 1024, 3),   # more than 8 products: two launches
    ([300, 70], 14336, 8),                                 # k walked in phases
    ([2000, 2000], 4096, 20),                              # two 16-position tiles
])
def test_grouped_matches_single(shapes, k, m):
    """Products with their own tensor scales in one launch: each equals its oracle product."""
    say(f"nvfp4 gemm grouped: {len(shapes)} products k={k} m={m}")
    items, refs = [], []
    for i, n in enumerate(shapes):
        w = synth.weights(77, 100 * i + n, n, k, sigma=0.02 * (i + 1))
        c, s, g, _ = nv.quantize(w)
        x = synth.activations(77, 100 * i + n, m, k)
        items.append((dev(c), dev(s), torch.tensor([g], dtype=torch.float32, device="cuda"), dev_bf16(x)))
        refs.append((c, s, g, x))
    # the products share the activations only in the layer case; here each has its own
    ys = mxs.nvfp4_verify_gemm_grouped(items)
    torch.cuda.synchronize()
    for (c, s, g, x), y in zip(refs, ys):
        check_gemm(c, s, g, x, host(y), label=f"grouped n={c.shape[0]}")


@pytest.mark.parametrize("shapes,k,m", [
    ([4096, 1024, 1024], 4096, 5),                         # q | k | v
    ([300, 17, 1000, 64, 129, 5, 77, 256, 33, 500], 1024, 3),   # two launches, ragged
    ([8192], 14336, 5),                                    # phases with two row tiles per block
    ([300, 70], 14336, 8),                                 # phases, one row tile per block
    ([2000, 2000], 4096, 20),                              # two 16-position tiles
])
def test_grouped_tiled_matches_row_layout(shapes, k, m):
    """nvfp4_verify_gemm_grouped_tiled (codes tiled by mxfp4_tile_codes) returns the row-layout
    result bit for bit, and the oracle bar on the small products."""
    say(f"nvfp4 gemm grouped tiled: {shapes} k={k} m={m}")
    items, titems, hosts = [], [], []
    for i, n in enumerate(shapes):
        w = synth.weights(78, 100 * i + n, n, k, sigma=0.02 * (i + 1))
        xb = synth.activations(78, 100 * i + n, m, k)
        dc, ds, dg = mxs.nvfp4_quantize(dev(w))
        x = dev_bf16(xb)
        items.append((dc, ds, dg, x))
        titems.append((mxs.mxfp4_tile_codes(dc), ds, dg, n, x))
        hosts.append((w, xb))
    ys = mxs.nvfp4_verify_gemm_grouped(items)
    yt = mxs.nvfp4_verify_gemm_grouped_tiled(titems)
    torch.cuda.synchronize()
    for n, a, b, (w, xb) in zip(shapes, ys, yt, hosts):
        assert torch.equal(a, b), (n, k, m)
        if n * k <= 1 << 22:
            c, s, g, _ = nv.quantize(w)
            check_gemm(c, s, g, xb, host(b), label=f"grouped tiled n={n}")


@pytest.mark.parametrize("t", [1, 5, 8])
def test_bench_launches_tiled_match_row_layout(t):
    """The four launches the NVFP4 bench times on the 8B-class layer (q|k|v and gate|up grouped, o
    and down single; codes tiled by mxfp4_tile_codes) return the row-layout results bit for bit,
    the row layout being held to the oracle at these shapes above."""
    say(f"nvfp4 bench launches, tiled vs row layout, T={t}")
    groups = [([4096, 1024, 1024], 4096), ([4096], 4096), ([14336, 14336], 4096), ([4096], 14336)]
    for gi, (shapes, k) in enumerate(groups):
        items, titems = [], []
        for i, n in enumerate(shapes):
            w = synth.weights(79, 10 * gi + i, n, k)
            dc, ds, dg = mxs.nvfp4_quantize(dev(w))
            del w
            x = dev_bf16(synth.activations(79, 10 * gi + i, t, k))
            items.append((dc, ds, dg, x))
            titems.append((mxs.mxfp4_tile_codes(dc), ds, dg, n, x))
        ys = mxs.nvfp4_verify_gemm_grouped(items)
        yt = mxs.nvfp4_verify_gemm_grouped_tiled(titems)
        torch.cuda.synchronize()
        for n, a, b in zip(shapes, ys, yt):
            assert torch.equal(a, b), (shapes, n, k, t)
        say(f"  {shapes} k={k}: bit-identical")
