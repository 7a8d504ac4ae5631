"""mxfp4_verify_gemm on the GPU vs the fp64 oracle (relative L2 <= 2e-3, per-element bound)."""
import numpy as np
import pytest
import torch

import mx_fp4_weight_amd as mxs
import synth
from oracle import mx as omx
from tests.gpu_util import check_gemm, dev, dev_bf16, host, say

pytestmark = pytest.mark.gpu


def run_gemm(codes, scales, xbits):
    y = mxs.mxfp4_verify_gemm(dev(codes), dev(scales), dev_bf16(xbits))
    torch.cuda.synchronize()
    return host(y)


def test_tiny_config():
    say("gemm: tiny 1024x1024 T=5")
    w = synth.weights(1, 0, 1024, 1024)
    codes, scales, _ = omx.quantize(w)
    x = synth.activations(1, 0, 5, 1024)
    check_gemm(codes, scales, 1024, 1024, x, run_gemm(codes, scales, x), label="tiny")


def test_one_hot_columns_exact():
    """x = e_k returns column k of the dequantized matrix exactly (fp32 sums of one term)."""
    say("gemm: one-hot")
    n, k = 80, 256
    codes, scales, _ = omx.quantize(synth.weights(7, 1, n, k))
    cols = [0, 1, 31, 32, 127, 128, 255]
    x = np.zeros((len(cols), k), np.float32)
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    y = run_gemm(codes, scales, synth.f32_to_bf16_bits(x))
    wd = omx.dequantize(codes, scales, k)
    for i, c in enumerate(cols):
        assert np.array_equal(y[i].astype(np.float64), wd[:, c])


@pytest.mark.parametrize("n,k,m", [
    # k % 512 != 0: activations read from global memory by every wave
    (1, 32, 1), (17, 32, 5), (16, 96, 3), (33, 160, 8), (1000, 4128, 5), (300, 1056, 16),
    (129, 640, 33), (2048, 288, 7),
    # k % 512 == 0: persistent kernel with activations in LDS (partial row blocks,
    # several column tiles, k split into sub-slices, waves past the last group)
    (5, 8192, 1), (64, 512, 17), (1000, 4096, 5), (17, 1024, 3), (4100, 512, 9),
    (130, 14336, 5), (33, 2048, 16), (100, 512, 40), (70000, 512, 2), (3, 11776, 8),
    # 16 positions over k = 4608 do not fit in LDS: two phases, 263 row blocks
    (4200, 4608, 16),
    # one partial-tile buffer so that two workgroups share a CU's LDS (8 positions over
    # k = 4096; 12 over k = 3072 with 563 row blocks, two on some workgroups)
    (4100, 4096, 8), (9000, 3072, 12),
])
def test_ragged_shapes(n, k, m):
    say(f"gemm: ragged n={n} k={k} m={m}")
    w = synth.weights(7, n + 3 * k + m, n, k)
    codes, scales, _ = omx.quantize(w)
    x = synth.activations(7, n + 3 * k + m, m, k)
    check_gemm(codes, scales, n, k, x, run_gemm(codes, scales, x), label=f"{n}x{k}x{m}")


@pytest.mark.parametrize("n,k,m", [
    # activations of all of k do not fit in LDS: k is walked in phases, each staged
    # in turn (two phases; three phases with a short last one; 16 positions)
    (300, 14336, 8), (100, 28672, 5), (70, 28672, 16), (33, 14336, 7), (257, 28672, 13),
    (17, 16384, 11),
])
def test_phased_k_shapes(n, k, m):
    say(f"gemm: phased n={n} k={k} m={m}")
    w = synth.weights(10, n + 3 * k + m, n, k)
    codes, scales, _ = omx.quantize(w)
    x = synth.activations(10, n + 3 * k + m, m, k)
    check_gemm(codes, scales, n, k, x, run_gemm(codes, scales, x), label=f"phased {n}x{k}x{m}")


@pytest.mark.parametrize("n,k,m", [
    # enough row blocks for one workgroup per pair of blocks on every CU: each workgroup
    # walks its pair phase by phase (two and four phases); 513 row blocks leave the last
    # pair without its second block
    (8200, 14336, 8), (8193, 16384, 16),
])
def test_phased_pairs(n, k, m):
    say(f"gemm: phased pairs n={n} k={k} m={m}")
    w = synth.weights(11, n + k + m, n, k)
    codes, scales, _ = omx.quantize(w)
    del w
    x = synth.activations(11, n + k + m, m, k)
    rng = np.random.default_rng(n + k)
    rows = np.unique(np.concatenate([rng.choice(n, size=160, replace=False),
                                     np.arange(0, 16), np.arange(n - 24, n), [4112, 4128]]))
    y = run_gemm(codes, scales, x)
    check_gemm(codes, scales, n, k, x, y[:, rows], rows=rows, label=f"pairs {n}x{k}x{m}")


@pytest.mark.parametrize("n,k,m", [
    # m > 32 with k % 128 == 0: the dense kernel (128 weight rows x 80 positions per tile,
    # k split in two halves of alternating 128-k groups)
    (1, 128, 33), (130, 384, 80), (257, 1024, 100), (1000, 2304, 161), (64, 128, 320),
    (300, 896, 81), (129, 3200, 47), (1024, 1024, 240),
    # m > 32 with k % 128 != 0: fallback kernel
    (50, 96, 40), (33, 1056, 65),
])
def test_dense_ragged_shapes(n, k, m):
    say(f"gemm: dense ragged n={n} k={k} m={m}")
    w = synth.weights(9, n + 3 * k + m, n, k)
    codes, scales, _ = omx.quantize(w)
    x = synth.activations(9, n + 3 * k + m, m, k)
    check_gemm(codes, scales, n, k, x, run_gemm(codes, scales, x), label=f"dense {n}x{k}x{m}")


def test_one_hot_dense_exact():
    """One-hot activation rows through the dense kernel return weight columns exactly."""
    say("gemm: one-hot dense")
    n, k, m = 200, 640, 96
    codes, scales, _ = omx.quantize(synth.weights(7, 2, n, k))
    cols = np.random.default_rng(5).integers(0, k, m)
    x = np.zeros((m, k), np.float32)
    x[np.arange(m), cols] = 1.0
    y = run_gemm(codes, scales, synth.f32_to_bf16_bits(x))
    wd = omx.dequantize(codes, scales, k)
    for i, c in enumerate(cols):
        assert np.array_equal(y[i].astype(np.float64), wd[:, c]), i


@pytest.mark.parametrize("m", [5, 40])
def test_scale_extremes(m):
    """Block scales from 2^-100 to 2^120 (products stay in the fp32 normal range), all-zero blocks."""
    say(f"gemm: scale extremes m={m}")
    n, k = 32, 512
    rng = np.random.default_rng(3)
    w = rng.standard_normal((n, k)).astype(np.float32)
    mags = np.float32(2.0) ** rng.integers(-100, 120, (n, k // 32)).astype(np.float32)
    w = (w.reshape(n, -1, 32) * mags[..., None]).reshape(n, k).astype(np.float32)
    w[3] = 0
    w[5, :64] = -0.0
    codes, scales, _ = omx.quantize(w)
    assert scales[3].max() == 0 and scales.max() >= 240
    x = synth.activations(7, 99, m, k, sigma=1e-3)
    check_gemm(codes, scales, n, k, x, run_gemm(codes, scales, x), label="scales")


@pytest.mark.parametrize("n,k", [(4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336)])
def test_8b_shapes_t_sweep(n, k):
    """The 8B-class layer shapes at every T = 1..8, full outputs."""
    say(f"gemm: 8B {n}x{k} T=1..8")
    w = synth.weights(2, n * 7 + k, n, k)
    codes, scales, _ = omx.quantize(w)
    x8 = synth.activations(2, n * 7 + k, 8, k)
    from oracle import gemm as ogemm
    ref = ogemm.verify_gemm(codes, scales, n, k, x8)
    bound = ogemm.abs_bound(codes, scales, n, k, x8)
    dc, ds = dev(codes), dev(scales)
    for t in range(1, 9):
        y = mxs.mxfp4_verify_gemm(dc, ds, dev_bf16(x8[:t]))
        torch.cuda.synchronize()
        got = host(y).astype(np.float64)
        err = got - ref[:t]
        rel = np.linalg.norm(err) / np.linalg.norm(ref[:t])
        assert rel <= 2e-3, (t, rel)
        assert np.all(np.abs(err) <= 1e-4 * bound[:t]), t


@pytest.mark.parametrize("n,k", [(8192, 8192), (1024, 8192), (28672, 8192), (8192, 28672)])
def test_70b_shapes_outliers(n, k):
    """70B-class shapes at T = 5 with 1% outlier input channels x20; weights quantized on the GPU,
    codes of the sampled rows checked bit-exact, outputs of the sampled rows against the oracle."""
    say(f"gemm: 70B {n}x{k} T=5 outliers")
    idx = n * 3 + k
    w = synth.weights(3, idx, n, k, outlier_frac=0.01)
    dcodes, dscales = mxs.mxfp4_quantize(dev(w))
    x = synth.activations(3, idx, 5, k)
    y = mxs.mxfp4_verify_gemm(dcodes, dscales, dev_bf16(x))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(idx).choice(n, 254, replace=False), [0, n - 1]]))
    rc, rs, _ = omx.quantize(w[rows])
    assert np.array_equal(host(dcodes)[rows], rc) and np.array_equal(host(dscales)[rows], rs)
    sub_c = np.zeros((n, k // 2), np.uint8)
    sub_s = np.zeros((n, k // 32), np.uint8)
    sub_c[rows], sub_s[rows] = rc, rs
    check_gemm(sub_c, sub_s, n, k, x, host(y)[:, rows], rows=rows, label=f"70B {n}x{k}")


def test_70b_lm_head_sampled():
    """lm_head 128256x8192 at T = 5: generated and quantized on the GPU in row chunks."""
    say("gemm: 70B lm_head 128256x8192")
    n, k = 128256, 8192
    idx = 99
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n, k // 32), dtype=torch.uint8, device="cuda")
    step = 8192
    for r0 in range(0, n, step):
        r1 = min(n, r0 + step)
        w = synth.weights(3, idx, n, k, outlier_frac=0.01, row_start=r0, row_stop=r1)
        mxs.mxfp4_quantize(dev(w), codes=codes[r0:r1], scales=scales[r0:r1])
    x = synth.activations(3, idx, 5, k)
    y = mxs.mxfp4_verify_gemm(codes, scales, dev_bf16(x))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(idx).choice(n, 126, replace=False), [0, n - 1]]))
    w_rows = np.concatenate([synth.weights(3, idx, n, k, outlier_frac=0.01, row_start=r, row_stop=r + 1)
                             for r in rows])
    rc, rs, _ = omx.quantize(w_rows)
    hc, hs = host(codes[torch.from_numpy(rows).cuda()]), host(scales[torch.from_numpy(rows).cuda()])
    assert np.array_equal(hc, rc) and np.array_equal(hs, rs)
    sub_c = np.zeros((n, k // 2), np.uint8)
    sub_s = np.zeros((n, k // 32), np.uint8)
    sub_c[rows], sub_s[rows] = rc, rs
    check_gemm(sub_c, sub_s, n, k, x, host(y)[:, rows], rows=rows, label="lm_head")


def test_batched_320_rows_sampled():
    """64 sequences x 5 positions = 320 rows against 8192x28672 (the batched verification case)."""
    say("gemm: batched 320x8192x28672")
    n, k, m = 8192, 28672, 320
    w = synth.weights(4, 0, n, k)
    dcodes, dscales = mxs.mxfp4_quantize(dev(w))
    x = synth.activations(4, 0, m, k)
    y = mxs.mxfp4_verify_gemm(dcodes, dscales, dev_bf16(x))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(4).choice(n, 126, replace=False), [0, n - 1]]))
    rc, rs, _ = omx.quantize(w[rows])
    assert np.array_equal(host(dcodes)[rows], rc) and np.array_equal(host(dscales)[rows], rs)
    sub_c = np.zeros((n, k // 2), np.uint8)
    sub_s = np.zeros((n, k // 32), np.uint8)
    sub_c[rows], sub_s[rows] = rc, rs
    check_gemm(sub_c, sub_s, n, k, x, host(y)[:, rows], rows=rows, label="batched")


@pytest.mark.parametrize("shapes,k,m", [
    ([4096, 1024, 1024], 4096, 5),          # q | k | v (k and v in 8-row blocks)
    ([1000, 130, 17, 9], 1024, 5),          # 8-row blocks for all but the largest, partial ones
    ([1000, 130, 17, 9], 1024, 16),
    ([14336, 14336], 4096, 5),              # gate | up
    ([17, 300, 1, 4100, 64, 2048, 5, 33, 999], 512, 9),   # ten products: two launches, ragged
    ([130, 70], 1056, 3),                   # k % 512 != 0: one fallback launch per product
    ([300, 129], 1024, 64),                 # m > 32: one dense launch per product
    ([300, 129], 14336, 8),                 # k walked in two phases, one row block per workgroup
])
def test_grouped_matches_oracle(shapes, k, m):
    say(f"gemm grouped: {shapes} k={k} m={m}")
    items, hosts = [], []
    for i, n in enumerate(shapes):
        c, s_, _ = omx.quantize(synth.weights(8, 40 + i, n, k))
        x = synth.activations(8, 40 + i, m, k)
        items.append((dev(c), dev(s_), dev_bf16(x)))
        hosts.append((c, s_, x, n))
    ys = mxs.mxfp4_verify_gemm_grouped(items)
    torch.cuda.synchronize()
    for (c, s_, x, n), y in zip(hosts, ys):
        check_gemm(c, s_, n, k, x, host(y), label=f"grouped n={n}")
    # the single entry point gives bit-identical results for the same tile choice
    y1 = mxs.mxfp4_verify_gemm(*items[0])
    torch.cuda.synchronize()
    assert np.array_equal(host(y1), host(ys[0]))


@pytest.mark.parametrize("n,k,m", [
    # m > 32: the row-layout call runs the same dense kernel, so the sums are bit-identical
    (1, 128, 33), (17, 384, 80), (130, 384, 81), (257, 1024, 100), (1000, 2304, 161), (300, 896, 320),
    (129, 3200, 47), (1024, 1024, 240), (2049, 4096, 96),
    # m <= 32: the dense kernel against the oracle only (the row layout runs the skinny kernel)
    (5, 512, 1), (200, 640, 5), (1000, 1152, 32),
])
def test_tiled_dense_matches_row_layout(n, k, m):
    """mxfp4_verify_gemm_tiled over mxfp4_tile_codes / mxfp4_tile_scales: bit-identical to
    mxfp4_verify_gemm where both run the dense kernel, and the oracle bar on every shape."""
    say(f"gemm: tiled dense n={n} k={k} m={m}")
    idx = n + 3 * k + m
    codes, scales, _ = omx.quantize(synth.weights(10, idx, n, k))
    x = synth.activations(10, idx, m, k)
    dc, ds, dx = dev(codes), dev(scales), dev_bf16(x)
    tc, ts = mxs.mxfp4_tile_codes(dc), mxs.mxfp4_tile_scales(ds)
    y_tiled = host(mxs.mxfp4_verify_gemm_tiled(tc, ts, n, k, dx))
    torch.cuda.synchronize()
    if m > 32:
        y_row = host(mxs.mxfp4_verify_gemm(dc, ds, dx))
        assert np.array_equal(y_tiled, y_row), (n, k, m)
    check_gemm(codes, scales, n, k, x, y_tiled, label=f"tiled dense {n}x{k}x{m}")


def test_tiled_batched_320_rows_sampled():
    """The batched verification case (64 sequences x 5 positions, 8192x28672) through the tiled
    weights: bit-identical to the row layout, and sampled rows against the oracle."""
    say("gemm: tiled batched 320x8192x28672")
    n, k, m = 8192, 28672, 320
    w = synth.weights(11, 0, n, k)
    dcodes, dscales = mxs.mxfp4_quantize(dev(w))
    x = synth.activations(11, 0, m, k)
    dx = dev_bf16(x)
    y_row = mxs.mxfp4_verify_gemm(dcodes, dscales, dx)
    y = mxs.mxfp4_verify_gemm_tiled(mxs.mxfp4_tile_codes(dcodes), mxs.mxfp4_tile_scales(dscales), n, k, dx)
    torch.cuda.synchronize()
    assert torch.equal(y, y_row)
    rows = np.unique(np.concatenate([np.random.default_rng(11).choice(n, 126, replace=False), [0, n - 1]]))
    rc, rs, _ = omx.quantize(w[rows])
    sub_c = np.zeros((n, k // 2), np.uint8)
    sub_s = np.zeros((n, k // 32), np.uint8)
    sub_c[rows], sub_s[rows] = rc, rs
    check_gemm(sub_c, sub_s, n, k, x, host(y)[:, rows], rows=rows, label="tiled batched")


def _tiled(dc, ds):
    return mxs.mxfp4_tile_codes(dc), mxs.mxfp4_tile_scales(ds)


@pytest.mark.parametrize("n,k,m", [
    (17, 512, 1), (300, 1024, 5), (4096, 4096, 5), (4100, 4096, 8), (1000, 2048, 16), (129, 3072, 32),
    (2048, 14336, 5),   # k walked in two phases
    # k % 512 != 0: the dense kernel on tiled weights (the row layout runs the fallback): oracle only
    (130, 1152, 5), (50, 640, 1),
])
def test_tiled_skinny_matches_row_layout(n, k, m):
    """mxfp4_verify_gemm_tiled at m <= 32: the skinny kernel on tiled codes and scales returns the
    row-layout result bit for bit, and the oracle bar."""
    say(f"gemm: tiled skinny n={n} k={k} m={m}")
    idx = n + 3 * k + m
    codes, scales, _ = omx.quantize(synth.weights(12, idx, n, k))
    x = synth.activations(12, idx, m, k)
    dc, ds, dx = dev(codes), dev(scales), dev_bf16(x)
    tc, ts = _tiled(dc, ds)
    y_tiled = host(mxs.mxfp4_verify_gemm_tiled(tc, ts, n, k, dx))
    torch.cuda.synchronize()
    if k % 512 == 0:
        assert np.array_equal(y_tiled, host(mxs.mxfp4_verify_gemm(dc, ds, dx))), (n, k, m)
    check_gemm(codes, scales, n, k, x, y_tiled, label=f"tiled skinny {n}x{k}x{m}")


@pytest.mark.parametrize("n,k,m", [(8200, 14336, 8), (8193, 16384, 16), (8192, 28672, 5)])
def test_tiled_phased_pairs_match_row_layout(n, k, m):
    """Several phases and pairs of row blocks (and a ragged last pair) on tiled weights:
    bit-identical to the row layout."""
    say(f"gemm: tiled phased pairs n={n} k={k} m={m}")
    dc, ds = mxs.mxfp4_quantize(dev(synth.weights(13, n + k + m, n, k)))
    dx = dev_bf16(synth.activations(13, n + k + m, m, k))
    tc, ts = _tiled(dc, ds)
    y_row = mxs.mxfp4_verify_gemm(dc, ds, dx)
    y_tiled = mxs.mxfp4_verify_gemm_tiled(tc, ts, n, k, dx)
    torch.cuda.synchronize()
    assert torch.equal(y_tiled, y_row), (n, k, m)


@pytest.mark.parametrize("shapes,k,m", [
    ([4096, 1024, 1024], 4096, 5),          # q | k | v (the row layout runs k and v in 8-row blocks)
    ([1000, 130, 17, 9], 1024, 5),          # partial row blocks
    ([1000, 130, 17, 9], 1024, 16),
    ([14336, 14336], 4096, 5),              # gate | up
    ([17, 300, 1, 4100, 64, 2048, 5, 33, 999], 512, 9),   # two launches, ragged
    ([300, 129], 14336, 8),                 # two phases
    ([300, 129], 1024, 64),                 # dense kernel per product
])
def test_grouped_tiled_matches_row_layout(shapes, k, m):
    """mxfp4_verify_gemm_grouped_tiled against the oracle on the small products, and bit for bit
    against the row-layout grouped call where both use the same row blocks (the row layout splits
    small products of a group into 8-row blocks, which changes nothing in any sum: a row's
    products and their order are those of its 16-row block)."""
    say(f"gemm: grouped tiled {shapes} k={k} m={m}")
    items, tiled, host_w = [], [], []
    for i, n in enumerate(shapes):
        codes, scales, _ = omx.quantize(synth.weights(14, 100 * i + len(shapes), n, k))
        x = synth.activations(14, len(shapes), m, k)
        dc, ds, dx = dev(codes), dev(scales), dev_bf16(x)
        items.append((dc, ds, dx))
        tiled.append((*_tiled(dc, ds), n, dx))
        host_w.append((codes, scales, x))
    ys_row = mxs.mxfp4_verify_gemm_grouped(items)
    ys_t = mxs.mxfp4_verify_gemm_grouped_tiled(tiled)
    torch.cuda.synchronize()
    for n, yr, yt, (codes, scales, x) in zip(shapes, ys_row, ys_t, host_w):
        assert torch.equal(yt, yr), (n, k, m)
        if n * k <= 1 << 22:
            check_gemm(codes, scales, n, k, x, host(yt), label=f"grouped tiled {n}x{k}x{m}")
