"""MX-quantized activations and the W4A8 / W4A4 verify GEMM on the GPU vs the oracle
(oracle/mxact.py).

mx_quantize_act: codes, scales and flags bit-exact (the rounding is integer
arithmetic on both sides). mx_verify_gemm_act: relative L2 <= 2e-3 against the
fp64 product of the quantized operands, each element within 1e-4 of
sum_k |x^_k w^_k|; one-hot activations return weight columns exactly.
"""
import numpy as np
import pytest
import torch

import mx_fp4_weight_amd as mxs
import synth
from oracle import gemm as ogemm
from oracle import mx as omx
from oracle import mxact as oa
from tests.gpu_util import ELEM, REL_L2, dev, dev_bf16, host, say

pytestmark = pytest.mark.gpu

FMTS = [oa.FMT_FP8, oa.FMT_FP4]
NAME = {oa.FMT_FP8: "fp8", oa.FMT_FP4: "fp4"}


def gpu_quantize(xbits, fmt):
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    c, s = mxs.mx_quantize_act(dev_bf16(xbits), fmt, dev_flags=flags)
    torch.cuda.synchronize()
    return host(c), host(s), int(flags.item())


def check_quantize(xbits, fmt, label):
    c, s, f = gpu_quantize(xbits, fmt)
    rc, rs, rf = oa.quantize(xbits, fmt)
    assert np.array_equal(s, rs), (label, np.argwhere(s != rs)[:5])
    assert np.array_equal(c, rc), (label, np.argwhere(c != rc)[:5])
    assert f == rf, (label, f, rf)
    return rc, rs


def run_gemm(wc, ws, ac, asc, fmt):
    y = mxs.mx_verify_gemm_act(dev(wc), dev(ws), dev(ac), dev(asc), fmt)
    torch.cuda.synchronize()
    return host(y)


def check_gemm(wc, ws, n, k, ac, asc, fmt, y_gpu, rows=None, label=""):
    ref = oa.gemm(wc, ws, n, k, ac, asc, fmt, rows=rows)
    wsel = (wc, ws) if rows is None else (wc[rows], ws[rows])
    bound = np.abs(oa.dequantize(ac, asc, fmt, k)) @ np.abs(omx.dequantize(wsel[0], wsel[1], k)).T
    got = np.asarray(y_gpu, np.float64)
    assert got.shape == ref.shape, (label, got.shape, ref.shape)
    assert np.isfinite(got).all(), label
    err = got - ref
    rel = np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300)
    assert rel <= REL_L2, (label, rel)
    worst = np.max(np.abs(err) - ELEM * bound)
    assert worst <= 1e-30, (label, worst)
    return rel


# ------------------------------------------------------------------ quantizer

@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_random_bit_exact(fmt):
    say(f"act quantize {NAME[fmt]}: 320x4096 N(0,1) and 7x1024 wide-range blocks")
    check_quantize(synth.activations(71, fmt, 320, 4096), fmt, "n01")
    r = synth.rng(71, 1, fmt)
    v = r.standard_normal((7, 1024)) * 2.0 ** r.integers(-120, 120, (7, 32)).repeat(32, axis=1)
    check_quantize(synth.f32_to_bf16_bits(v.astype(np.float32)), fmt, "wide")


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_every_bf16_in_a_block(fmt):
    """Every finite bf16 pattern of both signs, 31 per block beside a block maximum that fixes the
    scale (448 for FP8, 6 for FP4), and again in blocks of 32 that set their own scale: every
    rounding path, ties, subnormal inputs and outputs."""
    say(f"act quantize {NAME[fmt]}: every bf16 value")
    vals = np.arange(0, 0x7F80, dtype=np.uint16)              # all non-negative finite bf16 patterns
    vals = np.concatenate([vals, vals | 0x8000])
    per = 31 * 32                                              # whole 1024-wide rows of blocks
    fixed = np.concatenate([vals, np.zeros((-len(vals)) % per, np.uint16)]).reshape(-1, 31)
    top = synth.f32_to_bf16_bits(np.float32(448.0 if fmt == oa.FMT_FP8 else 6.0))
    blocks = np.concatenate([np.full((len(fixed), 1), top, np.uint16), fixed], axis=1)
    check_quantize(blocks.reshape(-1, 1024), fmt, "fixed max")
    own = np.concatenate([vals, np.zeros((-len(vals)) % 1024, np.uint16)]).reshape(-1, 1024)
    check_quantize(own, fmt, "own max")


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_edge_blocks(fmt):
    say(f"act quantize {NAME[fmt]}: edge blocks")
    rows = np.zeros((8, 32), np.float32)
    rows[0, 0] = 256.0
    rows[0, 1:8] = [1.0625, 1.1875, 17.0, 19.0, 0.001953125 * 1.5, 2.0 ** -10, -(2.0 ** -10)]
    rows[1, 0] = 480.0
    rows[1, 1] = -470.0
    rows[1, 2] = 7.5
    rows[2, 3] = -0.0
    rows[3, :] = 3.0
    rows[4, 0] = 2.0 ** -133
    rows[4, 1] = -(2.0 ** -130)
    rows[5, 5] = np.nan
    rows[6, 9] = -np.inf
    xb = synth.f32_to_bf16_bits(rows)
    xb[7, :] = 0x7F7F                                   # largest finite bf16, both signs
    xb[7, 1::2] = 0xFF7F
    check_quantize(xb.reshape(2, 128), fmt, "edges")


# ------------------------------------------------------------------ GEMM

@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_one_hot_exact(fmt):
    say(f"act gemm {NAME[fmt]}: one-hot")
    n, k = 200, 640
    wc, ws, _ = omx.quantize(synth.weights(72, fmt, n, k))
    cols = synth.rng(72, 1, fmt).integers(0, k, 96)
    x = np.zeros((96, k), np.float32)
    x[np.arange(96), cols] = 1.0
    ac, asc, _ = oa.quantize(synth.f32_to_bf16_bits(x), fmt)
    y = run_gemm(wc, ws, ac, asc, fmt)
    wd = omx.dequantize(wc, ws, k)
    for i, c in enumerate(cols):
        assert np.array_equal(y[i].astype(np.float64), wd[:, c]), i


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k,m", [
    (1, 128, 1), (17, 128, 5), (130, 384, 80), (257, 1024, 100), (1000, 2304, 161), (64, 128, 320),
    (300, 896, 81), (129, 3200, 47), (1024, 1024, 240), (33, 640, 33), (5, 512, 1), (128, 4096, 16),
])
def test_gemm_ragged_shapes(fmt, n, k, m):
    say(f"act gemm {NAME[fmt]}: n={n} k={k} m={m}")
    idx = n + 3 * k + m
    wc, ws, _ = omx.quantize(synth.weights(73, idx, n, k))
    ac, asc, _ = oa.quantize(synth.activations(73, idx, m, k), fmt)
    check_gemm(wc, ws, n, k, ac, asc, fmt, run_gemm(wc, ws, ac, asc, fmt), label=f"{n}x{k}x{m}")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_scale_extremes(fmt):
    """Weight and activation block scales far apart (products of 2^(sw + sx - 254) near the fp32
    range), all-zero blocks on both sides."""
    say(f"act gemm {NAME[fmt]}: scale extremes")
    n, k, m = 64, 512, 40
    r = synth.rng(74, 0, fmt)
    w = r.standard_normal((n, k)) * 2.0 ** r.integers(-60, 60, (n, k // 32)).repeat(32, axis=1)
    w[3] = 0
    x = r.standard_normal((m, k)) * 2.0 ** r.integers(-50, 50, (m, k // 32)).repeat(32, axis=1)
    x[5, :64] = 0
    wc, ws, _ = omx.quantize(w.astype(np.float32))
    ac, asc, _ = oa.quantize(synth.f32_to_bf16_bits(x.astype(np.float32)), fmt)
    check_gemm(wc, ws, n, k, ac, asc, fmt, run_gemm(wc, ws, ac, asc, fmt), label="extremes")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_nan_activation_block(fmt):
    """A refused activation block (scale 0xFF) turns that position's outputs into NaN only."""
    say(f"act gemm {NAME[fmt]}: NaN activation block")
    n, k, m = 96, 512, 20
    wc, ws, _ = omx.quantize(synth.weights(75, fmt, n, k))
    x = synth.activations(75, fmt, m, k)
    x[7, 100] = 0x7FC0                                   # bf16 NaN
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    dac, das = mxs.mx_quantize_act(dev_bf16(x), fmt, dev_flags=flags)
    y = host(mxs.mx_verify_gemm_act(dev(wc), dev(ws), dac, das, fmt))
    assert int(flags.item()) == mxs.FLAG_NONFINITE
    assert np.isnan(y[7]).all()
    keep = [i for i in range(m) if i != 7]
    ac, asc, _ = oa.quantize(x[keep], fmt)
    check_gemm(wc, ws, n, k, ac, asc, fmt, y[keep], label="nan block")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_batched_shape_sampled(fmt):
    """64 sequences x 5 positions against 8192x28672: weights and activations quantized on the
    GPU (sampled weight rows and all activations checked bit-exact), sampled outputs; the distance
    to the weight-only product of the bf16 activations is reported."""
    say(f"act gemm {NAME[fmt]}: batched 320x8192x28672")
    n, k, m = 8192, 28672, 320
    w = synth.weights(76, 0, n, k)
    dwc, dws = mxs.mxfp4_quantize(dev(w))
    x = synth.activations(76, fmt, m, k)
    dac, das = mxs.mx_quantize_act(dev_bf16(x), fmt)
    y = mxs.mx_verify_gemm_act(dwc, dws, dac, das, fmt)
    torch.cuda.synchronize()
    ac, asc, _ = oa.quantize(x, fmt)
    assert np.array_equal(host(dac), ac) and np.array_equal(host(das), asc)
    rows = np.unique(np.concatenate([synth.rng(76, 1, fmt).choice(n, 126, replace=False), [0, n - 1]]))
    rc, rs, _ = omx.quantize(w[rows])
    assert np.array_equal(host(dwc)[rows], rc) and np.array_equal(host(dws)[rows], rs)
    yr = host(y)[:, rows]
    sub_c = np.zeros((n, k // 2), np.uint8)
    sub_s = np.zeros((n, k // 32), np.uint8)
    sub_c[rows], sub_s[rows] = rc, rs
    check_gemm(sub_c, sub_s, n, k, ac, asc, fmt, yr, rows=rows, label="batched")
    wonly = ogemm.verify_gemm(sub_c, sub_s, n, k, x, rows=rows)
    say(f"  {NAME[fmt]} activations vs bf16 activations: rel L2 "
        f"{np.linalg.norm(yr - wonly) / np.linalg.norm(wonly):.3e}")


def tile_ref(codes, n, k):
    """The tiled layout written out with NumPy: (16-row tile, 128-k group, block g, row r, 16 bytes)."""
    n16 = (n + 15) // 16 * 16
    full = np.zeros((n16, k // 2), np.uint8)
    full[:n] = codes
    t = full.reshape(n16 // 16, 16, k // 128, 4, 16)     # tile, r, group, g, byte
    return t.transpose(0, 2, 3, 1, 4).reshape(-1)        # tile, group, g, r, byte


@pytest.mark.parametrize("n,k", [(1, 128), (16, 256), (17, 384), (100, 1024), (1000, 2304), (4099, 4096)])
def test_tile_codes_layout(n, k):
    """mxfp4_tile_codes is the documented byte permutation (random bytes, ragged n)."""
    say(f"tile codes n={n} k={k}")
    codes = synth.rng(77, n, k).integers(0, 256, (n, k // 2), dtype=np.uint8)
    got = host(mxs.mxfp4_tile_codes(dev(codes)))
    torch.cuda.synchronize()
    assert got.size == mxs.mxfp4_tiled_bytes(n, k)
    assert np.array_equal(got, tile_ref(codes, n, k))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k,m", [
    (1, 128, 1), (17, 128, 5), (130, 384, 80), (257, 1024, 100), (1000, 2304, 161), (300, 896, 81),
    (129, 3200, 47), (1024, 1024, 240), (5, 512, 1),
])
def test_gemm_tiled_matches_row_layout(fmt, n, k, m):
    """The tiled-weight product equals the row-layout product bit for bit (same operands, same
    sums), and the oracle bar on one shape in three."""
    say(f"act gemm tiled {NAME[fmt]}: n={n} k={k} m={m}")
    idx = n + 3 * k + m
    wc, ws, _ = omx.quantize(synth.weights(78, idx, n, k))
    ac, asc, _ = oa.quantize(synth.activations(78, idx, m, k), fmt)
    dwc, dws, dac, das = dev(wc), dev(ws), dev(ac), dev(asc)
    y_row = host(mxs.mx_verify_gemm_act(dwc, dws, dac, das, fmt))
    tiled = mxs.mxfp4_tile_codes(dwc)
    tiled_s = mxs.mxfp4_tile_scales(dws)
    y_tiled = host(mxs.mx_verify_gemm_act_tiled(tiled, tiled_s, n, k, dac, das, fmt))
    torch.cuda.synchronize()
    assert np.array_equal(y_tiled, y_row), (n, k, m)
    if idx % 3 == 0:
        check_gemm(wc, ws, n, k, ac, asc, fmt, y_tiled, label=f"tiled {n}x{k}x{m}")


def tile_scales_ref(scales, n, k):
    """The tiled scale layout written out with NumPy: (128-row tile, 512-k window, row r, 16 bytes)."""
    n128, kb, win = (n + 127) // 128 * 128, k // 32, (k + 511) // 512
    full = np.zeros((n128, win * 16), np.uint8)
    full[:n, :kb] = scales
    return full.reshape(n128 // 128, 128, win, 16).transpose(0, 2, 1, 3).reshape(-1)


@pytest.mark.parametrize("n,k", [(1, 128), (128, 512), (129, 384), (300, 1664), (1000, 2304), (257, 4096)])
def test_tile_scales_layout(n, k):
    """mxfp4_tile_scales is the documented byte layout (random bytes, ragged n and k)."""
    say(f"tile scales n={n} k={k}")
    scales = synth.rng(79, n, k).integers(0, 256, (n, k // 32), dtype=np.uint8)
    got = host(mxs.mxfp4_tile_scales(dev(scales)))
    torch.cuda.synchronize()
    assert got.size == mxs.mxfp4_tiled_scale_bytes(n, k)
    assert np.array_equal(got, tile_scales_ref(scales, n, k))
