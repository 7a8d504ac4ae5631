"""mxfp4_quantize on the GPU vs the oracle quantizer: bit-exact codes, scales and flags."""
import numpy as np
import pytest
import torch

import mx_fp4_weight_amd as mxs
import synth
from oracle import mx as omx
from tests.gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


def gpu_quantize(w: np.ndarray):
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    codes, scales = mxs.mxfp4_quantize(dev(w), dev_flags=flags)
    torch.cuda.synchronize()
    return host(codes), host(scales), int(flags.item())


def test_tiny_config_bit_exact():
    say("quantize: tiny 1024x1024")
    w = synth.weights(1, 0, 1024, 1024)
    c, s, f = gpu_quantize(w)
    rc, rs, rf = omx.quantize(w)
    assert np.array_equal(c, rc) and np.array_equal(s, rs) and f == rf == 0


def test_hand_built_edge_blocks():
    say("quantize: edge blocks")
    rows = []
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    r = np.zeros(64, np.float32)
    r[:7] = ties
    r[7:14] = [-t for t in ties]
    r[14] = 4.0
    r[32:39] = [np.nextafter(np.float32(t), np.float32(0)) for t in ties]
    r[39:46] = [np.nextafter(np.float32(t), np.float32(9)) for t in ties]
    r[46] = 4.0
    rows.append(r)
    r = np.zeros(64, np.float32)
    r[3] = -0.0
    r[33] = 7.5                    # saturates
    r[34] = -7.99
    rows.append(r)
    r = np.zeros(64, np.float32)
    r[0] = np.float32(1e-45)       # subnormals: exponent clamps at -127
    r[1] = np.float32(2.0 ** -127)
    r[2] = -np.float32(3e-39)
    r[32] = np.finfo(np.float32).max
    r[33] = -np.finfo(np.float32).max
    rows.append(r)
    rng = np.random.default_rng(0)
    for scale in [1e-38, 1e-20, 1.0, 1e20, 1e37]:
        rows.append((rng.standard_normal(64) * scale).astype(np.float32))
    rows.append((rng.standard_t(1.5, 64)).astype(np.float32))
    w = np.stack(rows)
    c, s, f = gpu_quantize(w)
    rc, rs, rf = omx.quantize(w)
    assert np.array_equal(s, rs)
    assert np.array_equal(c, rc)
    assert f == rf == 0


def test_nonfinite_blocks_flagged():
    say("quantize: non-finite blocks")
    w = np.ones((3, 96), np.float32)
    w[0, 40] = np.nan
    w[2, 95] = -np.inf
    c, s, f = gpu_quantize(w)
    rc, rs, rf = omx.quantize(w)
    assert np.array_equal(c, rc) and np.array_equal(s, rs)
    assert f == rf == mxs.FLAG_NONFINITE


def test_exhaustive_magnitudes_one_scale():
    """Every fp32 in [0, 8) with 9 dropped mantissa bits, in blocks whose max fixes e = 0."""
    say("quantize: dense sweep")
    bits = np.arange(0, np.float32(8.0).view(np.uint32), 512, dtype=np.uint32)
    vals = bits.view(np.float32)
    nb = (vals.size + 30) // 31
    nb = (nb + 31) // 32 * 32               # whole 1024-element rows
    w = np.zeros((nb, 32), np.float32)
    flat = np.zeros(nb * 31, np.float32)
    flat[:vals.size] = vals
    w[:, :31] = flat.reshape(nb, 31)
    w[:, 31] = 4.0                           # amax in [4, 8): e = 0 for every block
    w[1::2] *= -1
    w = w.reshape(-1, 1024)
    c, s, _ = gpu_quantize(w)
    rc, rs, _ = omx.quantize(w)
    assert np.array_equal(c, rc) and np.array_equal(s, rs)


@pytest.mark.parametrize("n,k", [(4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336)])
def test_8b_shapes_bit_exact(n, k):
    say(f"quantize: 8B shape {n}x{k}")
    w = synth.weights(2, n * 7 + k, n, k)
    c, s, f = gpu_quantize(w)
    rc, rs, rf = omx.quantize(w)
    assert np.array_equal(c, rc) and np.array_equal(s, rs) and f == rf == 0


@pytest.mark.parametrize("n,k", [(8192, 8192), (28672, 8192), (8192, 28672)])
def test_70b_shapes_with_outliers_sampled(n, k):
    """Outlier channels x20 stress the block scales; every block of 64 sampled rows is compared."""
    say(f"quantize: 70B shape {n}x{k} with outliers")
    w = synth.weights(3, n * 3 + k, n, k, outlier_frac=0.01)
    c, s, f = gpu_quantize(w)
    rows = np.unique(np.concatenate([np.random.default_rng(n + k).choice(n, 62, replace=False), [0, n - 1]]))
    rc, rs, _ = omx.quantize(w[rows])
    assert np.array_equal(c[rows], rc) and np.array_equal(s[rows], rs) and f == 0
    # the outlier columns do change the scales of the blocks that hold them
    cols = synth.outlier_columns(3, n * 3 + k, k, 0.01)
    assert np.mean(np.isin(np.arange(k // 32), cols // 32)) > 0.2
