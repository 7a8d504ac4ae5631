"""The shared input generator: determinism, chunked regeneration, bf16 rounding."""
import numpy as np
import torch

import synth


def test_weights_regenerate_by_row_range():
    full = synth.weights(2, 3, 700, 64)
    part = synth.weights(2, 3, 700, 64, row_start=250, row_stop=530)
    assert np.array_equal(full[250:530], part)
    assert full.dtype == np.float32
    assert abs(full.std() - 0.02) < 0.001


def test_outliers_scale_whole_columns():
    base = synth.weights(3, 1, 300, 800)
    w = synth.weights(3, 1, 300, 800, outlier_frac=0.01)
    cols = synth.outlier_columns(3, 1, 800, 0.01)
    assert cols.size == 8
    ratio = w[:, cols] / base[:, cols]
    assert np.allclose(ratio, 20.0)
    mask = np.ones(800, bool)
    mask[cols] = False
    assert np.array_equal(w[:, mask], base[:, mask])


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = rng.standard_normal(100000).astype(np.float32) * np.float32(3.0)
    a[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 65504.0]   # ties
    ours = synth.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_logits_structure_and_seeds():
    t, d = synth.logits(1, 0, 4, 1024, 2.0, 0.5)
    assert t.shape == (5, 1024) and d.shape == (4, 1024)
    assert abs((t[:4] - d).std() - 0.5) < 0.03
    t2, _ = synth.logits(1, 0, 4, 1024, 2.0, 0.5)
    assert np.array_equal(t, t2)
    t3, _ = synth.logits(1, 1, 4, 1024, 2.0, 0.5)
    assert not np.array_equal(t, t3)
    tok = synth.gumbel_tokens(1, 0, d)
    assert tok.shape == (4,) and tok.dtype == np.int32 and (tok >= 0).all() and (tok < 1024).all()
    u = synth.uniforms(1, 0, 4)
    assert u.dtype == np.float32 and u.shape == (5,) and (u >= 0).all() and (u < 1).all()


def test_gumbel_tokens_follow_softmax():
    v = 6
    z = np.log(np.array([0.4, 0.2, 0.15, 0.1, 0.1, 0.05])).astype(np.float32)
    draws = np.array([synth.gumbel_tokens(9, s, z[None])[0] for s in range(6000)])
    freq = np.bincount(draws, minlength=v) / draws.size
    assert np.abs(freq - np.exp(z.astype(np.float64))).max() < 0.02
