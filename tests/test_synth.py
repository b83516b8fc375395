"""Checks of the seeded input generators (CPU only)."""
import numpy as np
import torch

import synth


def test_same_seed_same_bytes_and_slice_independence():
    cfg = synth.scaled(synth.WAN_LAYER, n_heads=2, tokens=6000)
    a = synth.kv_tokens(cfg, 3, 1, 0, 6000)
    b = synth.kv_tokens(cfg, 3, 1, 0, 6000)
    assert torch.equal(a, b)
    # a chunk generated on its own equals the same slice of the whole stream
    part = synth.kv_tokens(cfg, 3, 1, 1000, 4680)
    assert torch.equal(part, a[:, 1000:5680])
    other = synth.kv_tokens(cfg, 4, 1, 0, 6000)
    assert not torch.equal(a, other)


def test_structure_prototypes_drift_outliers():
    cfg = synth.scaled(synth.WAN_LAYER, n_heads=1, tokens=3 * synth.FRAME_TOKENS)
    x = synth.kv_tokens(cfg, 0, 0, 0, cfg.tokens)[0].float()
    f0 = x[:synth.FRAME_TOKENS]
    f1 = x[synth.FRAME_TOKENS:2 * synth.FRAME_TOKENS]
    scale = synth.channel_scale(cfg, 0, 0)[0]
    assert int((scale == 10.0).sum()) == cfg.n_out
    # same spatial position in consecutive frames: same prototype + drift + fresh noise
    d = (f1 - f0) / scale
    sd = float(d.std())
    expect = (2 * 0.1 ** 2 + 0.02 ** 2) ** 0.5
    assert abs(sd - expect) / expect < 0.05
    # channel magnitudes: outlier channels ~10x the rest
    ch_sd = (x / 1.0).std(dim=0)
    assert float(ch_sd[scale == 10.0].mean() / ch_sd[scale == 1.0].mean()) > 7


def test_tiny_recipe_statistics():
    cfg = synth.TINY
    x = synth.kv_tokens(cfg, 0, 0, 0, cfg.tokens).float()
    assert x.dtype == torch.float32 and x.shape == (2, 4096, 64)
    scale = synth.channel_scale(cfg, 0, 0)
    base = torch.log(scale[scale < 5.0])
    # lognormal(0, 0.5) channel scales
    assert abs(float(base.std()) - 0.5) < 0.15
    # about 32 distinct prototypes: token-to-nearest-token distances cluster near 2*0.01*64
    xs = (x[0] / scale[0]).numpy()[:512]
    d2 = ((xs[:, None, :] - xs[None, :, :]) ** 2).sum(-1)
    np.fill_diagonal(d2, np.inf)
    nearest = d2.min(axis=1)
    assert np.median(nearest) < 4 * 2 * 0.01 * 64


def test_queries_and_predictor_shapes():
    cfg = synth.scaled(synth.WIDE_HEAD, n_heads=2)
    q = synth.queries(synth.WAN_LAYER, 0, 10)
    assert q.dtype == torch.bfloat16 and q.shape == (12, 10, 128)
    B, U, V = synth.predictor(cfg, 0, 0)
    assert B.shape == (2, 128, 128) and U.shape == (256, 32) and V.shape == (256, 32)
    assert abs(float(B.float().var()) - 1.0 / 128) < 0.1 / 128
