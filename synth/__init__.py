"""Seeded synthetic KV caches, queries and predictor weights.

This module only draws random inputs; it holds none of the codec's
arithmetic and is shared by the tests, the oracle runs and the benchmark.

The pages measure on real video models (LongCat-Video, HY-WorldPlay,
Self-Forcing on Wan2.1, MAGI-1) and datasets that are not available here;
these seeded caches stand in for them.  Shapes follow a Wan2.1-style latent
layout: 1560 tokens per 480p latent frame, 4680-token chunks (three frames).
The structure follows the QVG explainer's observation ("Sommario tecnico"
2.A) that spatially or temporally close video tokens are similar: each
spatial position of a head carries one of a set of Gaussian prototypes that
drift slowly from frame to frame, plus per-token noise, with a few outlier
channels scaled up.

Recipe, per (layer, tensor K|V, head):
  prototypes P0 ~ N(0, 1)                      [n_proto, d]
  per frame f >= 1: P_f = P_{f-1} + N(0, drift^2)   (drift std 0.02; 0 for Tiny)
  label per spatial position (Tiny: per token), uniform over prototypes
  channel scale: lognormal(0, 0.5) per channel for Tiny, else 1; then
  n_out distinct channels multiplied by the outlier factor
  token t = f*1560 + p:  x_t = scale * (P_f[label(p)] + eps_t),  eps ~ N(0, 0.1^2)
  cast to the cache dtype (bf16 round-to-nearest-even, or fp32 for Tiny)
Queries ~ N(0, 1).  Predictor B, U, V ~ N(0, 1/128) (variance), cast to bf16.

Every draw comes from a torch.Generator seeded from
numpy.random.SeedSequence(0x51564730, spawn_key=(config, layer, kv, purpose, index)),
so a slice of a stream does not depend on how the stream is chunked.  The
generator runs on the device that receives the tensor; values are
reproducible per device type.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np
import torch

FRAME_TOKENS = 1560
BASE_SEED = 0x51564730
_PURPOSE = {"prototypes": 1, "drift": 2, "noise": 3, "labels": 4, "channels": 5,
            "queries": 6, "predictor": 7}


@dataclass(frozen=True)
class Config:
    name: str
    index: int
    n_layers: int
    n_heads: int
    tokens: int               # cache tokens per layer
    head_dim: int
    dtype: str                # "f32" or "bf16"
    n_proto: int
    n_out: int
    out_factor: float
    lognormal_channels: bool
    drift: float
    per_token_labels: bool
    n_clusters: int
    iters: int
    n_stages: int
    bits: int
    group: int
    q_tokens: int
    q_dtype: str
    chunk_tokens: int         # tokens per encode call when the stream is built
    xlayer_rank: int = 0
    variants: Tuple = field(default_factory=tuple)


TINY = Config("tiny", 0, 1, 2, 4096, 64, "f32", 32, 2, 10.0, True, 0.0, True,
              16, 5, 2, 2, 64, 256, "f32", 4096)
WAN_LAYER = Config("wan_layer", 1, 1, 12, 32760, 128, "bf16", 256, 4, 10.0, False, 0.02,
                   False, 256, 5, 2, 2, 32, 4680, "bf16", 32760)
WHOLE_CACHE = Config("whole_cache", 2, 30, 12, 32760 + 4680, 128, "bf16", 256, 4, 10.0, False,
                     0.02, False, 256, 5, 2, 2, 32, 4680, "bf16", 4680)
LONG_ROLLOUT = Config("long_rollout", 3, 30, 12, 187200, 128, "bf16", 256, 4, 10.0, False, 0.02,
                      False, 256, 5, 3, 2, 32, 4680, "bf16", 4680)
WIDE_HEAD = Config("wide_head", 4, 40, 40, 62400, 128, "bf16", 256, 8, 20.0, False, 0.02,
                   False, 512, 5, 2, 2, 64, 0, "bf16", 62400, xlayer_rank=32,
                   variants=(("int2x2", 2, 2, 64), ("int4x1", 1, 4, 64)))

CONFIGS = {c.name: c for c in (TINY, WAN_LAYER, WHOLE_CACHE, LONG_ROLLOUT, WIDE_HEAD)}


def _gen(cfg, layer, kv, purpose, index, device):
    ss = np.random.SeedSequence(BASE_SEED, spawn_key=(cfg.index, layer, kv, _PURPOSE[purpose], index))
    seed = int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _torch_dtype(name):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def channel_scale(cfg, layer, kv, device="cpu"):
    """[H, d] float32 per-channel scale (lognormal for Tiny, outliers scaled up)."""
    g = _gen(cfg, layer, kv, "channels", 0, device)
    H, d = cfg.n_heads, cfg.head_dim
    if cfg.lognormal_channels:
        scale = torch.exp(0.5 * torch.randn((H, d), generator=g, device=device))
    else:
        scale = torch.ones((H, d), device=device)
    for h in range(H):
        idx = torch.randperm(d, generator=g, device=device)[:cfg.n_out]
        scale[h, idx] *= cfg.out_factor
    return scale


def kv_tokens(cfg, layer, kv, t0, n, device="cpu", out_dtype: Optional[torch.dtype] = None):
    """Tokens [t0, t0+n) of one (layer, kv) stream: [H, n, d] in the cache dtype."""
    H, d = cfg.n_heads, cfg.head_dim
    dtype = out_dtype or _torch_dtype(cfg.dtype)
    out = torch.empty((H, n, d), dtype=dtype, device=device)
    if n == 0:
        return out
    scale = channel_scale(cfg, layer, kv, device)
    protos = torch.randn((H, cfg.n_proto, d), generator=_gen(cfg, layer, kv, "prototypes", 0, device),
                         device=device)
    if cfg.per_token_labels:
        labels = torch.randint(cfg.n_proto, (H, cfg.tokens),
                               generator=_gen(cfg, layer, kv, "labels", 0, device), device=device)
        eps = 0.1 * torch.randn((H, cfg.tokens, d), generator=_gen(cfg, layer, kv, "noise", 0, device),
                                device=device)
        sl = slice(t0, t0 + n)
        x = protos[torch.arange(H, device=device)[:, None], labels[:, sl]] + eps[:, sl]
        out.copy_((scale[:, None, :] * x).to(dtype))
        return out
    labels = torch.randint(cfg.n_proto, (H, FRAME_TOKENS),
                           generator=_gen(cfg, layer, kv, "labels", 0, device), device=device)
    hidx = torch.arange(H, device=device)[:, None]
    f_first, f_last = t0 // FRAME_TOKENS, (t0 + n - 1) // FRAME_TOKENS
    P = protos
    for f in range(1, f_first + 1):
        P = P + cfg.drift * torch.randn(P.shape, generator=_gen(cfg, layer, kv, "drift", f, device),
                                        device=device)
    for f in range(f_first, f_last + 1):
        if f > f_first:
            P = P + cfg.drift * torch.randn(P.shape, generator=_gen(cfg, layer, kv, "drift", f, device),
                                            device=device)
        a = max(t0, f * FRAME_TOKENS)
        b = min(t0 + n, (f + 1) * FRAME_TOKENS)
        p0, p1 = a - f * FRAME_TOKENS, b - f * FRAME_TOKENS
        eps = 0.1 * torch.randn((H, FRAME_TOKENS, d), generator=_gen(cfg, layer, kv, "noise", f, device),
                                device=device)
        x = P[hidx, labels[:, p0:p1]] + eps[:, p0:p1]
        out[:, a - t0:b - t0] = (scale[:, None, :] * x).to(dtype)
    return out


def queries(cfg, layer, n, device="cpu"):
    """[H, n, d] queries ~ N(0, 1) in the configured query dtype."""
    q = torch.randn((cfg.n_heads, n, cfg.head_dim), generator=_gen(cfg, layer, 0, "queries", 0, device),
                    device=device)
    return q.to(_torch_dtype(cfg.q_dtype))


def predictor(cfg, layer, kv, device="cpu", rank=None):
    """Cross-layer predictor for layer -> layer+1: B [H, d, d], U, V [H*d, r], all bf16."""
    H, d = cfg.n_heads, cfg.head_dim
    r = rank or cfg.xlayer_rank
    g = _gen(cfg, layer, kv, "predictor", 0, device)
    std = (1.0 / 128.0) ** 0.5
    B = (std * torch.randn((H, d, d), generator=g, device=device)).to(torch.bfloat16)
    U = (std * torch.randn((H * d, r), generator=g, device=device)).to(torch.bfloat16)
    V = (std * torch.randn((H * d, r), generator=g, device=device)).to(torch.bfloat16)
    return B, U, V


def scaled(cfg, **kw):
    """A copy of ``cfg`` with some fields replaced (smaller test shapes)."""
    from dataclasses import replace
    return replace(cfg, **kw)
