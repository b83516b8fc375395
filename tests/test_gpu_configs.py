"""GPU parity on the shapes of the larger workloads (whole cache, long
rollout, wide heads), through the C-ABI, against the oracle.

The oracle runs on a subset of heads (every head where a step couples them);
the library always encodes every head.  Bar as in test_gpu_parity: ids,
snapshots, codes and (sigma, z) bit-exact, fp32 reconstruction bit-exact,
bf16 reconstruction = nearest-even rounding of it, attention within
2e-2 * max(1, |O_ref|).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import attend as o_attend
from oracle import xlayer as o_xlayer
from parity_util import (assert_stream_equal, attention_tolerance_check, bf16_of, f32_bits,
                         make_codec, oracle_stream)

pytestmark = pytest.mark.gpu
DEV = "cuda"
CHUNK = 4680


def _say(msg):
    print(msg, flush=True)


def test_long_rollout_one_layer_full_length():
    """One layer of the long-rollout workload at its full length: 12 heads,
    187200 tokens encoded as 40 calls of 4680 (centroid caching across the
    calls), 3 INT2 stages; then the 4680-query attention read of the whole
    packed layer.  Oracle: head 0."""
    cfgs = synth.LONG_ROLLOUT
    H, d, T = cfgs.n_heads, cfgs.head_dim, cfgs.tokens
    n_chunks = T // CHUNK
    codec = make_codec(H, d, cfgs.n_clusters, cfgs.n_stages, cfgs.bits, cfgs.group, iters=cfgs.iters,
                       max_tokens=T, max_chunks=n_chunks, max_chunk_tokens=CHUNK, max_q=cfgs.q_tokens)
    ost = [oracle_stream(1, d, cfgs.n_clusters, cfgs.iters, cfgs.n_stages, cfgs.bits, cfgs.group, "bf16")
           for _ in range(2)]
    _say(f"long rollout: {n_chunks} chunks of {CHUNK}, {H} heads")
    for c in range(n_chunks):
        k = synth.kv_tokens(cfgs, 0, 0, c * CHUNK, CHUNK)
        v = synth.kv_tokens(cfgs, 0, 1, c * CHUNK, CHUNK)
        codec.encode_chunk(k.to(DEV), v.to(DEV))
        ost[0].encode(k.float().numpy()[:1])
        ost[1].encode(v.float().numpy()[:1])
    torch.cuda.synchronize()
    assert codec.chunk_starts(0) == [c * CHUNK for c in range(n_chunks)]
    for kv in (0, 1):
        assert_stream_equal(codec, 0, kv, ost[kv], heads=[0])
        t0, t1 = T - 3 * CHUNK - 17, T          # a window across the last chunk boundaries
        rec = codec.reconstruct(0, 1, kv, t0, t1)[0, :1].cpu().numpy()
        np.testing.assert_array_equal(f32_bits(rec), f32_bits(ost[kv].xhat()[:, t0:t1]))
    q = synth.queries(cfgs, 0, cfgs.q_tokens)
    out, lse = codec.attend(0, q.to(DEV))
    sample = np.arange(0, cfgs.q_tokens, 97)
    o_ref, lse_ref = o_attend.attend(q.float().numpy()[:1, sample], ost[0].xhat(), ost[1].xhat())
    err = attention_tolerance_check(out.cpu().numpy()[:1, sample], lse.cpu().numpy()[:1, sample],
                                    o_ref, lse_ref)
    _say(f"long rollout attention (head 0, sampled) max abs err {err:.3e}")


def test_whole_cache_multi_layer_chunk():
    """The whole-cache call pattern on 4 layers of the Wan shape (12 heads):
    a two-chunk prefix, then one call that encodes a 4680-token chunk for
    every layer at once, then the reconstruction of every layer.  Oracle:
    head 0 of each layer."""
    cfgs = synth.WHOLE_CACHE
    L, H, d = 4, cfgs.n_heads, cfgs.head_dim
    n_list = [CHUNK, CHUNK, CHUNK]
    T = sum(n_list)
    codec = make_codec(H, d, cfgs.n_clusters, cfgs.n_stages, cfgs.bits, cfgs.group, iters=cfgs.iters,
                       max_tokens=T, max_chunks=len(n_list), max_chunk_tokens=CHUNK, n_layers=L, max_q=0)
    ost = {(l, kv): oracle_stream(1, d, cfgs.n_clusters, cfgs.iters, cfgs.n_stages, cfgs.bits, cfgs.group,
                                  "bf16") for l in range(L) for kv in (0, 1)}
    t0 = 0
    for i, n in enumerate(n_list):
        ks = torch.stack([synth.kv_tokens(cfgs, l, 0, t0, n) for l in range(L)])
        vs = torch.stack([synth.kv_tokens(cfgs, l, 1, t0, n) for l in range(L)])
        _say(f"whole cache: call {i} ({L} layers x {n} tokens)")
        codec.encode_chunk(ks.to(DEV), vs.to(DEV))
        for l in range(L):
            ost[(l, 0)].encode(ks[l].float().numpy()[:1])
            ost[(l, 1)].encode(vs[l].float().numpy()[:1])
        t0 += n
    torch.cuda.synchronize()
    for kv in (0, 1):
        recb = codec.reconstruct(0, L, kv, 0, T, out_dtype=torch.bfloat16)[:, :1].float().cpu().numpy()
        for l in range(L):
            assert_stream_equal(codec, l, kv, ost[(l, kv)], heads=[0])
            np.testing.assert_array_equal(f32_bits(recb[l]), f32_bits(bf16_of(ost[(l, kv)].xhat())),
                                          err_msg=f"layer {l} kv {kv}")
    rec = codec.reconstruct(2, 2, 1, CHUNK - 5, T)[:, :1].cpu().numpy()
    for i, l in enumerate((2, 3)):
        np.testing.assert_array_equal(f32_bits(rec[i]), f32_bits(ost[(l, 1)].xhat()[:, CHUNK - 5:]))


@pytest.mark.parametrize("S,bits", [(2, 2), (1, 4)])
def test_wide_head_variants(S, bits):
    """Wide heads: 40 heads, C = 512, G = 64, INT2 x 2 stages or INT4 x 1 stage,
    6240 tokens (four latent frames).  Oracle: heads 0 and 39."""
    cfgs = synth.scaled(synth.WIDE_HEAD, tokens=4 * 1560, n_stages=S, bits=bits)
    H, d, T, C = cfgs.n_heads, cfgs.head_dim, cfgs.tokens, cfgs.n_clusters
    heads = [0, H - 1]
    codec = make_codec(H, d, C, S, bits, cfgs.group, iters=cfgs.iters, max_tokens=T, max_chunks=1, max_q=0)
    k = synth.kv_tokens(cfgs, 0, 0, 0, T)
    v = synth.kv_tokens(cfgs, 0, 1, 0, T)
    _say(f"wide head S={S} b={bits}: {H} heads x {T} tokens, C={C}")
    codec.encode_chunk(k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    for kv, x in ((0, k), (1, v)):
        o = oracle_stream(len(heads), d, C, cfgs.iters, S, bits, cfgs.group, "bf16")
        o.encode(x.float().numpy()[heads])
        assert_stream_equal(codec, 0, kv, o, heads=heads)
        rec = codec.reconstruct(0, 1, kv, 0, T)[0].cpu().numpy()[heads]
        np.testing.assert_array_equal(f32_bits(rec), f32_bits(o.xhat()))


def test_wide_head_cross_layer():
    """Cross-layer residual mode on the wide-head shape: 40 heads, rank 32,
    C = 512, G = 64, two layers of one latent frame (1560 tokens).  The
    low-rank term couples all heads, so the oracle runs on every head."""
    cfgs = synth.scaled(synth.WIDE_HEAD, n_layers=2, tokens=1560)
    L, H, d, T, C, r = 2, cfgs.n_heads, cfgs.head_dim, cfgs.tokens, cfgs.n_clusters, cfgs.xlayer_rank
    parts = []
    for kv in (0, 1):
        B, U, V = synth.predictor(cfgs, 0, kv, rank=r)
        parts += [B.reshape(-1), U.reshape(-1), V.reshape(-1)]
    blob = torch.cat(parts)
    codec = make_codec(H, d, C, cfgs.n_stages, cfgs.bits, cfgs.group, iters=cfgs.iters, max_tokens=T,
                       max_chunks=1, n_layers=L, max_q=0, xlayer=1, rank=r, predictor=blob.to(DEV))
    xs = {kv: torch.stack([synth.kv_tokens(cfgs, l, kv, 0, T) for l in range(L)]) for kv in (0, 1)}
    _say(f"wide head cross-layer: {L} layers x {H} heads x {T} tokens, rank {r}")
    codec.encode_chunk(xs[0].to(DEV), xs[1].to(DEV))
    torch.cuda.synchronize()
    for kv in (0, 1):
        rec = codec.reconstruct(0, L, kv, 0, T).cpu().numpy()
        o0 = oracle_stream(H, d, C, cfgs.iters, cfgs.n_stages, cfgs.bits, cfgs.group, "bf16")
        o0.encode(xs[kv][0].float().numpy())
        assert_stream_equal(codec, 0, kv, o0)
        np.testing.assert_array_equal(f32_bits(rec[0]), f32_bits(o0.xhat()))
        B, U, V = synth.predictor(cfgs, 0, kv, rank=r)
        pred = o_xlayer.predict(o0.xhat(), B.float().numpy(), U.float().numpy(), V.float().numpy())
        o1 = oracle_stream(H, d, C, cfgs.iters, cfgs.n_stages, cfgs.bits, cfgs.group, "bf16")
        o1.encode_residual(xs[kv][1].float().numpy(), pred)
        assert_stream_equal(codec, 1, kv, o1, check_ids=False)
        np.testing.assert_array_equal(f32_bits(rec[1]), f32_bits(o1.xhat()), err_msg=f"layer 1 kv {kv}")
