"""GPU parity at the full sizes of the larger workloads, and on the k-means
paths that large cluster counts take, through the C-ABI, against the oracle.

Inputs are generated on the device (as the benchmark does) and copied back
for the oracle, which runs on sampled heads (every head where a step couples
them).  Bar as in test_gpu_parity: ids, snapshots, codes and (sigma, z)
bit-exact, fp32 reconstruction bit-exact.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import xlayer as o_xlayer
from parity_util import assert_stream_equal, f32_bits, make_codec, oracle_stream

pytestmark = pytest.mark.gpu
DEV = "cuda"
CHUNK = 4680


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("S,bits", [(2, 2), (1, 4)])
def test_wide_head_full_length(S, bits):
    """Wide heads at their full length: 40 heads x 62400 tokens, C = 512,
    G = 64, 8 outlier channels x20, INT2 x 2 stages or INT4 x 1 stage, one
    call (the launch shapes of the benchmark's wide-head layer).  Oracle:
    heads 0 and 39 of K and V."""
    cfgs = synth.scaled(synth.WIDE_HEAD, n_stages=S, bits=bits)
    H, d, T, C = cfgs.n_heads, cfgs.head_dim, cfgs.tokens, cfgs.n_clusters
    heads = [0, H - 1]
    codec = make_codec(H, d, C, S, bits, cfgs.group, iters=cfgs.iters, max_tokens=T, max_chunks=1, max_q=0)
    k = synth.kv_tokens(cfgs, 0, 0, 0, T, device=DEV)
    v = synth.kv_tokens(cfgs, 0, 1, 0, T, device=DEV)
    _say(f"wide head full length S={S} b={bits}: {H} heads x {T} tokens, C={C}")
    codec.encode_chunk(k, v)
    torch.cuda.synchronize()
    for kv, x in ((0, k), (1, v)):
        o = oracle_stream(len(heads), d, C, cfgs.iters, S, bits, cfgs.group, "bf16")
        o.encode(x[heads].float().cpu().numpy())
        assert_stream_equal(codec, 0, kv, o, heads=heads)
        rec = codec.reconstruct(0, 1, kv, 0, T)[0][heads].cpu().numpy()
        np.testing.assert_array_equal(f32_bits(rec), f32_bits(o.xhat()))
        _say(f"  kv {kv}: heads {heads} bit-exact")


def test_wide_head_cross_layer_chunk():
    """Cross-layer residual mode on the wide-head shape at a chunk of 4680
    tokens: 40 heads, rank 32, C = 512, G = 64, two layers.  The low-rank
    term couples all heads, so the oracle runs on every head."""
    cfgs = synth.scaled(synth.WIDE_HEAD, n_layers=2)
    L, H, d, T, C, r = 2, cfgs.n_heads, cfgs.head_dim, CHUNK, cfgs.n_clusters, cfgs.xlayer_rank
    parts = []
    for kv in (0, 1):
        B, U, V = synth.predictor(cfgs, 0, kv, rank=r)
        parts += [B.reshape(-1), U.reshape(-1), V.reshape(-1)]
    codec = make_codec(H, d, C, cfgs.n_stages, cfgs.bits, cfgs.group, iters=cfgs.iters, max_tokens=T,
                       max_chunks=1, n_layers=L, max_q=0, xlayer=1, rank=r, predictor=torch.cat(parts).to(DEV))
    xs = {kv: torch.stack([synth.kv_tokens(cfgs, l, kv, 0, T, device=DEV) for l in range(L)]) for kv in (0, 1)}
    _say(f"wide head cross-layer: {L} layers x {H} heads x {T} tokens, rank {r}")
    codec.encode_chunk(xs[0], xs[1])
    torch.cuda.synchronize()
    for kv in (0, 1):
        rec = codec.reconstruct(0, L, kv, 0, T).cpu().numpy()
        x0 = xs[kv][0].float().cpu().numpy()
        x1 = xs[kv][1].float().cpu().numpy()
        o0 = oracle_stream(H, d, C, cfgs.iters, cfgs.n_stages, cfgs.bits, cfgs.group, "bf16")
        o0.encode(x0)
        assert_stream_equal(codec, 0, kv, o0)
        np.testing.assert_array_equal(f32_bits(rec[0]), f32_bits(o0.xhat()))
        B, U, V = synth.predictor(cfgs, 0, kv, rank=r)
        pred = o_xlayer.predict(o0.xhat(), B.float().numpy(), U.float().numpy(), V.float().numpy())
        o1 = oracle_stream(H, d, C, cfgs.iters, cfgs.n_stages, cfgs.bits, cfgs.group, "bf16")
        o1.encode_residual(x1, pred)
        assert_stream_equal(codec, 1, kv, o1, check_ids=False)
        np.testing.assert_array_equal(f32_bits(rec[1]), f32_bits(o1.xhat()), err_msg=f"layer 1 kv {kv}")
        _say(f"  kv {kv}: both layers bit-exact")


def test_whole_cache_prefix_then_chunk_eight_layers():
    """The whole-cache pattern at its real sizes on 8 layers of the Wan shape:
    a 32760-token prefix per layer (one call for all layers), then one call
    encoding a 4680-token chunk into every layer, then the reconstruction of
    all 37440 tokens of every layer.  Oracle: head 5 of each layer."""
    cfgs = synth.WHOLE_CACHE
    L, H, d = 8, cfgs.n_heads, cfgs.head_dim
    n_list = [32760, CHUNK]
    T = sum(n_list)
    h = 5
    codec = make_codec(H, d, cfgs.n_clusters, cfgs.n_stages, cfgs.bits, cfgs.group, iters=cfgs.iters,
                       max_tokens=T, max_chunks=2, max_chunk_tokens=32760, n_layers=L, max_q=0)
    ost = {(l, kv): oracle_stream(1, d, cfgs.n_clusters, cfgs.iters, cfgs.n_stages, cfgs.bits, cfgs.group,
                                  "bf16") for l in range(L) for kv in (0, 1)}
    t0 = 0
    for i, n in enumerate(n_list):
        ks = torch.stack([synth.kv_tokens(cfgs, l, 0, t0, n, device=DEV) for l in range(L)])
        vs = torch.stack([synth.kv_tokens(cfgs, l, 1, t0, n, device=DEV) for l in range(L)])
        _say(f"whole cache: call {i} ({L} layers x {n} tokens)")
        codec.encode_chunk(ks, vs)
        kh = ks[:, h:h + 1].float().cpu().numpy()
        vh = vs[:, h:h + 1].float().cpu().numpy()
        for l in range(L):
            ost[(l, 0)].encode(kh[l])
            ost[(l, 1)].encode(vh[l])
        t0 += n
    torch.cuda.synchronize()
    for kv in (0, 1):
        rec = codec.reconstruct(0, L, kv, 0, T)[:, h].cpu().numpy()
        for l in range(L):
            assert_stream_equal(codec, l, kv, ost[(l, kv)], heads=[h])
            np.testing.assert_array_equal(f32_bits(rec[l]), f32_bits(ost[(l, kv)].xhat()[0]),
                                          err_msg=f"layer {l} kv {kv}")
    _say("whole cache: 8 layers x K,V bit-exact on head 5")


@pytest.mark.parametrize("dtype,C,d", [("bf16", 1500, 64), ("bf16", 5000, 64), ("f32", 300, 128)])
def test_large_cluster_counts(dtype, C, d):
    """The k-means paths of larger codebooks: bf16 with C = 1500 (scalar
    assignment, bitonic tile sort) and C = 5000 (scalar assignment,
    member-list update), fp32 with C = 300 (fp32 assignment, counting sort
    for C <= 1024, 2-byte ids).  6000 tokens of two heads in two calls
    (warm start), 2 INT2 stages, G = 32."""
    cfgs = synth.scaled(synth.WAN_LAYER, n_heads=2, head_dim=d, n_clusters=C, tokens=6000, dtype=dtype)
    H = cfgs.n_heads
    n_list = [4000, 2000]
    codec = make_codec(H, d, C, 2, 2, 32, iters=cfgs.iters, max_tokens=sum(n_list), max_chunks=2, dtype=dtype,
                       max_q=0)
    ost = [oracle_stream(H, d, C, cfgs.iters, 2, 2, 32, dtype) for _ in range(2)]
    t0 = 0
    for n in n_list:
        k = synth.kv_tokens(cfgs, 0, 0, t0, n)
        v = synth.kv_tokens(cfgs, 0, 1, t0, n)
        _say(f"C={C} {dtype} d={d}: call of {n} tokens")
        codec.encode_chunk(k.to(DEV), v.to(DEV))
        ost[0].encode(k.float().numpy())
        ost[1].encode(v.float().numpy())
        t0 += n
    torch.cuda.synchronize()
    for kv in (0, 1):
        assert_stream_equal(codec, 0, kv, ost[kv])
        rec = codec.reconstruct(0, 1, kv, 0, t0)[0].cpu().numpy()
        np.testing.assert_array_equal(f32_bits(rec), f32_bits(ost[kv].xhat()))
