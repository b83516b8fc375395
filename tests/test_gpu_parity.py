"""GPU parity: the HIP library, called through the C-ABI, against the oracle.

Bar: cluster ids, codebook snapshots, packed codes and (sigma, z) are
bit-exact; fp32 reconstruction is bit-exact (bf16 output = nearest-even
rounding of it); attention output within 2e-2 * max(1, |O_ref|) and the same
for LSE.  Inputs are the seeded synthetic caches of `synth`.
"""
import numpy as np
import pytest
import torch

import synth
from parity_util import (assert_stream_equal, attention_tolerance_check, bf16_of, f32_bits,
                         make_codec, o_attend, oracle_stream)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _encode_and_oracle(cfgs, n_list, dtype, heads=None, layer=0, codec=None, max_q=256):
    """Encode chunks of the seeded stream; returns codec, (oracle K, oracle V), inputs."""
    H, d = cfgs.n_heads, cfgs.head_dim
    total = sum(n_list)
    if codec is None:
        codec = make_codec(H, d, cfgs.n_clusters, cfgs.n_stages, cfgs.bits, cfgs.group, iters=cfgs.iters,
                           max_tokens=total, max_chunks=len(n_list), dtype=dtype, max_q=max_q)
    hs = list(range(H)) if heads is None else heads
    ost = [oracle_stream(len(hs), d, cfgs.n_clusters, cfgs.iters, cfgs.n_stages, cfgs.bits, cfgs.group,
                         dtype) for _ in range(2)]
    xs = [[], []]
    t0 = 0
    for n in n_list:
        k = synth.kv_tokens(cfgs, layer, 0, t0, n)
        v = synth.kv_tokens(cfgs, layer, 1, t0, n)
        codec.encode_chunk(k.to(DEV), v.to(DEV))
        for kv, x in ((0, k), (1, v)):
            xn = x.float().numpy()[hs]
            ost[kv].encode(xn)
            xs[kv].append(xn)
        t0 += n
    torch.cuda.synchronize()
    return codec, ost, [np.concatenate(x, axis=1) for x in xs]


def test_tiny_full():
    cfgs = synth.TINY
    _say("tiny: encode 2x4096 fp32")
    codec, ost, _ = _encode_and_oracle(cfgs, [4096], "f32")
    for kv in (0, 1):
        assert_stream_equal(codec, 0, kv, ost[kv])
        rec = codec.reconstruct(0, 1, kv, 0, 4096)[0].cpu().numpy()
        np.testing.assert_array_equal(f32_bits(rec), f32_bits(ost[kv].xhat()))
        recb = codec.reconstruct(0, 1, kv, 0, 4096, out_dtype=torch.bfloat16)[0].float().cpu().numpy()
        np.testing.assert_array_equal(f32_bits(recb), f32_bits(bf16_of(ost[kv].xhat())))
    q = synth.queries(cfgs, 0, 256)
    out, lse = codec.attend(0, q.to(DEV))
    o_ref, lse_ref = o_attend.attend(q.numpy(), ost[0].xhat(), ost[1].xhat())
    err = attention_tolerance_check(out.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref)
    _say(f"tiny attention max abs err {err:.3e}")


EDGE = [
    # name, overrides, chunk sizes, dtype
    ("T_below_C_bf16", dict(n_heads=2, head_dim=128, n_clusters=256, group=32, tokens=100), [100], "bf16"),
    ("int4_g64_ragged", dict(n_heads=3, head_dim=128, n_clusters=7, n_stages=1, bits=4, group=64,
                             tokens=1000), [1000], "bf16"),
    ("single_cluster_3stage_f32", dict(n_heads=2, head_dim=128, n_clusters=1, n_stages=3, group=32,
                                       tokens=333), [333], "f32"),
    ("u16_ids_4stage_d64", dict(n_heads=2, head_dim=64, n_clusters=300, n_stages=4, group=32,
                                tokens=777), [777], "bf16"),
    ("three_chunks_warm", dict(n_heads=2, head_dim=128, n_clusters=32, group=32, tokens=1531),
     [1000, 530, 1], "bf16"),
    ("no_iterations", dict(n_heads=2, head_dim=64, n_clusters=16, iters=0, group=64, tokens=500),
     [500], "f32"),
]


@pytest.mark.parametrize("name,over,chunks,dtype", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(name, over, chunks, dtype):
    base = synth.WAN_LAYER if dtype == "bf16" else synth.scaled(synth.TINY, per_token_labels=False,
                                                                 drift=0.02)
    cfgs = synth.scaled(base, **over)
    _say(f"edge {name}: chunks {chunks}")
    codec, ost, _ = _encode_and_oracle(cfgs, chunks, dtype, max_q=300)
    total = sum(chunks)
    assert codec.chunk_starts(0) == list(np.cumsum([0] + chunks[:-1]))
    for kv in (0, 1):
        assert_stream_equal(codec, 0, kv, ost[kv])
        # a ragged window across chunk boundaries
        t0, t1 = (total // 3, total - 1) if total > 3 else (0, total)
        rec = codec.reconstruct(0, 1, kv, t0, t1)[0].cpu().numpy()
        np.testing.assert_array_equal(f32_bits(rec), f32_bits(ost[kv].xhat()[:, t0:t1]))
    q = synth.queries(synth.scaled(cfgs, q_dtype=dtype), 0, 77)
    out, lse = codec.attend(0, q.to(DEV), out_dtype=torch.bfloat16)
    o_ref, lse_ref = o_attend.attend(q.float().numpy(), ost[0].xhat(), ost[1].xhat())
    attention_tolerance_check(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref)


def test_rewind_and_reencode():
    cfgs = synth.scaled(synth.WAN_LAYER, n_heads=2, n_clusters=16, tokens=3000)
    codec = make_codec(2, 128, 16, 2, 2, 32, max_tokens=3000, max_chunks=4)
    k = synth.kv_tokens(cfgs, 0, 0, 0, 3000)
    v = synth.kv_tokens(cfgs, 0, 1, 0, 3000)
    codec.encode_chunk(k[:, :1000].to(DEV), v[:, :1000].to(DEV))
    codec.encode_chunk(k[:, 1000:2000].to(DEV), v[:, 1000:2000].to(DEV))
    codec.rewind(0, 1, 1000)
    assert codec.chunk_starts(0) == [0]
    codec.encode_chunk(k[:, 1000:2700].to(DEV), v[:, 1000:2700].to(DEV))
    torch.cuda.synchronize()
    for kv, x in ((0, k), (1, v)):
        o = oracle_stream(2, 128, 16, 5, 2, 2, 32, "bf16")
        o.encode(x[:, :1000].float().numpy())
        o.encode(x[:, 1000:2700].float().numpy())
        assert_stream_equal(codec, 0, kv, o)


def test_multi_layer_call_matches_per_layer_oracle():
    cfgs = synth.scaled(synth.WHOLE_CACHE, n_layers=3, n_heads=2, n_clusters=32, tokens=1200)
    codec = make_codec(2, 128, 32, 2, 2, 32, max_tokens=1200, max_chunks=2, n_layers=3)
    ks = torch.stack([synth.kv_tokens(cfgs, l, 0, 0, 700) for l in range(3)])
    vs = torch.stack([synth.kv_tokens(cfgs, l, 1, 0, 700) for l in range(3)])
    codec.encode_chunk(ks.to(DEV), vs.to(DEV))              # one call, three layers
    ks2 = torch.stack([synth.kv_tokens(cfgs, l, 0, 700, 500) for l in range(3)])
    vs2 = torch.stack([synth.kv_tokens(cfgs, l, 1, 700, 500) for l in range(3)])
    codec.encode_chunk(ks2.to(DEV), vs2.to(DEV))
    torch.cuda.synchronize()
    rec = codec.reconstruct(0, 3, 1, 0, 1200).cpu().numpy()
    for l in range(3):
        for kv, (a, b) in ((0, (ks, ks2)), (1, (vs, vs2))):
            o = oracle_stream(2, 128, 32, 5, 2, 2, 32, "bf16")
            o.encode(a[l].float().numpy())
            o.encode(b[l].float().numpy())
            assert_stream_equal(codec, l, kv, o)
            if kv == 1:
                np.testing.assert_array_equal(f32_bits(rec[l]), f32_bits(o.xhat()))


def test_wan_layer_full_size_sampled_heads():
    """Full Wan-layer shape (12 heads x 32760 tokens, C=256); the oracle runs heads 0 and 7."""
    cfgs = synth.WAN_LAYER
    heads = [0, 7]
    _say("wan layer: encode 12x32760x128 bf16 (K and V)")
    codec, ost, _ = _encode_and_oracle(cfgs, [32760], "bf16", heads=heads, max_q=4680)
    for kv in (0, 1):
        assert_stream_equal(codec, 0, kv, ost[kv], heads=heads)
        for oi, h in enumerate(heads):
            rec = codec.reconstruct(0, 1, kv, 0, 32760)[0, h].cpu().numpy()
            np.testing.assert_array_equal(f32_bits(rec), f32_bits(ost[kv].xhat()[oi]))
    q = synth.queries(cfgs, 0, 4680)
    out, lse = codec.attend(0, q.to(DEV))
    sample = np.arange(0, 4680, 73)
    o_ref, lse_ref = o_attend.attend(q.float().numpy()[heads][:, sample], ost[0].xhat(), ost[1].xhat())
    err = attention_tolerance_check(out.cpu().numpy()[heads][:, sample], lse.cpu().numpy()[heads][:, sample],
                                    o_ref, lse_ref)
    _say(f"wan layer attention (sampled) max abs err {err:.3e}")
    # the same read with the next 4680-token chunk still in bf16
    kn = synth.kv_tokens(cfgs, 0, 0, 32760, 4680)
    vn = synth.kv_tokens(cfgs, 0, 1, 32760, 4680)
    out, lse = codec.attend_with_chunk(0, q.to(DEV), kn.to(DEV), vn.to(DEV))
    khat = np.concatenate([ost[0].xhat(), kn.float().numpy()[heads]], axis=1)
    vhat = np.concatenate([ost[1].xhat(), vn.float().numpy()[heads]], axis=1)
    o_ref, lse_ref = o_attend.attend(q.float().numpy()[heads][:, sample], khat, vhat)
    err = attention_tolerance_check(out.cpu().numpy()[heads][:, sample], lse.cpu().numpy()[heads][:, sample],
                                    o_ref, lse_ref)
    _say(f"wan layer attention with a fresh 4680-token chunk (sampled) max abs err {err:.3e}")


def test_encode_is_deterministic():
    cfgs = synth.scaled(synth.WAN_LAYER, n_heads=4, tokens=6000)
    arenas = []
    for _ in range(2):
        codec = make_codec(4, 128, 256, 2, 2, 32, max_tokens=6000, max_chunks=1, max_q=0)
        codec.arena.zero_()      # bytes the encoder never writes must not differ either
        k = synth.kv_tokens(cfgs, 0, 0, 0, 6000).to(DEV)
        v = synth.kv_tokens(cfgs, 0, 1, 0, 6000).to(DEV)
        codec.encode_chunk(k, v)
        torch.cuda.synchronize()
        arenas.append(codec.arena.cpu())
    assert torch.equal(arenas[0], arenas[1])


def test_attend_is_deterministic():
    # the split partials are merged in a fixed order and every key tile is
    # walked in one order: repeated reads of one cache give the same bytes,
    # with the query blocks split across blocks (1000 queries over 6000 keys
    # of 4 heads) and without
    cfgs = synth.scaled(synth.WAN_LAYER, n_heads=4, tokens=6000)
    codec = make_codec(4, 128, 256, 2, 2, 32, max_tokens=6000, max_chunks=1, max_q=1000)
    codec.encode_chunk(synth.kv_tokens(cfgs, 0, 0, 0, 6000).to(DEV), synth.kv_tokens(cfgs, 0, 1, 0, 6000).to(DEV))
    for n_q in (1000, 64):
        q = synth.queries(cfgs, 0, n_q).to(DEV)
        runs = [codec.attend(0, q) for _ in range(3)]
        torch.cuda.synchronize()
        for out, lse in runs[1:]:
            assert torch.equal(out, runs[0][0]) and torch.equal(lse, runs[0][1])


def _near_tie_tokens(H, T, d, seed):
    """bf16-exact tokens built so that most are near-ties for the nearest
    centroid.  With no k-means iteration the codebook is the strided initial
    one, rows floor(k T / 8) = +v, -v, +w, -w, 4v, -4v, 4w, -4w (v all ones,
    w alternating +-1).  Other tokens: 80 % gamma (v + w) + delta (+v and +w
    within a few 2^-8 of each other, the rest far: two-way near-ties), 10 %
    delta alone (four-way near-ties; delta = 0 gives exact ties), 10 % random
    normal rounded to bf16 (decided by the screen).  delta puts +-2^-8 on
    eight random channels."""
    rng = np.random.default_rng(seed)
    v = np.ones(d, np.float32)
    w = np.where(np.arange(d) % 2 == 0, 1.0, -1.0).astype(np.float32)
    cents = np.stack([v, -v, w, -w, 4 * v, -4 * v, 4 * w, -4 * w])
    x = np.zeros((H, T, d), np.float32)
    for h in range(H):
        kind = rng.random(T)
        delta = np.zeros((T, d), np.float32)
        ch = rng.integers(0, d, size=(T, 8))
        sg = rng.choice(np.array([-1.0, 0.0, 1.0], np.float32), size=(T, 8)) * 2.0 ** -8
        np.put_along_axis(delta, ch, sg, axis=1)
        pair = 2.0 ** -5 * (v + w)[None, :] + delta
        far = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).bfloat16().float().numpy()
        x[h] = np.where((kind < 0.8)[:, None], pair, np.where((kind < 0.9)[:, None], delta, far))
        x[h, (np.arange(8) * T) // 8] = cents
    xb = torch.from_numpy(x).bfloat16()
    assert torch.equal(xb.float(), torch.from_numpy(x))          # every value is bf16-exact
    return xb


def test_near_ties_pair_list_and_full_rescoring():
    """Near-tie tokens in bulk: most tokens need the exact fp64 decision
    between their two best centroids, some between four, some are exact ties
    (lowest index wins).  96 227 tokens per head make each block of the
    screening kernel take three 256-token tiles, so its pair list (512
    entries) overflows and the overflow goes to the full rescoring."""
    H, d, T, C = 2, 128, 3 * 32768 - 77, 8
    k = _near_tie_tokens(H, T, d, 11)
    v = _near_tie_tokens(H, T, d, 12)
    codec = make_codec(H, d, C, 2, 2, 32, iters=0, max_tokens=T, max_chunks=1, max_q=0)
    _say(f"near ties: {H} heads x {T} tokens, C={C}, no iterations")
    codec.encode_chunk(k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    for kv, x in ((0, k), (1, v)):
        o = oracle_stream(H, d, C, 0, 2, 2, 32, "bf16")
        o.encode(x.float().numpy())
        ids = o.chunks[0][0].ids
        assert np.count_nonzero(ids == 0) > T // 20 and np.count_nonzero(ids == 2) > T // 20
        assert_stream_equal(codec, 0, kv, o)


@pytest.mark.parametrize("n_new,out_dtype", [(4680, torch.float32), (77, torch.bfloat16), (1, torch.float32)],
                         ids=["chunk4680_f32", "ragged77_bf16", "one_token_f32"])
def test_attend_with_fresh_chunk(n_new, out_dtype):
    """Attention over the packed cache followed by a fresh bf16 chunk equals
    the oracle's attention over the concatenated keys (cache rebuilt by the
    oracle, fresh rows as given), within the attention tolerance."""
    cfgs = synth.scaled(synth.WAN_LAYER, n_heads=2, tokens=3000 + n_new)
    _say(f"fresh chunk: cache 3000 + fresh {n_new}, out {out_dtype}")
    codec, ost, _ = _encode_and_oracle(cfgs, [3000], "bf16", max_q=512)
    kn = synth.kv_tokens(cfgs, 0, 0, 3000, n_new)
    vn = synth.kv_tokens(cfgs, 0, 1, 3000, n_new)
    q = synth.queries(cfgs, 0, 300)
    out, lse = codec.attend_with_chunk(0, q.to(DEV), kn.to(DEV), vn.to(DEV), out_dtype=out_dtype)
    khat = np.concatenate([ost[0].xhat(), kn.float().numpy()], axis=1)
    vhat = np.concatenate([ost[1].xhat(), vn.float().numpy()], axis=1)
    o_ref, lse_ref = o_attend.attend(q.float().numpy(), khat, vhat)
    err = attention_tolerance_check(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref)
    _say(f"fresh chunk {n_new}: max abs err {err:.3e}")


def test_attend_with_fresh_chunk_edges():
    """No fresh tokens: the same bytes as qkv_attend.  Empty cache: attention
    over the fresh tokens alone, against the oracle."""
    cfgs = synth.scaled(synth.WAN_LAYER, n_heads=2, tokens=2000)
    codec, ost, _ = _encode_and_oracle(cfgs, [1500], "bf16", max_q=512)
    q = synth.queries(cfgs, 0, 257).to(DEV)
    empty = torch.empty((2, 0, 128), dtype=torch.bfloat16, device=DEV)
    o1, l1 = codec.attend(0, q)
    o2, l2 = codec.attend_with_chunk(0, q, empty, empty)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    fresh = make_codec(2, 128, 256, 2, 2, 32, max_tokens=2000, max_chunks=1, max_q=512)
    kn = synth.kv_tokens(cfgs, 0, 0, 0, 500)
    vn = synth.kv_tokens(cfgs, 0, 1, 0, 500)
    out, lse = fresh.attend_with_chunk(0, q, kn.to(DEV), vn.to(DEV))
    o_ref, lse_ref = o_attend.attend(q.float().cpu().numpy(), kn.float().numpy(), vn.float().numpy())
    attention_tolerance_check(out.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_codebook_reuse_matches_oracle(dtype):
    """Codebook reuse: the first call runs the k-means, later calls only
    assign their tokens to its codebook (one snapshot per stream); after a
    rewind to 0 the next call runs the k-means again."""
    base = synth.WAN_LAYER if dtype == "bf16" else synth.scaled(synth.TINY, per_token_labels=False, drift=0.02)
    cfgs = synth.scaled(base, n_heads=2, head_dim=128, n_clusters=64, group=32, tokens=4000)
    n_list = [1560, 1560, 880]
    S, b, it = cfgs.n_stages, cfgs.bits, cfgs.iters
    codec = make_codec(2, 128, 64, S, b, 32, iters=it, max_tokens=4000, max_chunks=3, dtype=dtype, max_q=256,
                       reuse=1)
    ost = [oracle_stream(2, 128, 64, it, S, b, 32, dtype, reuse=True) for _ in range(2)]
    t0 = 0
    _say(f"codebook reuse {dtype}: chunks {n_list}")
    for n in n_list:
        k = synth.kv_tokens(cfgs, 0, 0, t0, n)
        v = synth.kv_tokens(cfgs, 0, 1, t0, n)
        codec.encode_chunk(k.to(DEV), v.to(DEV))
        ost[0].encode(k.float().numpy())
        ost[1].encode(v.float().numpy())
        t0 += n
    torch.cuda.synchronize()
    for kv in (0, 1):
        assert_stream_equal(codec, 0, kv, ost[kv])
        rec = codec.reconstruct(0, 1, kv, 0, t0)[0].cpu().numpy()
        np.testing.assert_array_equal(f32_bits(rec), f32_bits(ost[kv].xhat()))
    q = synth.queries(synth.scaled(cfgs, q_dtype=dtype), 0, 256)
    out, lse = codec.attend(0, q.to(DEV))
    o_ref, lse_ref = o_attend.attend(q.float().numpy(), ost[0].xhat(), ost[1].xhat())
    attention_tolerance_check(out.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref)
    # rewind to 0: the next call clusters afresh
    codec.rewind(0, 1, 0)
    k = synth.kv_tokens(cfgs, 0, 0, 1560, 1560)
    v = synth.kv_tokens(cfgs, 0, 1, 1560, 1560)
    codec.encode_chunk(k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    for kv, x in ((0, k), (1, v)):
        o = oracle_stream(2, 128, 64, it, S, b, 32, dtype, reuse=True)
        o.encode(x.float().numpy())
        assert_stream_equal(codec, 0, kv, o)


def test_attend_with_fresh_chunk_d64_fp32_queries():
    """The fresh-chunk read at d = 64 with fp32 queries, a 3-chunk cache
    (several codebook snapshots) and a ragged fresh chunk."""
    cfgs = synth.scaled(synth.WAN_LAYER, n_heads=3, head_dim=64, n_clusters=32, group=32, tokens=2600,
                        q_dtype="f32")
    codec, ost, _ = _encode_and_oracle(cfgs, [700, 900, 400], "bf16", max_q=300)
    kn = synth.kv_tokens(cfgs, 0, 0, 2000, 333)
    vn = synth.kv_tokens(cfgs, 0, 1, 2000, 333)
    q = synth.queries(cfgs, 0, 199)
    assert q.dtype == torch.float32
    out, lse = codec.attend_with_chunk(0, q.to(DEV), kn.to(DEV), vn.to(DEV), out_dtype=torch.bfloat16)
    khat = np.concatenate([ost[0].xhat(), kn.float().numpy()], axis=1)
    vhat = np.concatenate([ost[1].xhat(), vn.float().numpy()], axis=1)
    o_ref, lse_ref = o_attend.attend(q.numpy(), khat, vhat)
    attention_tolerance_check(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref)


@pytest.mark.parametrize("index,dtype", [(101, "bf16"), (102, "bf16"), (103, "f32")])
def test_other_seeds_bit_exact(index, dtype):
    """The bit-exact bar on data drawn from other seeds (a wan_layer-shaped
    stream with 2 heads, two warm-started calls; one fp32 cache that takes
    the non-MFMA assignment)."""
    base = synth.WAN_LAYER if dtype == "bf16" else synth.scaled(synth.TINY, per_token_labels=False, drift=0.02)
    cfgs = synth.scaled(base, index=index, n_heads=2, head_dim=128, n_clusters=256, group=32, tokens=8000)
    _say(f"seed index {index} ({dtype}): 2 heads x (5000 + 3000) tokens")
    codec, ost, _ = _encode_and_oracle(cfgs, [5000, 3000], dtype, max_q=128)
    for kv in (0, 1):
        assert_stream_equal(codec, 0, kv, ost[kv])
        rec = codec.reconstruct(0, 1, kv, 0, 8000)[0].cpu().numpy()
        np.testing.assert_array_equal(f32_bits(rec), f32_bits(ost[kv].xhat()))
    q = synth.queries(synth.scaled(cfgs, q_dtype=dtype), 0, 128)
    out, lse = codec.attend(0, q.to(DEV))
    o_ref, lse_ref = o_attend.attend(q.float().numpy(), ost[0].xhat(), ost[1].xhat())
    attention_tolerance_check(out.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref)
