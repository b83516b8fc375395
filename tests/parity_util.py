"""Helpers shared by the GPU parity tests: run the oracle on the same seeded
inputs and compare the library's arena contents and outputs with it."""
import numpy as np
import torch

from oracle import attend as o_attend
from oracle import numerics
from oracle import stream as o_stream
from oracle import xlayer as o_xlayer

import kv_cache_quantization_head_amd as qkv


def make_codec(H, d, C, S, bits, G, iters=5, max_tokens=4096, max_chunks=4, dtype="bf16",
               max_q=256, n_layers=1, max_chunk_tokens=0, xlayer=0, rank=0, predictor=None, reuse=0,
               adapt=0, outliers=0):
    cfg = qkv.config(n_layers, H, d, C, S, bits, G, kmeans_iters=iters, max_tokens=max_tokens,
                     max_chunk_tokens=max_chunk_tokens, max_chunks=max_chunks,
                     kv_dtype=qkv.QKV_BF16 if dtype == "bf16" else qkv.QKV_F32,
                     max_query_tokens=max_q, xlayer=xlayer, xlayer_rank=rank, codebook_reuse=reuse,
                     xlayer_adapt=adapt, outlier_channels=outliers)
    return qkv.Codec(cfg, device="cuda", predictor=predictor)


def oracle_stream(H, d, C, iters, S, bits, G, dtype, reuse=False, outliers=False):
    return o_stream.Stream(H, d, C, iters, S, bits, G, dtype, reuse=reuse, outliers=outliers)


def f32_bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def assert_stream_equal(codec, layer, kv, ostream, heads=None, check_ids=True):
    """Bit-exact comparison of ids, snapshots, codes and (sigma, z) for the given heads.

    ostream holds heads in the order of `heads` (all heads when None).
    """
    cfg = codec.cfg
    heads = list(range(cfg.n_heads)) if heads is None else list(heads)
    S = cfg.n_stages
    for oi, h in enumerate(heads):
        if check_ids:
            ids = codec.ids(layer, kv)[h].cpu().numpy().astype(np.int64) & 0xFFFF
            ref_ids = np.concatenate([ch[oi].ids for ch in ostream.chunks])
            bad = np.count_nonzero(ids != ref_ids)
            assert bad == 0, f"layer {layer} kv {kv} head {h}: {bad} ids differ"
            for c, ch in enumerate(ostream.chunks):
                cb = codec.codebook(layer, kv, c)[h].float().cpu().numpy()
                np.testing.assert_array_equal(f32_bits(cb), f32_bits(ch[oi].codebook),
                                              err_msg=f"codebook chunk {c} head {h}")
        for s in range(S):
            codes = codec.codes(layer, kv, s)[h].cpu().numpy()
            ref = np.concatenate([ch[oi].packed[s] for ch in ostream.chunks])
            nbad = np.count_nonzero(codes != ref)
            assert nbad == 0, f"layer {layer} kv {kv} head {h} stage {s}: {nbad} code bytes differ"
            meta = codec.meta(layer, kv, s)[h].cpu().numpy().view(np.uint16)
            ref_s = np.concatenate([ch[oi].sigmas[s] for ch in ostream.chunks]).view(np.uint16)
            ref_z = np.concatenate([ch[oi].zs[s] for ch in ostream.chunks]).view(np.uint16)
            np.testing.assert_array_equal(meta[..., 0], ref_s, err_msg=f"sigma stage {s} head {h}")
            np.testing.assert_array_equal(meta[..., 1], ref_z, err_msg=f"z stage {s} head {h}")


def oracle_xhat(ostream):
    return ostream.xhat()


def softmax_abs_mass(q, khat, vhat):
    """sum_k p_k |v_kj| per (head, query, channel), p the exact softmax of the
    bf16 operands' logits (fp64): the scale of the terms whose sum is O."""
    qb = bf16_of(q).astype(np.float64)
    kb = bf16_of(khat).astype(np.float64)
    vb = np.abs(bf16_of(vhat).astype(np.float64))
    out = np.empty(qb.shape)
    for h in range(qb.shape[0]):
        s = qb[h] @ kb[h].T / np.sqrt(qb.shape[2])
        p = np.exp(s - s.max(axis=1, keepdims=True))
        out[h] = (p / p.sum(axis=1, keepdims=True)) @ vb[h]
    return out


def attention_tolerance_check(out, lse, o_ref, lse_ref, tol=2e-2, mass=None):
    """|O - O_ref| <= tol * max(1, |O_ref|) elementwise; the same for LSE.

    With ``mass`` (``softmax_abs_mass``), 2^-7 * mass is added to the bound:
    the probabilities enter the PV product in bf16 (relative rounding 2^-9
    each, and the row sum carries the same), so an output that is a
    cancelling sum of large values is off by up to 2^-8 * sum_k p_k |v_k|
    however small |O| is."""
    out = np.asarray(out, dtype=np.float64)
    err = np.abs(out - o_ref)
    bound = tol * np.maximum(1.0, np.abs(o_ref))
    if mass is not None:
        bound = bound + 2.0 ** -7 * mass
    worst = float((err / bound).max())
    assert np.all(err <= bound), f"attention error {worst:.3f} of the bound (max abs {err.max():.3e})"
    if lse is not None:
        lerr = np.abs(np.asarray(lse, np.float64) - lse_ref)
        assert np.all(lerr <= tol * np.maximum(1.0, np.abs(lse_ref))), lerr.max()
    return float(err.max())


def bf16_of(x):
    return numerics.round_to_bf16(x)


__all__ = ["make_codec", "oracle_stream", "assert_stream_equal", "attention_tolerance_check", "softmax_abs_mass",
           "o_attend", "o_xlayer", "bf16_of", "f32_bits"]
