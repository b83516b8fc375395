"""GPU parity of the cross-layer residual mode (Coral-KV block-DPLR predictor).

Layer 0 is coded with SAS + PRQ; each layer l >= 1 is coded as the residual
against the prediction from the bf16 reconstruction of layer l-1.  Codes,
(sigma, z) and the fp32 reconstruction of every layer must be bit-exact
against the oracle chain.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import stream as o_stream
from oracle import xlayer as o_xlayer
from parity_util import assert_stream_equal, f32_bits, make_codec, oracle_stream

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _predictor_blob(cfgs, n_layers, rank):
    parts = []
    for l in range(n_layers - 1):
        for kv in (0, 1):
            B, U, V = synth.predictor(cfgs, l, kv, rank=rank)
            parts += [B.reshape(-1), U.reshape(-1), V.reshape(-1)]
    return torch.cat(parts)


@pytest.mark.parametrize("G,S,bits", [(64, 2, 2), (64, 1, 4), (32, 2, 2)])
def test_cross_layer_chain(G, S, bits):
    L, H, n, r, C = 3, 4, 300, 8, 16
    cfgs = synth.scaled(synth.WIDE_HEAD, n_layers=L, n_heads=H, tokens=n, n_clusters=C,
                        n_stages=S, bits=bits, group=G, xlayer_rank=r)
    blob = _predictor_blob(cfgs, L, r)
    codec = make_codec(H, 128, C, S, bits, G, max_tokens=n, max_chunks=1, n_layers=L, max_q=0,
                       xlayer=1, rank=r, predictor=blob.to(DEV))
    xs = {kv: torch.stack([synth.kv_tokens(cfgs, l, kv, 0, n) for l in range(L)]) for kv in (0, 1)}
    print(f"xlayer G={G} S={S} b={bits}: encode {L} layers", flush=True)
    codec.encode_chunk(xs[0].to(DEV), xs[1].to(DEV))
    torch.cuda.synchronize()
    for kv in (0, 1):
        rec = codec.reconstruct(0, L, kv, 0, n).cpu().numpy()
        o0 = oracle_stream(H, 128, C, 5, S, bits, G, "bf16")
        o0.encode(xs[kv][0].float().numpy())
        assert_stream_equal(codec, 0, kv, o0)
        np.testing.assert_array_equal(f32_bits(rec[0]), f32_bits(o0.xhat()))
        prev = o0.xhat()
        for l in range(1, L):
            B, U, V = synth.predictor(cfgs, l - 1, kv, rank=r)
            pred = o_xlayer.predict(prev, B.float().numpy(), U.float().numpy(), V.float().numpy())
            ol = oracle_stream(H, 128, C, 5, S, bits, G, "bf16")
            ol.encode_residual(xs[kv][l].float().numpy(), pred)
            assert_stream_equal(codec, l, kv, ol, check_ids=False)
            np.testing.assert_array_equal(f32_bits(rec[l]), f32_bits(ol.xhat()),
                                          err_msg=f"layer {l} kv {kv}")
            prev = ol.xhat()
        # a later window through the chain: layers 1..2 only, tokens [50, 250)
        part = codec.reconstruct(1, 2, kv, 50, 250).cpu().numpy()
        np.testing.assert_array_equal(f32_bits(part), f32_bits(rec[1:, :, 50:250]))


def _bf16_step(v):
    """Spacing of bf16 values around v (v a bf16 value, not zero)."""
    e = np.floor(np.log2(np.abs(v)))
    return 2.0 ** (e - 7)


def test_adapted_predictor_refit_and_chain():
    """Adapted mode: the blocks of layers 1 and 2 are re-fitted on the first
    call's tokens (600), then used for that call and the next (200).  The
    re-fitted bf16 blocks equal the oracle's (the fp64 solves differ only in
    rounding order: a block element may differ by one bf16 step only where
    the fp64 value sits on a rounding midpoint to 1e-8); given the device's
    blocks, codes and reconstructions of every layer are bit-exact."""
    L, H, r, C, S, bits, G = 3, 4, 8, 16, 2, 2, 64
    n1, n2 = 600, 200
    n = n1 + n2
    cfgs = synth.scaled(synth.WIDE_HEAD, n_layers=L, n_heads=H, tokens=n, n_clusters=C,
                        n_stages=S, bits=bits, group=G, xlayer_rank=r)
    blob = _predictor_blob(cfgs, L, r)
    codec = make_codec(H, 128, C, S, bits, G, max_tokens=n, max_chunks=2, n_layers=L, max_q=0,
                       xlayer=1, rank=r, predictor=blob.to(DEV), adapt=1)
    xs = {kv: torch.stack([synth.kv_tokens(cfgs, l, kv, 0, n) for l in range(L)]) for kv in (0, 1)}
    print(f"adapted xlayer: {L} layers, calls of {n1} and {n2} tokens", flush=True)
    codec.encode_chunk(xs[0][:, :, :n1].contiguous().to(DEV), xs[1][:, :, :n1].contiguous().to(DEV))
    codec.encode_chunk(xs[0][:, :, n1:].contiguous().to(DEV), xs[1][:, :, n1:].contiguous().to(DEV))
    torch.cuda.synchronize()
    blocks = {l: codec.adapted_blocks(l).float().cpu().numpy() for l in range(1, L)}
    for kv in (0, 1):
        rec = codec.reconstruct(0, L, kv, 0, n).cpu().numpy()
        o0 = oracle_stream(H, 128, C, 5, S, bits, G, "bf16")
        o0.encode(xs[kv][0, :, :n1].float().numpy())
        o0.encode(xs[kv][0, :, n1:].float().numpy())
        assert_stream_equal(codec, 0, kv, o0)
        prev = o0.xhat()
        for l in range(1, L):
            _, U, V = synth.predictor(cfgs, l - 1, kv, rank=r)
            U, V = U.float().numpy(), V.float().numpy()
            x_l = xs[kv][l].float().numpy()
            Bfit, Bb = o_xlayer.refit_block(prev[:, :n1], x_l[:, :n1], U, V)
            dev_b = blocks[l][kv]
            bad = np.argwhere(dev_b != Bb)
            assert len(bad) <= dev_b.size // 1000, f"layer {l} kv {kv}: {len(bad)} block elements differ"
            for h, i, j in bad:
                g, o, f = dev_b[h, i, j], Bb[h, i, j], Bfit[h, i, j]
                assert abs(g - o) == _bf16_step(max(abs(g), abs(o)))
                assert abs(f - (g + o) / 2) <= 1e-8 * abs(f)
            pred = o_xlayer.predict(prev, dev_b, U, V)
            ol = oracle_stream(H, 128, C, 5, S, bits, G, "bf16")
            ol.encode_residual(x_l[:, :n1], pred[:, :n1])
            ol.encode_residual(x_l[:, n1:], pred[:, n1:])
            assert_stream_equal(codec, l, kv, ol, check_ids=False)
            np.testing.assert_array_equal(f32_bits(rec[l]), f32_bits(ol.xhat()), err_msg=f"layer {l} kv {kv}")
            prev = ol.xhat()


@pytest.mark.parametrize("adapt", [0, 1])
def test_cross_layer_attend_sweep(adapt):
    """Attention over cross-layer coded layers, read in order 0, 1, 2 after
    the last encode call: each layer's keys are its chain reconstruction
    (held by the library as a rolling bf16 copy of one layer, in slices of
    the 300-token chunk size; 557 tokens = one full and one partial slice).
    Reference: the oracle's attention over the oracle chain's x-hat (with the
    device's re-fitted blocks in adapted mode).  Also: reading out of order
    and after an encode call are state errors; the read with a fresh chunk
    matches the oracle over the concatenated keys."""
    from oracle import attend as o_attend
    from parity_util import attention_tolerance_check, softmax_abs_mass
    import kv_cache_quantization_head_amd as qkv
    from kv_cache_quantization_head_amd import binding as Bd

    L, H, r, C, S, bits, G = 3, 4, 8, 16, 2, 2, 64
    n1, n2, n3, nq = 300, 257, 100, 200
    n = n1 + n2
    cfgs = synth.scaled(synth.WIDE_HEAD, n_layers=L, n_heads=H, tokens=n + n3, n_clusters=C,
                        n_stages=S, bits=bits, group=G, xlayer_rank=r)
    blob = _predictor_blob(cfgs, L, r)
    codec = make_codec(H, 128, C, S, bits, G, max_tokens=n + n3, max_chunks=3, max_chunk_tokens=n1,
                       n_layers=L, max_q=nq, xlayer=1, rank=r, predictor=blob.to(DEV), adapt=adapt)
    xs = {kv: torch.stack([synth.kv_tokens(cfgs, l, kv, 0, n + n3) for l in range(L)]) for kv in (0, 1)}
    print(f"xlayer read (adapt={adapt}): {L} layers, calls of {n1} and {n2} tokens", flush=True)
    codec.encode_chunk(xs[0][:, :, :n1].contiguous().to(DEV), xs[1][:, :, :n1].contiguous().to(DEV))
    codec.encode_chunk(xs[0][:, :, n1:n].contiguous().to(DEV), xs[1][:, :, n1:n].contiguous().to(DEV))
    torch.cuda.synchronize()
    # oracle chain x-hat of every layer (as the encode parity tests build it)
    xhat = {}
    for kv in (0, 1):
        o0 = oracle_stream(H, 128, C, 5, S, bits, G, "bf16")
        o0.encode(xs[kv][0, :, :n1].float().numpy())
        o0.encode(xs[kv][0, :, n1:n].float().numpy())
        xhat[(0, kv)] = o0.xhat()
        for l in range(1, L):
            B, U, V = synth.predictor(cfgs, l - 1, kv, rank=r)
            Bm = codec.adapted_blocks(l).float().cpu().numpy()[kv] if adapt else B.float().numpy()
            pred = o_xlayer.predict(xhat[(l - 1, kv)], Bm, U.float().numpy(), V.float().numpy())
            ol = oracle_stream(H, 128, C, 5, S, bits, G, "bf16")
            ol.encode_residual(xs[kv][l, :, :n1].float().numpy(), pred[:, :n1])
            ol.encode_residual(xs[kv][l, :, n1:n].float().numpy(), pred[:, n1:])
            xhat[(l, kv)] = ol.xhat()
    qs = [synth.queries(cfgs, l, nq) for l in range(L)]

    def check(l):
        out, lse = codec.attend(l, qs[l].to(DEV))
        o_ref, lse_ref = o_attend.attend(qs[l].float().numpy(), xhat[(l, 0)], xhat[(l, 1)])
        # the generator's x20 outlier channels: outputs that are cancelling
        # sums of large values (bf16 probabilities, see the bound's note)
        mass = softmax_abs_mass(qs[l].float().numpy(), xhat[(l, 0)], xhat[(l, 1)])
        err = attention_tolerance_check(out.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, mass=mass)
        print(f"  layer {l}: max abs err {err:.3e}", flush=True)

    check(0)
    with pytest.raises(qkv.QkvError) as e:     # layer 2 before layer 1
        codec.attend(2, qs[2].to(DEV))
    assert e.value.status == Bd.QKV_E_STATE
    check(1)
    check(2)
    # again from layer 0 (a second denoising step), with the fresh chunk on layer 1
    check(0)
    kn = xs[0][1, :, n:].contiguous()
    vn = xs[1][1, :, n:].contiguous()
    out, lse = codec.attend_with_chunk(1, qs[1].to(DEV), kn.to(DEV), vn.to(DEV))
    kcat = np.concatenate([xhat[(1, 0)], kn.float().numpy()], axis=1)
    vcat = np.concatenate([xhat[(1, 1)], vn.float().numpy()], axis=1)
    o_ref, lse_ref = o_attend.attend(qs[1].float().numpy(), kcat, vcat)
    attention_tolerance_check(out.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref,
                              mass=softmax_abs_mass(qs[1].float().numpy(), kcat, vcat))
    # an encode call empties the rolling copy: layer 1 needs layer 0 first
    codec.encode_chunk(xs[0][:, :, n:].contiguous().to(DEV), xs[1][:, :, n:].contiguous().to(DEV))
    with pytest.raises(qkv.QkvError) as e:
        codec.attend(1, qs[1].to(DEV))
    assert e.value.status == Bd.QKV_E_STATE
