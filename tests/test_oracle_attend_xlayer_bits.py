"""Pins for the oracle's attention read, cross-layer predictor and storage cost (CPU only)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import attend, bits, numerics, prq, stream, xlayer
import synth


def test_attend_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((3, 40, 64)).astype(np.float32)
    k = rng.standard_normal((3, 333, 64)).astype(np.float32) * 2
    v = rng.standard_normal((3, 333, 64)).astype(np.float32)
    o, lse = attend.attend(q, k, v)
    qb = torch.from_numpy(numerics.round_to_bf16(q)).double()
    kb = torch.from_numpy(numerics.round_to_bf16(k)).double()
    vb = torch.from_numpy(numerics.round_to_bf16(v)).double()
    ref = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    logits = (qb @ kb.transpose(-1, -2)) / 8.0
    np.testing.assert_allclose(lse, torch.logsumexp(logits, -1).numpy(), rtol=1e-13)


def test_attend_equal_keys_gives_mean_value():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((2, 5, 32)).astype(np.float32)
    k = np.broadcast_to(rng.standard_normal((2, 1, 32)), (2, 77, 32)).astype(np.float32)
    v = numerics.round_to_bf16(rng.standard_normal((2, 77, 32)))
    o, lse = attend.attend(q, k, v)
    np.testing.assert_allclose(o, np.broadcast_to(v.astype(np.float64).mean(axis=1, keepdims=True),
                                                  o.shape), rtol=1e-12, atol=1e-13)
    logit = (numerics.round_to_bf16(q).astype(np.float64) @ numerics.round_to_bf16(k[:, :1]).astype(
        np.float64).transpose(0, 2, 1))[..., 0] / np.sqrt(32)
    np.testing.assert_allclose(lse, logit + np.log(77), rtol=1e-12)


def test_attend_split_merge_identity():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 9, 64)).astype(np.float32)
    k = rng.standard_normal((2, 100, 64)).astype(np.float32) * 3
    v = rng.standard_normal((2, 100, 64)).astype(np.float32)
    o, lse = attend.attend(q, k, v)
    o1, l1 = attend.attend(q, k[:, :37], v[:, :37])
    o2, l2 = attend.attend(q, k[:, 37:], v[:, 37:])
    om, lm = attend.merge(o1, l1, o2, l2)
    np.testing.assert_allclose(om, o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lm, lse, rtol=1e-13)


def test_xlayer_zero_predictor_is_plain_prq():
    cfg = synth.scaled(synth.WIDE_HEAD, n_heads=3, tokens=200, xlayer_rank=4)
    x0 = synth.kv_tokens(cfg, 0, 0, 0, 200).float().numpy()
    x1 = synth.kv_tokens(cfg, 1, 0, 0, 200).float().numpy()
    H, d, r = 3, 128, 4
    pred = xlayer.predict(x0, np.zeros((H, d, d)), np.zeros((H * d, r)), np.zeros((H * d, r)))
    assert np.all(pred == 0)
    r0 = xlayer.residual(x1, pred)
    np.testing.assert_array_equal(r0, x1)
    ch = stream.encode_residual_head(x1[0], pred[0], 2, 2, 64)
    codes, *_ = prq.quantize(x1[0], 2, 2, 64)
    np.testing.assert_array_equal(ch.packed[0], prq.pack(codes[0], 2))


def test_xlayer_identity_predictor_zero_residual():
    cfg = synth.scaled(synth.WIDE_HEAD, n_heads=2, tokens=64)
    x = synth.kv_tokens(cfg, 0, 1, 0, 64).float().numpy()          # bf16 values
    H, d, r = 2, 128, 8
    B = np.broadcast_to(np.eye(d), (H, d, d))
    rng = np.random.default_rng(4)
    V = numerics.round_to_bf16(rng.standard_normal((H * d, r)) * 0.1)
    pred = xlayer.predict(x, B, np.zeros((H * d, r)), V)
    np.testing.assert_array_equal(pred, x)
    assert np.all(xlayer.residual(x, pred) == 0)


def test_xlayer_matches_dense_matrix_form():
    # block-diagonal + low-rank equals the dense (H*d x H*d) matrix it stands for,
    # up to fp64 rounding and the bf16 rounding of the rank-r projection
    rng = np.random.default_rng(5)
    H, d, r, T = 3, 16, 4, 50
    xh = numerics.round_to_bf16(rng.standard_normal((H, T, d)))
    B = numerics.round_to_bf16(rng.standard_normal((H, d, d)) / 4)
    U = numerics.round_to_bf16(rng.standard_normal((H * d, r)) / 4)
    V = numerics.round_to_bf16(rng.standard_normal((H * d, r)) / 4)
    pred = xlayer.predict(xh, B, U, V)
    y = np.transpose(xh, (1, 0, 2)).reshape(T, H * d).astype(np.float64)
    Wbd = np.zeros((H * d, H * d))
    for h in range(H):
        Wbd[h * d:(h + 1) * d, h * d:(h + 1) * d] = B[h]
    w = numerics.round_to_bf16(y @ V.astype(np.float64)).astype(np.float64)
    dense = y @ Wbd.T + w @ U.astype(np.float64).T
    ref = np.transpose(dense.reshape(T, H, d), (1, 0, 2)).astype(np.float32)
    np.testing.assert_array_equal(pred, ref)   # fp64 sums of exact products: no rounding here


@pytest.mark.parametrize("name,S,b,G,d,C,cbb,n,expect", [
    ("tiny", 2, 2, 64, 64, 16, 4, 4096, Fraction(21, 4)),
    ("wan_layer", 2, 2, 32, 128, 256, 2, 32760, None),
    ("whole_cache_chunk", 2, 2, 32, 128, 256, 2, 4680, None),
    ("long_rollout", 3, 2, 32, 128, 256, 2, 4680, None),
    ("wide_int2", 2, 2, 64, 128, 512, 2, 62400, None),
    ("wide_int4", 1, 4, 64, 128, 512, 2, 62400, None),
])
def test_bits_per_element_closed_form(name, S, b, G, d, C, cbb, n, expect):
    got = bits.bits_per_element(S, b, G, d, C, cbb, n)
    if expect is not None:
        assert got == expect
    # count the bytes the oracle actually stores for one head of one call
    id_bytes = 1 if C <= 256 else 2
    stored_bits = 8 * (S * n * d * b // 8 + S * n * (d // G) * 4 + n * id_bytes + C * d * cbb)
    assert Fraction(stored_bits, n * d) == got
    table = {"tiny": 5.25, "wan_layer": 6.19, "whole_cache_chunk": 6.94, "long_rollout": 9.94,
             "wide_int2": 5.26, "wide_int4": 4.76}
    assert round(float(got), 2) == table[name]


def test_stored_sizes_match_closed_form_on_encoded_head():
    cfg = synth.scaled(synth.TINY, tokens=1024)
    x = synth.kv_tokens(cfg, 0, 0, 0, 1024)[0].numpy()
    ch = stream.encode_head(x, 16, 2, 2, 2, 64, "f32")
    nbytes = sum(p.nbytes for p in ch.packed) + sum(s.nbytes + z.nbytes for s, z in zip(ch.sigmas, ch.zs)) \
        + 1024 * 1 + ch.codebook.astype(np.float32).nbytes
    assert Fraction(8 * nbytes, 1024 * 64) == bits.bits_per_element(2, 2, 64, 64, 16, 4, 1024)


def test_refit_recovers_an_exact_block_predictor():
    """Adapted mode: when x_{l+1} is exactly B_true y + U w (computed in fp64
    from bf16 factors), the least-squares re-fit returns B_true up to the tiny
    ridge bias, and its bf16 rounding is B_true itself."""
    rng = np.random.default_rng(5)
    H, T, d, r = 2, 600, 16, 3
    xprev = rng.standard_normal((H, T, d)).astype(np.float32)
    Btrue = numerics.round_to_bf16(0.3 * rng.standard_normal((H, d, d)))
    U = numerics.round_to_bf16(0.2 * rng.standard_normal((H * d, r)))
    V = numerics.round_to_bf16(0.2 * rng.standard_normal((H * d, r)))
    y = numerics.round_to_bf16(xprev).astype(np.float64)
    w = numerics.round_to_bf16(np.transpose(y, (1, 0, 2)).reshape(T, H * d) @ V.astype(np.float64))
    lowrank = (w @ U.astype(np.float64).T).reshape(T, H, d).transpose(1, 0, 2)
    xnext = np.einsum("hij,htj->hti", Btrue.astype(np.float64), y) + lowrank
    B, Bb = xlayer.refit_block(xprev, xnext, U, V)
    np.testing.assert_allclose(B, Btrue, rtol=0, atol=1e-4)
    np.testing.assert_array_equal(Bb, Btrue)


def test_refit_without_low_rank_is_ridge_least_squares():
    """With U = 0 the re-fit is the ridge solution of min |Y B^T - X|, which
    numpy's lstsq of the augmented system [Y; sqrt(lam) I] gives as well."""
    rng = np.random.default_rng(6)
    H, T, d = 1, 300, 8
    xprev = rng.standard_normal((H, T, d)).astype(np.float32)
    xnext = rng.standard_normal((H, T, d))
    U = np.zeros((d, 1), np.float32)
    V = np.zeros((d, 1), np.float32)
    B, _ = xlayer.refit_block(xprev, xnext, U, V)
    y = numerics.round_to_bf16(xprev).astype(np.float64)[0]
    lam = xlayer.REFIT_RIDGE * np.trace(y.T @ y) / d
    Ya = np.vstack([y, np.sqrt(lam) * np.eye(d)])
    Xa = np.vstack([xnext[0], np.zeros((d, d))])
    ref = np.linalg.lstsq(Ya, Xa, rcond=None)[0].T
    np.testing.assert_allclose(B[0], ref, rtol=1e-10, atol=1e-12)
