"""Pins for the oracle's progressive residual quantization (CPU only).

QVG explainer, "Sommario tecnico" 2.B: quantize the smoothed residual, then
repeat on what remains, coarse to fine; decode dequantizes and adds the
centroids back.  Pins: hand-computed bytes and stage values, error bounds
that follow from the quantizer's definition, a lossless special case, an
independent textbook round-to-nearest quantizer, and the decode identity.
"""
import json
import os

import numpy as np
import pytest

from oracle import numerics, prq, sas, stream
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_pack_hand_values():
    # INT2 codes [0, 1, 2, 3] -> 0b11_10_01_00 = 0xE4; INT4 [1, 2] -> 0x21
    assert prq.pack(np.array([[0, 1, 2, 3]]), 2).tolist() == [[0xE4]]
    assert prq.pack(np.array([[1, 2]]), 4).tolist() == [[0x21]]
    rng = np.random.default_rng(1)
    for bits in (2, 4):
        q = rng.integers(0, 2 ** bits, (17, 128)).astype(np.uint8)
        np.testing.assert_array_equal(prq.unpack(prq.pack(q, bits), bits, 128), q)


def test_golden_stage_values():
    with open(os.path.join(GOLDEN, "prq_hand_cases.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        r = np.array([case["r"]], np.float32)
        q, s, z, rh, rn = prq.quantize_stage(r, case["bits"], len(case["r"]))
        assert q[0].tolist() == case["codes"], case["name"]
        assert float(z[0, 0]) == case["z"], case["name"]
        assert float(s[0, 0]) == case["sigma"], case["name"]
        assert rh[0].tolist() == case["rhat"], case["name"]
        assert prq.pack(q, case["bits"])[0].tolist() == case["packed"], case["name"]


def _residual_like(rng, T, d, scale):
    return (rng.standard_normal((T, d)) * scale).astype(np.float32)


@pytest.mark.parametrize("bits,group", [(2, 32), (2, 64), (4, 64), (2, 8)])
def test_stage_error_bound(bits, group):
    rng = np.random.default_rng(bits * 100 + group)
    r = _residual_like(rng, 500, 128, rng.uniform(0.01, 5.0, (500, 1)))
    q, s, z, rh, rn = prq.quantize_stage(r, bits, group)
    T = r.shape[0]
    rg = r.reshape(T, -1, group).astype(np.float64)
    mn = rg.min(axis=2)
    mx = rg.max(axis=2)
    sf = s.astype(np.float64)
    zf = z.astype(np.float64)
    sigma_exact = (mx - zf) / (2 ** bits - 1)
    err = np.abs(rg - rh.reshape(T, -1, group).astype(np.float64))
    ulp = np.spacing(np.abs(rg).astype(np.float32)).astype(np.float64)
    bound = (np.abs(sf) / 2 + np.abs(mn - zf) + 3 * np.abs(sigma_exact - sf))[:, :, None] + 2 * ulp
    assert np.all(err <= bound * (1 + 1e-6))
    # codes in range, r_next is the fp32 difference
    assert q.max() <= 2 ** bits - 1
    np.testing.assert_array_equal(rn, r - rh)


@pytest.mark.parametrize("bits,group", [(2, 32), (4, 64)])
def test_group_max_shrinks_per_stage(bits, group):
    rng = np.random.default_rng(7)
    r = _residual_like(rng, 400, 128, 0.3)
    levels = 2 ** bits - 1
    for _ in range(3):
        q, s, z, rh, rn = prq.quantize_stage(r, bits, group)
        T = r.shape[0]
        old = np.abs(r.reshape(T, -1, group)).max(axis=2)
        new = np.abs(rn.reshape(T, -1, group)).max(axis=2)
        mn = r.reshape(T, -1, group).min(axis=2).astype(np.float64)
        mx = r.reshape(T, -1, group).max(axis=2).astype(np.float64)
        sf = s.astype(np.float64)
        slack = np.abs(mn - z.astype(np.float64)) + 3 * np.abs((mx - z) / levels - sf) \
            + 4 * np.spacing(old)
        assert np.all(new <= old / levels + slack + 1e-30)
        r = rn


def test_tensor_residual_norm_shrinks_on_seeded_configs():
    for cfg in (synth.scaled(synth.TINY, tokens=2048),
                synth.scaled(synth.WAN_LAYER, n_heads=2, tokens=3120)):
        x = synth.kv_tokens(cfg, 0, 1, 0, cfg.tokens)[0].float().numpy()
        ids, cb = sas.kmeans(x, cfg.n_clusters, 2, cfg.dtype)
        r = sas.centroid_residual(x, cb, ids)
        norms = [np.linalg.norm(r.astype(np.float64))]
        for _ in range(3):
            *_, r = prq.quantize_stage(r, cfg.bits, cfg.group)
            norms.append(np.linalg.norm(r.astype(np.float64)))
        assert all(b < a for a, b in zip(norms, norms[1:])), norms


def test_degenerate_groups():
    r = np.zeros((3, 64), np.float32)
    r[1] = 0.25                      # constant group: sigma rounds to 0
    r[2, :32] = -1.5
    q, s, z, rh, rn = prq.quantize_stage(r, 2, 32)
    assert np.all(q == 0)
    assert np.all(s.astype(np.float32) == 0)
    np.testing.assert_array_equal(rh, r)
    assert np.all(rn == 0)


def test_lossless_grid_case():
    # each group holds values z + q*step with an fp16-exact z, power-of-two step
    # and codes that reach both ends: sigma = step exactly, codes come back
    rng = np.random.default_rng(9)
    T, d, G, bits = 64, 128, 32, 2
    q = rng.integers(0, 4, (T, d)).astype(np.uint8)
    q.reshape(T, -1, G)[:, :, 0] = 0
    q.reshape(T, -1, G)[:, :, 1] = 3
    step = np.ldexp(1.0, rng.integers(-8, 2, (T, d // G)))
    z = rng.integers(-64, 64, (T, d // G)) * 2.0 ** -6
    x = (z[:, :, None] + q.reshape(T, -1, G) * step[:, :, None]).reshape(T, d).astype(np.float32)
    codes, sig, zs, rh, rn = prq.quantize(x, 1, bits, G)
    np.testing.assert_array_equal(codes[0], q)
    np.testing.assert_array_equal(sig[0].astype(np.float64), step)
    np.testing.assert_array_equal(prq.reconstruct(np.zeros_like(x), rh), x)


def _textbook_rtn(x, bits, group):
    """Per-group asymmetric min-max round-to-nearest, written independently.

    zero = min and scale = (max - zero) / (2^b - 1), both stored in fp16; the
    code is the nearest integer (ties to even) to the true quotient
    (x - zero) / scale, clipped to the code range; the dequantized value is the
    real number code * scale + zero rounded once to fp32.  Also returns, per
    element, the distance of the quotient from the nearest rounding boundary.
    """
    out = np.empty_like(x)
    codes = np.empty(x.shape, np.int64)
    margin = np.full(x.shape, np.inf)
    for t in range(x.shape[0]):
        for g0 in range(0, x.shape[1], group):
            v = x[t, g0:g0 + group].astype(np.float64)
            zero = float(np.float16(v.min()))
            scale = float(np.float16(np.float32(np.float32(v.max()) - np.float32(zero))
                                     / np.float32(2 ** bits - 1)))
            if scale == 0.0:
                c = np.zeros(group, np.int64)
            else:
                u = (v - zero) / scale
                c = np.clip(np.rint(u), 0, 2 ** bits - 1).astype(np.int64)
                margin[t, g0:g0 + group] = np.abs(u - np.floor(u) - 0.5)
            codes[t, g0:g0 + group] = c
            out[t, g0:g0 + group] = (c * scale + zero).astype(np.float32)
    return codes, out, margin


@pytest.mark.parametrize("bits,group", [(2, 32), (4, 64)])
def test_single_stage_zero_codebook_is_textbook_rtn(bits, group):
    cfg = synth.scaled(synth.TINY, tokens=256)
    x = synth.kv_tokens(cfg, 0, 0, 0, 256)[0].float().numpy()
    zero_cb = np.zeros((cfg.n_clusters, cfg.head_dim), np.float32)
    r0 = sas.centroid_residual(x, zero_cb, np.zeros(256, np.int64))
    codes, sig, zs, rh, rn = prq.quantize(r0, 1, bits, group)
    tc, tout, margin = _textbook_rtn(x, bits, group)
    # the oracle multiplies by fl32(1/sigma) in fp32; it may differ from the true
    # quotient only where that quotient sits within fp32 error of a half
    near = margin < 1e-5
    assert np.count_nonzero(near) <= 1e-3 * near.size
    np.testing.assert_array_equal(codes[0][~near], tc[~near])
    same = codes[0] == tc
    np.testing.assert_array_equal(prq.reconstruct(zero_cb[np.zeros(256, np.int64)], rh)[same],
                                  tout[same])


def test_decode_identity():
    cfg = synth.scaled(synth.WAN_LAYER, n_heads=1, tokens=2000)
    x = synth.kv_tokens(cfg, 0, 0, 0, 2000)[0].float().numpy()
    ch = stream.encode_head(x, 64, 3, 3, 2, 32, "bf16")
    # xhat = base + sum rhat, in stage order; decode from the stored bytes agrees
    xhat = prq.reconstruct_from_codes(ch.base, ch.packed, ch.sigmas, ch.zs, 2, 32)
    np.testing.assert_array_equal(xhat, ch.xhat)
    # x - xhat equals the last residual up to the roundings of the partial sums:
    # one half-ulp per fp32 operation, at the largest magnitude the sums reach
    diff = x.astype(np.float64) - ch.xhat.astype(np.float64)
    partial = [ch.base]
    for rh in ch.rhats:
        partial.append(partial[-1] + rh)
    big = np.maximum.reduce([np.abs(x)] + [np.abs(p) for p in partial])
    tol = 4 * np.spacing(big).astype(np.float64)
    assert np.all(np.abs(diff - ch.r_final.astype(np.float64)) <= tol)
