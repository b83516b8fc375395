"""Pins for the oracle's outlier-channel dual-scale stages (CPU only).

Q-ARVD explainer, section on outlier-aware adaptive dual-scale
quantization: channels whose L2 norm a MAD-based modified z-score flags
(with a minimum magnitude relative to the median) are quantized apart from
the normal channels; with no flagged channel the quantizer is the standard
one.  Pins: hand-derived flag decisions and stage values, the reduction to
plain PRQ when nothing is flagged, an independent per-subset textbook
quantizer, a library median, brute-force norms, error bounds per group, a
lossless case, and the decode identity.
"""
import json
import math
import os
import statistics

import numpy as np
import pytest
import torch

from oracle import outlier, prq, sas, stream
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cases():
    with open(os.path.join(GOLDEN, "outlier_cases.json")) as f:
        return json.load(f)


def test_golden_flag_cases():
    for case in _cases()["flag_cases"]:
        flags, _, _ = outlier.flags_from_norms(np.array(case["norms"], np.float64))
        assert flags.astype(int).tolist() == case["flags"], case["name"]


def test_golden_dual_stage_values():
    for case in _cases()["stage_cases"]:
        r = np.array([case["r"]], np.float32)
        flags = np.array(case["flags"], bool)
        q, s, z, rh, rn = outlier.quantize_stage_dual(r, case["bits"], case["group"], flags)
        assert q[0].tolist() == case["codes"], case["name"]
        assert s[0].astype(np.float64).tolist() == case["sigma"], case["name"]
        assert z[0].astype(np.float64).tolist() == case["z"], case["name"]
        assert rh[0].astype(np.float64).tolist() == case["rhat"], case["name"]
        assert prq.pack(q, case["bits"])[0].tolist() == case["packed"], case["name"]
        np.testing.assert_array_equal(rn, r - rh)


def test_flags_match_stdlib_median_rule():
    # the rule evaluated with Python's statistics.median (a library routine)
    # on random norm vectors with planted spikes
    rng = np.random.default_rng(7)
    for trial in range(200):
        d = int(rng.choice([8, 64, 128]))
        n = rng.gamma(4.0, 1.0, d)
        k = int(rng.integers(0, 5))
        n[rng.choice(d, k, replace=False)] *= rng.uniform(1.0, 30.0, k)
        med = statistics.median(n.tolist())
        mad = statistics.median([abs(v - med) for v in n.tolist()])
        want = [0.6745 * (v - med) > 3.5 * mad and v > 2.0 * med for v in n.tolist()]
        got, m2, a2 = outlier.flags_from_norms(n)
        assert got.tolist() == want
        assert m2 == med and a2 == mad


def test_norms_brute_force():
    rng = np.random.default_rng(3)
    r = (rng.standard_normal((37, 16)) * rng.uniform(0.1, 10, 16)).astype(np.float32)
    got = outlier.channel_norms(r)
    for j in range(16):
        want = math.sqrt(math.fsum(float(r[t, j]) ** 2 for t in range(37)))
        assert abs(got[j] - want) <= 1e-14 * want


def test_no_flag_reduces_to_plain_prq():
    rng = np.random.default_rng(11)
    for bits, G in ((2, 32), (4, 64), (2, 64)):
        r0 = rng.standard_normal((50, 128)).astype(np.float32)
        flags = np.zeros(128, bool)
        c1, s1, z1, rh1, rf1 = prq.quantize(r0, 3, bits, G)
        c2, s2, z2, rh2, rf2 = outlier.quantize_dual(r0, 3, bits, G, flags)
        for s in range(3):
            np.testing.assert_array_equal(c1[s], c2[s])
            np.testing.assert_array_equal(s1[s].view(np.uint16), s2[s][:, :-1].view(np.uint16))
            np.testing.assert_array_equal(z1[s].view(np.uint16), z2[s][:, :-1].view(np.uint16))
            assert not s2[s][:, -1].view(np.uint16).any() and not z2[s][:, -1].view(np.uint16).any()
        np.testing.assert_array_equal(rf1, rf2)


def _textbook_rtn(v, bits):
    """Asymmetric min-max round-to-nearest of one vector with fp16 scale and
    zero (the quantizer's reading), written out element by element."""
    lo = np.float16(np.float32(min(v)))
    sc = np.float16(np.float32(np.float32(max(v)) - np.float32(lo)) / np.float32(2 ** bits - 1))
    out = []
    for x in v:
        if np.float32(sc) == 0:
            q = 0
        else:
            u = np.float32(np.float32(np.float32(x) - np.float32(lo)) * np.float32(np.float32(1) / np.float32(sc)))
            q = int(min(max(np.rint(u), 0), 2 ** bits - 1))
        out.append(q)
    return out, sc, lo


def test_each_group_is_an_independent_textbook_quantizer():
    rng = np.random.default_rng(5)
    for bits, G in ((2, 32), (4, 32), (2, 64)):
        d = 128
        r = rng.standard_normal((20, d)).astype(np.float32)
        flags = np.zeros(d, bool)
        flags[rng.choice(d, 6, replace=False)] = True
        r[:, flags] *= 25
        q, s, z, _, _ = outlier.quantize_stage_dual(r, bits, G, flags)
        NG = d // G
        for t in range(20):
            members = [np.nonzero(~flags[g * G:(g + 1) * G])[0] + g * G for g in range(NG)]
            members.append(np.nonzero(flags)[0])
            for g, m in enumerate(members):
                codes, sc, lo = _textbook_rtn(r[t, m].tolist(), bits)
                assert q[t, m].tolist() == codes
                assert s[t, g] == sc and z[t, g] == lo


def test_group_error_bound_per_member_set():
    # P6 carried over: per group, max|r^s| <= max|r^{s-1}| / (2^b - 1) plus the
    # rounding slack of the fp16 scale and zero
    cfg = synth.scaled(synth.WAN_LAYER, n_heads=1, tokens=600)
    x = synth.kv_tokens(cfg, 0, 0, 0, 600).float().numpy()[0]
    ids, cb = sas.kmeans(x, 16, 3, "bf16")
    r0 = sas.centroid_residual(x, cb, ids)
    flags = outlier.channel_flags(r0)
    assert flags.sum() == cfg.n_out
    for bits in (2, 4):
        r = r0
        for _ in range(2):
            q, s, z, rh, rn = outlier.quantize_stage_dual(r, bits, 32, flags)
            sets = [np.nonzero(~flags[g * 32:(g + 1) * 32])[0] + g * 32 for g in range(4)]
            sets.append(np.nonzero(flags)[0])
            for m in sets:
                if len(m) == 0:
                    continue
                before = np.abs(r[:, m]).max(axis=1)
                after = np.abs(rn[:, m]).max(axis=1)
                slack = 4e-3 * before + 1e-6
                assert np.all(after <= before / (2 ** bits - 1) + slack)
            r = rn


def test_lossless_on_two_grids():
    # normal channels on a step-1 grid from 0, outlier channels on a step-64
    # grid from -128: both recovered exactly with one INT2 stage
    rng = np.random.default_rng(2)
    d, G = 64, 32
    flags = np.zeros(d, bool)
    flags[[5, 40]] = True
    r = rng.integers(0, 4, (30, d)).astype(np.float32)
    r[:, 0] = 0.0
    r[:, 1] = 3.0
    r[:, 32] = 0.0
    r[:, 33] = 3.0
    r[:, flags] = (-128 + 64 * rng.integers(0, 4, (30, 2))).astype(np.float32)
    r[:, 5] = -128.0
    r[:, 40] = 64.0
    codes, sig, zs, rhats, rfin = outlier.quantize_dual(r, 1, 2, G, flags)
    assert not rfin.any()
    # the plain quantizer cannot: the outliers stretch their groups' ranges
    _, _, _, _, rplain = prq.quantize(r, 1, 2, G)
    assert np.abs(rplain).max() > 0


def test_decode_identity_and_pack_flags():
    rng = np.random.default_rng(9)
    d, G, bits = 128, 32, 2
    base = rng.standard_normal((40, d)).astype(np.float32)
    flags = np.zeros(d, bool)
    flags[[0, 33, 127]] = True
    x = (base + rng.standard_normal((40, d)) * np.where(flags, 40.0, 1.0)).astype(np.float32)
    r0 = x - base
    codes, sig, zs, rhats, rfin = outlier.quantize_dual(r0, 2, bits, G, flags)
    packed = [prq.pack(q, bits) for q in codes]
    x1 = outlier.reconstruct_from_codes_dual(base, packed, sig, zs, bits, G, flags)
    np.testing.assert_array_equal(x1, prq.reconstruct(base, rhats))
    # x - xhat = r^S up to one half-ulp per fp32 operation at the largest
    # magnitude the partial sums reach
    partial = [base]
    for rh in rhats:
        partial.append(partial[-1] + rh)
    big = np.maximum.reduce([np.abs(x)] + [np.abs(p) for p in partial])
    diff = x.astype(np.float64) - x1.astype(np.float64)
    assert np.all(np.abs(diff - rfin.astype(np.float64)) <= 4 * np.spacing(big).astype(np.float64))
    assert outlier.pack_flags(flags).tolist() == [1, 2, 0, 0x80000000]


def test_stream_flags_find_planted_channels_and_cut_error():
    # empirical, like the tensor-level PRQ pin: on the generator's shape with
    # 4 channels scaled x10, the planted channels are the flagged ones and the
    # dual-scale stages leave a smaller residual than the plain ones
    cfg = synth.scaled(synth.WAN_LAYER, n_heads=2, tokens=1000)
    x = synth.kv_tokens(cfg, 0, 1, 0, 1000).float().numpy()
    planted = synth.channel_scale(cfg, 0, 1).numpy() > 1
    plain = stream.Stream(2, 128, 32, 3, 2, 2, 32, "bf16")
    dual = stream.Stream(2, 128, 32, 3, 2, 2, 32, "bf16", outliers=True)
    plain.encode(x)
    dual.encode(x)
    for h in range(2):
        assert dual.chunks[0][h].flags.tolist() == planted[h].tolist()
        np.testing.assert_array_equal(dual.chunks[0][h].ids, plain.chunks[0][h].ids)
        assert np.linalg.norm(dual.chunks[0][h].r_final) < 0.75 * np.linalg.norm(plain.chunks[0][h].r_final)
        assert outlier.flag_margin(outlier.channel_norms(
            sas.centroid_residual(x[h], dual.chunks[0][h].codebook, dual.chunks[0][h].ids))) > 1e-6


def test_stored_sizes_with_outliers_match_closed_form():
    # the bytes one encoded head holds with the option (codes, (sigma, z) with
    # the extra entry, ids, codebook, the d-bit flag mask) = the closed form;
    # at the Wan-layer shape that is 6.19 -> 6.69 bits per element
    from fractions import Fraction
    from oracle import bits
    cfg = synth.scaled(synth.WAN_LAYER, n_heads=1, tokens=1024)
    x = synth.kv_tokens(cfg, 0, 0, 0, 1024)[0].float().numpy()
    ch = stream.encode_head(x, 16, 2, 2, 2, 32, "bf16", outliers=True)
    nbytes = sum(p.nbytes for p in ch.packed) + sum(s.nbytes + z.nbytes for s, z in zip(ch.sigmas, ch.zs)) \
        + 1024 * 1 + ch.codebook.shape[0] * 128 * 2 + outlier.pack_flags(ch.flags).nbytes
    assert Fraction(8 * nbytes, 1024 * 128) == bits.bits_per_element(2, 2, 32, 128, 16, 2, 1024, outliers=True)
    plain = bits.bits_per_element(2, 2, 32, 128, 256, 2, 32760)
    dual = bits.bits_per_element(2, 2, 32, 128, 256, 2, 32760, outliers=True)
    assert round(float(plain), 2) == 6.19 and round(float(dual), 2) == 6.69
