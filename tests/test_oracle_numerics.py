"""Pins for the oracle's IEEE rounding helpers (CPU only)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import numerics, prq


def _rne_fraction(v, sig_bits, min_exp):
    """Round an exact Fraction to `sig_bits` significant bits, ties to even.

    min_exp is the exponent of the smallest normal; below it the quantum is fixed.
    """
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    e = max(e, min_exp)
    quantum = Fraction(2) ** (e - (sig_bits - 1))
    n = abs(v) / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def test_bf16_matches_torch_from_fp32():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        rng.standard_normal(1000).astype(np.float32) * 1e-38,
                        np.array([0.0, -0.0, 1.0, 65504.0, 3.0e38], np.float32)])
    ours = numerics.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_bf16_from_fp64_is_single_rounding():
    # Values just above a bf16 midpoint in fp64 that fp32 would first round onto the
    # midpoint (double rounding would then go to even, i.e. down).
    one = 1.0
    mid = one + 2.0 ** -8          # midpoint between 1 and 1 + 2**-7
    v = np.array([mid + 2.0 ** -40, mid - 2.0 ** -40, mid], dtype=np.float64)
    got = numerics.round_to_bf16(v).astype(np.float64)
    assert got[0] == one + 2.0 ** -7
    assert got[1] == one
    assert got[2] == one            # exact tie goes to the even significand
    rng = np.random.default_rng(2)
    for val in rng.standard_normal(300) * 37.0:
        exact = _rne_fraction(Fraction(float(val)), 8, -126)
        assert Fraction(float(numerics.round_to_bf16(np.array([val]))[0])) == exact


def test_fp16_rounding_matches_exact_rne():
    rng = np.random.default_rng(3)
    vals = np.concatenate([rng.standard_normal(300).astype(np.float32),
                           rng.standard_normal(100).astype(np.float32) * 1e-6])
    for val in vals:
        exact = _rne_fraction(Fraction(float(val)), 11, -14)
        assert Fraction(float(numerics.round_to_fp16(np.float32(val)))) == exact


def test_dequant_equals_exact_fma():
    rng = np.random.default_rng(4)
    q = rng.integers(0, 16, 2000)
    s = (rng.standard_normal(2000) * rng.choice([1e-4, 1e-2, 1.0, 30.0], 2000)).astype(np.float16)
    z = (rng.standard_normal(2000) * rng.choice([1e-4, 1e-2, 1.0, 30.0], 2000)).astype(np.float16)
    got = prq.dequant(q, s, z)
    for i in range(2000):
        exact = Fraction(int(q[i])) * Fraction(float(s[i])) + Fraction(float(z[i]))
        assert Fraction(float(got[i])) == _rne_fraction(exact, 24, -126)


def test_bf16_bits_roundtrip():
    x = numerics.round_to_bf16(np.linspace(-5, 5, 1001))
    np.testing.assert_array_equal(numerics.bf16_from_bits(numerics.bf16_bits(x)), x)
    with pytest.raises(ValueError):
        numerics.bf16_bits(np.array([1.0 + 2.0 ** -20], np.float32))
