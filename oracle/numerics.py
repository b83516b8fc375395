"""IEEE rounding helpers for the oracle (test infrastructure only).

All helpers are written from the IEEE-754 definitions:

* ``round_to_bf16`` -- round-to-nearest-even of a real value (given exactly
  as fp64 or fp32) to bfloat16 (8 significant bits, fp32 exponent range,
  subnormal quantum 2**-133), returned as float32 values.
* ``bf16_bits`` / ``bf16_from_bits`` -- bit patterns of bf16 values.
* ``round_to_fp16`` -- round-to-nearest-even to IEEE binary16 (numpy's
  float16 conversion is correctly rounded, half to even).
"""
import numpy as np


def round_to_bf16(v):
    """Round a float64/float32 array to the nearest bfloat16 value (ties to even).

    The rounding is done in one step from the given precision: the value is
    split as m * 2**e with 0.5 <= |m| < 1, the significand is scaled to 8 bits,
    rounded half-to-even with ``np.rint`` (exact in fp64) and scaled back.
    Values below the smallest normal use the subnormal quantum 2**-133.
    Magnitudes that round to 2**128 or beyond become infinity.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    finite = np.isfinite(v)
    vf = np.where(finite, v, 0.0)
    _, e = np.frexp(vf)
    e = np.maximum(e, -125)                 # bf16 normal exponent floor
    quantum = np.ldexp(1.0, e - 8)          # spacing of 8-bit significands
    r = np.rint(vf / quantum) * quantum     # division by a power of two is exact
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, r), r)
    out[finite] = r[finite]
    out[~finite] = v[~finite]
    return out.astype(np.float32)           # bf16 values are exact in fp32


def bf16_bits(x):
    """uint16 bit patterns of float32 values that are bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    if np.any(b & 0xFFFF):
        raise ValueError("value is not representable in bfloat16")
    return (b >> 16).astype(np.uint16)


def bf16_from_bits(b):
    """float32 values of uint16 bf16 bit patterns."""
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def round_to_fp16(x):
    """Round to IEEE binary16, nearest-even (numpy's conversion is correctly rounded)."""
    return np.asarray(x).astype(np.float16)
