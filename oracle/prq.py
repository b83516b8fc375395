"""Progressive Residual Quantization, bit packing and reconstruction (test infrastructure only).

QVG explainer, "Sommario tecnico" 2.B: after the first quantization of the
residual left by smoothing, the same quantization is applied again to what
remains, stage after stage, each stage capturing finer detail; the number of
stages trades quality for compression.  At decode time the quantized
residuals are dequantized and the centroids added back to rebuild the cache.
"L'essenziale" step B states the same coarse-to-fine loop in plain words.
The explainer's title fixes the code width at 2 bits; the 4-bit variant is
the same quantizer with b = 4.

Readings of what the pages leave open (all arithmetic IEEE fp32 unless
stated; one token's d-vector is cut into d/G groups of G contiguous channels):

* per group and stage: mn, mx = min, max of the current residual;
  z = fp16(mn); sigma = fp16(fl32(fl32(mx - z) / (2**b - 1))), both rounded
  to nearest even, and the quantizer uses the stored (rounded) values.
* if sigma == 0 the group is degenerate: every code is 0 and the
  dequantized value is z.
* otherwise inv = fl32(1 / sigma); u = fl32(fl32(r - z) * inv);
  code = clamp(round_half_even(u), 0, 2**b - 1); the dequantized value is
  rhat = fmaf(code, sigma, z) (one rounding).
* closed loop: the next stage quantizes fl32(r - rhat).
* packing: element j of a token's code row sits at byte floor(j*b/8), bit
  (j*b) mod 8 (least significant bits first).
* reconstruction: xhat = fl32(...fl32(fl32(base + rhat_1) + rhat_2)... + rhat_S),
  left to right, where base is the token's centroid (or the cross-layer
  prediction).
"""
import numpy as np


def dequant(code, sigma16, z16):
    """fmaf(code, sigma, z) evaluated exactly.

    code <= 15 has 4 bits and sigma is an fp16 value (11 significant bits),
    so code*sigma is exact in fp64; code*sigma and z are both integer
    multiples of 2**-24 (the fp16 quantum) below 2**20 in magnitude, so their
    fp64 sum is exact as well.  Rounding that exact value to fp32 once is by
    definition the fused multiply-add.
    """
    q64 = np.asarray(code, dtype=np.float64)
    s64 = np.asarray(sigma16, dtype=np.float16).astype(np.float64)
    z64 = np.asarray(z16, dtype=np.float16).astype(np.float64)
    return (q64 * s64 + z64).astype(np.float32)


def quantize_stage(r, bits, group):
    """One PRQ stage on a [T, d] fp32 residual.

    Returns codes [T, d] uint8, sigma [T, d/G] fp16, z [T, d/G] fp16,
    rhat [T, d] fp32 and the next residual fl32(r - rhat).
    """
    r = np.asarray(r, dtype=np.float32)
    T, d = r.shape
    if d % group:
        raise ValueError("group size must divide head_dim")
    levels = np.float32(2 ** bits - 1)
    rg = r.reshape(T, d // group, group)
    mn = rg.min(axis=2)
    mx = rg.max(axis=2)
    z = mn.astype(np.float16)
    zf = z.astype(np.float32)
    sigma = ((mx - zf) / levels).astype(np.float16)
    sf = sigma.astype(np.float32)
    degenerate = sf == np.float32(0)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        inv = np.float32(1) / sf
        u = (rg - zf[:, :, None]) * inv[:, :, None]
        q = np.clip(np.rint(u), np.float32(0), levels)
    q = np.where(degenerate[:, :, None], np.float32(0), q)
    codes = q.astype(np.uint8)
    rhat = dequant(codes, sigma[:, :, None], z[:, :, None])
    r_next = rg - rhat
    return (codes.reshape(T, d), sigma, z, rhat.reshape(T, d), r_next.reshape(T, d))


def quantize(r0, n_stages, bits, group):
    """All S stages.  Returns lists (codes, sigma, z, rhat) per stage and the final residual."""
    codes, sigmas, zs, rhats = [], [], [], []
    r = np.asarray(r0, dtype=np.float32)
    for _ in range(n_stages):
        q, s, z, rh, r = quantize_stage(r, bits, group)
        codes.append(q)
        sigmas.append(s)
        zs.append(z)
        rhats.append(rh)
    return codes, sigmas, zs, rhats, r


def pack(codes, bits):
    """Pack [T, d] codes LSB-first into [T, d*bits/8] bytes."""
    codes = np.asarray(codes, dtype=np.uint8)
    T, d = codes.shape
    per_byte = 8 // bits
    if (d * bits) % 8:
        raise ValueError("row does not fill whole bytes")
    c = codes.reshape(T, d // per_byte, per_byte).astype(np.uint32)
    out = np.zeros((T, d // per_byte), dtype=np.uint32)
    for i in range(per_byte):
        out |= c[:, :, i] << (i * bits)
    return out.astype(np.uint8)


def unpack(packed, bits, d):
    """Inverse of ``pack``."""
    packed = np.asarray(packed, dtype=np.uint8)
    per_byte = 8 // bits
    mask = (1 << bits) - 1
    T = packed.shape[0]
    out = np.zeros((T, d // per_byte, per_byte), dtype=np.uint8)
    for i in range(per_byte):
        out[:, :, i] = (packed >> (i * bits)) & mask
    return out.reshape(T, d)


def reconstruct(base, rhats):
    """xhat = fl32(...fl32(base + rhat_1)... + rhat_S), stages left to right."""
    x = np.asarray(base, dtype=np.float32).copy()
    for rh in rhats:
        x = x + np.asarray(rh, dtype=np.float32)
    return x


def reconstruct_from_codes(base, codes_packed, sigmas, zs, bits, group):
    """Decode path from stored data: unpack, dequantize, add to base in stage order."""
    base = np.asarray(base, dtype=np.float32)
    T, d = base.shape
    rhats = []
    for pk, s, z in zip(codes_packed, sigmas, zs):
        q = unpack(pk, bits, d).reshape(T, d // group, group)
        rhats.append(dequant(q, np.asarray(s)[:, :, None], np.asarray(z)[:, :, None]).reshape(T, d))
    return reconstruct(base, rhats)
