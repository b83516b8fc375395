"""Outlier-channel dual-scale residual quantization (test infrastructure only).

Q-ARVD explainer ("Q-ARVD: Quantizing Autoregressive Video Diffusion
Models", gist.science), "Quantizzazione Adattiva a Doppia Scala Consapevole
degli Outlier": per layer the L2 norm of every input channel is taken; a
modified z-score built on the median absolute deviation (MAD) flags a
channel whose magnitude is above a MAD-derived threshold and also above a
minimum multiple of the median (so that a layer whose MAD is tiny shows no
false outliers); flagged and normal channels are then quantized by
independent quantizers, and a layer with no flagged channel is quantized
the standard way.  The page states this for weights; here it is carried
over to the KV-cache residual that the progressive stages code.

Readings (the page gives no constant and no formula):

* unit of detection: one head of one (layer, K|V) stream and one encode
  call.  The norms are those of the residual the stages code, after the
  call's final assignment: n_j = sqrt(sum_t r0_tj^2) in fp64 (each square of
  an fp32 value is exact in fp64).
* modified z-score of Iglewicz and Hoaglin: M_j = 0.6745 (n_j - med) / MAD,
  med and MAD the medians over the d channels (mean of the two middle values,
  d being even).  Channel j is flagged when 0.6745 (n_j - med) > 3.5 MAD and
  n_j > 2 med: the usual cut 3.5, one-sided (only large channels are
  outliers), and the minimum magnitude "twice the median".  Written without
  the division, so MAD = 0 needs no special case.
* dual scale: in every stage each token's flagged channels form one extra
  group with its own fp16 (sigma, z); every normal group keeps its G
  channels minus the flagged ones.  Min, max, sigma, z, codes and the
  dequantized value follow the plain quantizer (prq) within each group.  A
  group with no channel stores (sigma, z) = (0, 0) and codes nothing.
* codes keep their channel positions; the metadata of a token and stage
  holds d/G + 1 entries, the last one the outlier group's.  The flags of a
  call are kept with its codebook snapshot (d bits per head).
"""
import numpy as np

from . import prq

MAD_Z = 0.6745       # Phi^-1(3/4): makes the MAD a consistent estimate of sigma
Z_CUT = 3.5          # modified z-score above which a channel is flagged
MIN_RATIO = 2.0      # a flagged channel's norm must also exceed MIN_RATIO * median


def channel_norms(r0):
    """n_j = sqrt(sum_t r0[t, j]^2) in fp64 over a [T, d] fp32 residual."""
    r = np.asarray(r0, dtype=np.float32).astype(np.float64)
    return np.sqrt(np.sum(r * r, axis=0))


def median_even(v):
    """Median of an even-length vector: mean of the two middle values."""
    s = np.sort(np.asarray(v, dtype=np.float64))
    m = s.shape[0] // 2
    return (s[m - 1] + s[m]) / 2.0


def flags_from_norms(norms):
    """Flag rule on the channel norms; returns (flags, med, mad)."""
    n = np.asarray(norms, dtype=np.float64)
    if n.shape[0] % 2:
        raise ValueError("head_dim is even")
    med = median_even(n)
    mad = median_even(np.abs(n - med))
    flags = (MAD_Z * (n - med) > Z_CUT * mad) & (n > MIN_RATIO * med)
    return flags, med, mad


def flag_margin(norms):
    """Smallest relative distance of any channel from either cut (both
    conditions), so a test can tell a decision the summation order could
    flip from a clear one."""
    n = np.asarray(norms, dtype=np.float64)
    _, med, mad = flags_from_norms(n)
    scale = np.maximum(np.abs(n) + med + mad, 1e-300)
    m1 = np.abs(MAD_Z * (n - med) - Z_CUT * mad) / scale
    m2 = np.abs(n - MIN_RATIO * med) / scale
    return float(min(m1.min(), m2.min()))


def channel_flags(r0):
    """Flags [d] of a head's call from its [T, d] residual."""
    return flags_from_norms(channel_norms(r0))[0]


def _group_params(vals, member, levels):
    """(sigma, z) fp16 of each row's members; rows with no member get (0, 0).

    vals [T, k] fp32, member [k] bool.
    """
    T = vals.shape[0]
    if not member.any():
        return np.zeros(T, np.float16), np.zeros(T, np.float16)
    sub = vals[:, member]
    mn = sub.min(axis=1)
    mx = sub.max(axis=1)
    z = mn.astype(np.float16)
    sigma = ((mx - z.astype(np.float32)) / levels).astype(np.float16)
    return sigma, z


def quantize_stage_dual(r, bits, group, flags):
    """One stage with the outlier group.

    Returns codes [T, d] uint8, sigma [T, d/G + 1] fp16, z [T, d/G + 1] fp16,
    rhat [T, d] fp32 and the next residual fl32(r - rhat).
    """
    r = np.asarray(r, dtype=np.float32)
    flags = np.asarray(flags, dtype=bool)
    T, d = r.shape
    if d % group:
        raise ValueError("group size must divide head_dim")
    NG = d // group
    levels = np.float32(2 ** bits - 1)
    sigma = np.zeros((T, NG + 1), np.float16)
    z = np.zeros((T, NG + 1), np.float16)
    for g in range(NG):
        cols = slice(g * group, (g + 1) * group)
        sigma[:, g], z[:, g] = _group_params(r[:, cols], ~flags[cols], levels)
    sigma[:, NG], z[:, NG] = _group_params(r, flags, levels)
    # each element's group: its own G-group, or the outlier group NG
    gidx = np.where(flags, NG, np.arange(d) // group)
    s_el = sigma[:, gidx]
    z_el = z[:, gidx]
    sf = s_el.astype(np.float32)
    zf = z_el.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        inv = np.float32(1) / sf
        u = (r - zf) * inv
        q = np.clip(np.rint(u), np.float32(0), levels)
    q = np.where(sf == np.float32(0), np.float32(0), q)
    codes = q.astype(np.uint8)
    rhat = prq.dequant(codes, s_el, z_el)
    return codes, sigma, z, rhat, r - rhat


def quantize_dual(r0, n_stages, bits, group, flags):
    """All S stages with the outlier group; lists per stage and the final residual."""
    codes, sigmas, zs, rhats = [], [], [], []
    r = np.asarray(r0, dtype=np.float32)
    for _ in range(n_stages):
        q, s, z, rh, r = quantize_stage_dual(r, bits, group, flags)
        codes.append(q)
        sigmas.append(s)
        zs.append(z)
        rhats.append(rh)
    return codes, sigmas, zs, rhats, r


def reconstruct_from_codes_dual(base, codes_packed, sigmas, zs, bits, group, flags):
    """Decode from stored data: unpack, dequantize each element with its
    group's (sigma, z), add to the base in stage order."""
    base = np.asarray(base, dtype=np.float32)
    T, d = base.shape
    gidx = np.where(np.asarray(flags, bool), d // group, np.arange(d) // group)
    rhats = []
    for pk, s, z in zip(codes_packed, sigmas, zs):
        q = prq.unpack(pk, bits, d)
        rhats.append(prq.dequant(q, np.asarray(s)[:, gidx], np.asarray(z)[:, gidx]))
    return prq.reconstruct(base, rhats)


def pack_flags(flags):
    """Flags [d] -> d/32 uint32 words, channel j at bit j % 32 of word j // 32."""
    f = np.asarray(flags, dtype=bool)
    words = np.zeros(f.shape[0] // 32, dtype=np.uint32)
    for j in np.nonzero(f)[0]:
        words[j // 32] |= np.uint32(1) << np.uint32(j % 32)
    return words
