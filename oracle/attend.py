"""Attention read over the reconstructed cache (test infrastructure only).

QVG explainer, "Sommario tecnico" 2.B (decode: dequantize the residuals and
add the centroids back) and section 3 (dequantization is fused into the
kernels); the 33-method study abstract notes that materialising BF16 copies
of the cache during attention defeats the compression.  The oracle states
only what the read computes; the fused kernel never stores the rebuilt K/V.

Readings: multi-head attention with as many query heads as KV heads, no
mask, scale 1/sqrt(d), over every token encoded so far.  The operands that
enter the products are the bf16 roundings (nearest even) of the queries and
of the reconstructed keys and values; logits, softmax and the weighted sum
are evaluated in fp64 with the row maximum subtracted.  LSE is the natural
log of the softmax denominator of the scaled logits.
"""
import numpy as np

from .numerics import round_to_bf16


def attend(q, khat, vhat, rows=256):
    """q [H, Tq, d]; khat, vhat [H, Tk, d] (fp32 reconstructions).

    Returns O [H, Tq, d] float64 and LSE [H, Tq] float64.  Query rows are
    independent; they are processed ``rows`` at a time only to bound memory.
    """
    qb = round_to_bf16(q).astype(np.float64)
    kb = round_to_bf16(khat).astype(np.float64)
    vb = round_to_bf16(vhat).astype(np.float64)
    H, Tq, d = q.shape
    scale = np.sqrt(np.float64(d))
    out = np.empty((H, Tq, vb.shape[-1]), dtype=np.float64)
    lse = np.empty((H, Tq), dtype=np.float64)
    for h in range(H):
        kt = np.ascontiguousarray(kb[h].T)
        for r0 in range(0, Tq, rows):
            logits = (qb[h, r0:r0 + rows] @ kt) / scale
            m = logits.max(axis=-1, keepdims=True)
            p = np.exp(logits - m)
            denom = p.sum(axis=-1, keepdims=True)
            out[h, r0:r0 + rows] = (p @ vb[h]) / denom
            lse[h, r0:r0 + rows] = (m + np.log(denom))[:, 0]
    return out, lse


def merge(o1, lse1, o2, lse2):
    """Combine two attention results over disjoint key sets by their LSE."""
    m = np.maximum(lse1, lse2)
    w1 = np.exp(lse1 - m)
    w2 = np.exp(lse2 - m)
    out = (o1 * w1[..., None] + o2 * w2[..., None]) / (w1 + w2)[..., None]
    return out, m + np.log(w1 + w2)
