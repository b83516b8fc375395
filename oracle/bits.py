"""Closed-form storage cost of the encoded cache (test infrastructure only).

QVG explainer, "Sommario tecnico" 4 and the title: the method reports the
compression of the KV cache at 2 bits per code.  With the readings of this
oracle (per-group fp16 scale and zero per stage, one cluster id per token,
one codebook snapshot per head per encode call) the stored bits per cached
element are

    S*b                         codes
  + S*2*16/G                    fp16 (sigma, z) per group per stage
  + 8*id_bytes/d                one id per token, shared by its d channels
  + 8*cb_bytes*C/n_call         the call's codebook, amortised over its tokens

with id_bytes = 1 for C <= 256, else 2, and cb_bytes the cache dtype's size.
With codebook reuse the stream keeps one codebook, so n_call is replaced by
every token the stream holds.  With outlier channels each token and stage
holds one more fp16 (sigma, z) pair (S*32/d) and each call one d-bit flag
mask per head (1/n_call).
"""
from fractions import Fraction


def bits_per_element(n_stages, bits, group, head_dim, n_clusters, cb_bytes, n_call,
                     with_ids=True, outliers=False):
    """Exact bits per element as a Fraction."""
    id_bytes = 1 if n_clusters <= 256 else 2
    total = Fraction(n_stages * bits) + Fraction(n_stages * 32, group)
    if outliers:
        total += Fraction(n_stages * 32, head_dim) + Fraction(1, n_call)
    if with_ids:
        total += Fraction(8 * id_bytes, head_dim)
        total += Fraction(8 * cb_bytes * n_clusters, n_call)
    return total


def compression_ratio(input_bytes, *args, **kw):
    """Ratio of the input's bits per element to the stored bits per element."""
    return Fraction(8 * input_bytes) / bits_per_element(*args, **kw)
