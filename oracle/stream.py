"""One (layer, K|V) cache stream encoded chunk by chunk (test infrastructure only).

QVG explainer, "Sommario tecnico" 2.A/2.B/3: the cache of each head is
smoothed by k-means and its residual quantized in stages; centroid caching
speeds the clustering up.  Readings: every encode call appends one chunk of
tokens and leaves one codebook snapshot per head; the k-means of a call
starts from the previous call's snapshot (or from strided tokens for the
stream's first call); a token always decodes with the snapshot of the call
that encoded it; earlier chunks are never re-encoded.

In cross-layer mode a layer >= 1 has no clustering: its base is the
prediction from the previous layer's reconstruction (see ``xlayer``).

Codebook reuse (the other reading of centroid caching, "Sommario tecnico"
3, offered as an option): only a stream's first call runs the k-means; a
later call assigns its tokens to that first codebook, with no iterations,
and keeps it as its snapshot.

Outlier channels (option, see ``outlier``): a call flags the channels of
each head whose residual norm stands out and codes them as one extra group
per token and stage; the flags are kept with the call's snapshot.
"""
import numpy as np

from . import outlier, prq, sas


class Chunk:
    """Encoded content of one call for one head: what the decoder needs."""

    def __init__(self, ids, codebook, packed, sigmas, zs, base, xhat, r_final, rhats, flags=None):
        self.ids = ids            # [n] cluster ids (None in cross-layer mode)
        self.codebook = codebook  # [C, d] snapshot (None in cross-layer mode)
        self.packed = packed      # S x [n, d*b/8] uint8
        self.sigmas = sigmas      # S x [n, d/G] fp16
        self.zs = zs              # S x [n, d/G] fp16
        self.base = base          # [n, d] fp32: centroid rows or prediction
        self.xhat = xhat          # [n, d] fp32 reconstruction
        self.r_final = r_final    # [n, d] fp32 residual after the last stage
        self.rhats = rhats        # S x [n, d] fp32 dequantized stages
        self.flags = flags        # [d] bool outlier channels of the call (None: option off)


def encode_head(x, n_clusters, iters, n_stages, bits, group, dtype, init=None, outliers=False):
    """Encode one head's new tokens x [n, d] with SAS + PRQ (optionally with
    the outlier-channel group)."""
    ids, cb = sas.kmeans(x, n_clusters, iters, dtype, init=init)
    base = cb[ids]
    r0 = sas.centroid_residual(x, cb, ids)
    flags = None
    if outliers:
        flags = outlier.channel_flags(r0)
        codes, sig, zs, rhats, r_fin = outlier.quantize_dual(r0, n_stages, bits, group, flags)
    else:
        codes, sig, zs, rhats, r_fin = prq.quantize(r0, n_stages, bits, group)
    packed = [prq.pack(q, bits) for q in codes]
    xhat = prq.reconstruct(base, rhats)
    return Chunk(ids, cb, packed, sig, zs, base, xhat, r_fin, rhats, flags)


def encode_residual_head(x, pred, n_stages, bits, group):
    """Encode one head's tokens against a given base (cross-layer prediction)."""
    r0 = np.asarray(x, dtype=np.float32) - np.asarray(pred, dtype=np.float32)
    codes, sig, zs, rhats, r_fin = prq.quantize(r0, n_stages, bits, group)
    packed = [prq.pack(q, bits) for q in codes]
    xhat = prq.reconstruct(pred, rhats)
    return Chunk(None, None, packed, sig, zs, np.asarray(pred, np.float32), xhat, r_fin, rhats)


class Stream:
    """Cache stream of one layer and tensor: all heads, all chunks so far."""

    def __init__(self, n_heads, head_dim, n_clusters, iters, n_stages, bits, group, dtype, reuse=False,
                 outliers=False):
        self.H, self.d = n_heads, head_dim
        self.C, self.iters = n_clusters, iters
        self.S, self.b, self.G = n_stages, bits, group
        self.dtype = dtype
        self.reuse = reuse
        self.outliers = outliers
        self.chunks = []          # list of per-head Chunk lists
        self.starts = []          # first token of each chunk

    @property
    def n_tokens(self):
        return sum(ch[0].xhat.shape[0] for ch in self.chunks) if self.chunks else 0

    def encode(self, x):
        """Append x [H, n, d]; the k-means warm-starts from the last snapshot
        (with reuse, a later call only assigns to the first codebook)."""
        prev = self.chunks[-1] if self.chunks else None
        per_head = []
        for h in range(self.H):
            init = None if prev is None else prev[h].codebook
            iters = 0 if (self.reuse and prev is not None) else self.iters
            per_head.append(encode_head(x[h], self.C, iters, self.S, self.b,
                                        self.G, self.dtype, init=init, outliers=self.outliers))
        self.starts.append(self.n_tokens)
        self.chunks.append(per_head)
        return per_head

    def encode_residual(self, x, pred):
        """Append x [H, n, d] coded against pred [H, n, d] (cross-layer layers)."""
        per_head = [encode_residual_head(x[h], pred[h], self.S, self.b, self.G)
                    for h in range(self.H)]
        self.starts.append(self.n_tokens)
        self.chunks.append(per_head)
        return per_head

    def xhat(self):
        """Reconstruction [H, T, d] fp32 of every token encoded so far."""
        return np.stack([np.concatenate([ch[h].xhat for ch in self.chunks], axis=0)
                         for h in range(self.H)])

    def field(self, name, stage=None):
        """Concatenate one per-chunk field over chunks: [H, T, ...]."""
        out = []
        for h in range(self.H):
            parts = []
            for ch in self.chunks:
                v = getattr(ch[h], name)
                parts.append(v if stage is None else v[stage])
            out.append(np.concatenate(parts, axis=0))
        return np.stack(out)
