"""Codebook reuse in the oracle (CPU): the other reading of centroid caching
(QVG explainer, "Sommario tecnico" 3) keeps a stream's first codebook and
only assigns later calls to it.

Pins: a later chunk's ids are the argmin of squared distances to the first
snapshot computed by scipy's cdist (an independent library routine); its
snapshot is the first one, unchanged; the first chunk equals the per-call
stream's first chunk; the codebook share of the storage cost is amortised
over every token of the stream (0.875 bits per element per 4680-token call
for C = 256 bf16 rows of 128 channels, 1/40 of that over 40 calls)."""
from fractions import Fraction

import numpy as np
from scipy.spatial.distance import cdist

from oracle import bits as o_bits
from oracle import stream as o_stream


def _drifting_tokens(rng, H, n, d, n_proto, t0):
    protos = np.random.default_rng(7).standard_normal((H, n_proto, d)).astype(np.float32)
    drift = 0.05 * (t0 / 300.0)
    lab = rng.integers(0, n_proto, size=(H, n))
    x = protos[np.arange(H)[:, None], lab] * (1.0 + drift) + 0.1 * rng.standard_normal((H, n, d))
    return x.astype(np.float32)


def test_reuse_assigns_later_chunks_to_the_first_codebook():
    rng = np.random.default_rng(3)
    H, d, C = 2, 16, 8
    chunks = [_drifting_tokens(rng, H, n, d, 6, t0) for n, t0 in ((300, 0), (257, 300), (1, 557))]
    reuse = o_stream.Stream(H, d, C, 5, 2, 2, 16, "f32", reuse=True)
    plain = o_stream.Stream(H, d, C, 5, 2, 2, 16, "f32")
    for x in chunks:
        reuse.encode(x)
        plain.encode(x)
    for h in range(H):
        first = reuse.chunks[0][h]
        np.testing.assert_array_equal(first.ids, plain.chunks[0][h].ids)
        np.testing.assert_array_equal(first.codebook, plain.chunks[0][h].codebook)
        for c in (1, 2):
            ch = reuse.chunks[c][h]
            np.testing.assert_array_equal(ch.codebook, first.codebook)
            dist = cdist(chunks[c][h].astype(np.float64), first.codebook.astype(np.float64), "sqeuclidean")
            np.testing.assert_array_equal(ch.ids, np.argmin(dist, axis=1))
            np.testing.assert_array_equal(ch.base, first.codebook[ch.ids])
    # the per-call stream moved its codebook on the drifting data
    assert not np.array_equal(plain.chunks[1][0].codebook, plain.chunks[0][0].codebook)


def test_reuse_codebook_share_of_the_storage_cost():
    per_call = o_bits.bits_per_element(2, 2, 32, 128, 256, 2, 4680)
    reused = o_bits.bits_per_element(2, 2, 32, 128, 256, 2, 40 * 4680)
    fixed = Fraction(4) + Fraction(2 * 32, 32) + Fraction(8, 128)
    assert per_call - fixed == Fraction(8 * 2 * 256, 4680)
    assert abs(float(per_call - fixed) - 0.875) < 1e-3
    assert (per_call - fixed) == 40 * (reused - fixed)
