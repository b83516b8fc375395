"""Centroid caching in the oracle's stream (CPU).

QVG explainer, "Sommario tecnico" 3: centroid caching speeds the k-means up.
Read as a warm start: the k-means of an encode call begins from the codebook
the previous call of the same stream and head left, not from strided tokens
and not from any older snapshot.

Pin: with one Lloyd iteration, the snapshot of call c must equal one Lloyd
step taken from call c-1's snapshot, written here independently of the
oracle: scipy's cdist argmin for the assignment, an exact (math.fsum) member
mean in fp64, one rounding to the cache dtype (numpy's float32 cast, torch's
bfloat16 cast), empty clusters unchanged; the stored ids are the cdist argmin
against that new codebook.  The data drift from call to call, so the first
snapshot, or a strided start, gives a different codebook and fails the pin.
"""
import math

import numpy as np
import pytest
import torch
from scipy.spatial.distance import cdist

from oracle import stream as o_stream


def _drifting_chunks(seed, H, d, n_proto, sizes):
    """Prototype tokens that move a little with every call."""
    rng = np.random.default_rng(seed)
    protos = rng.standard_normal((H, n_proto, d))
    out = []
    for n in sizes:
        protos = protos + 0.15 * rng.standard_normal(protos.shape)
        lab = rng.integers(0, n_proto, size=(H, n))
        x = protos[np.arange(H)[:, None], lab] + 0.1 * rng.standard_normal((H, n, d))
        out.append(x.astype(np.float32))
    return out


def _round(v64, dtype):
    if dtype == "f32":
        return v64.astype(np.float32)
    return torch.from_numpy(v64).to(torch.bfloat16).to(torch.float32).numpy()


def _lloyd_step(x, c_prev, dtype):
    """One assignment + mean update from c_prev, then the final assignment."""
    x64 = x.astype(np.float64)
    ids = np.argmin(cdist(x64, c_prev.astype(np.float64), "sqeuclidean"), axis=1)
    c_new = np.array(c_prev, dtype=np.float32, copy=True)
    for k in range(c_prev.shape[0]):
        members = x64[ids == k]
        if len(members) == 0:
            continue
        mean = np.array([math.fsum(members[:, j]) for j in range(x.shape[1])]) / len(members)
        c_new[k] = _round(mean, dtype)
    ids_final = np.argmin(cdist(x64, c_new.astype(np.float64), "sqeuclidean"), axis=1)
    return c_new, ids_final


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_each_call_warm_starts_from_the_previous_snapshot(dtype):
    H, d, C = 2, 16, 12
    chunks = _drifting_chunks(11, H, d, 9, (400, 300, 350, 257))
    if dtype == "bf16":
        chunks = [_round(x.astype(np.float64), "bf16") for x in chunks]
    s = o_stream.Stream(H, d, C, 1, 2, 2, 16, dtype)
    for x in chunks:
        s.encode(x)
    for c in range(1, len(chunks)):
        for h in range(H):
            prev = s.chunks[c - 1][h].codebook
            cb, ids = _lloyd_step(chunks[c][h], prev, dtype)
            got = s.chunks[c][h]
            np.testing.assert_array_equal(got.codebook, cb, err_msg=f"call {c} head {h}")
            np.testing.assert_array_equal(got.ids, ids, err_msg=f"call {c} head {h}")
            # the pin separates the readings: starting from the first
            # snapshot instead gives another codebook for c >= 2
            if c >= 2:
                other, _ = _lloyd_step(chunks[c][h], s.chunks[0][h].codebook, dtype)
                assert not np.array_equal(other, cb)


def test_first_call_starts_from_strided_tokens():
    H, d, C = 2, 16, 12
    (x,) = _drifting_chunks(5, H, d, 9, (401,))
    s = o_stream.Stream(H, d, C, 1, 2, 2, 16, "f32")
    s.encode(x)
    for h in range(H):
        start = x[h][(np.arange(C) * 401) // C]
        cb, ids = _lloyd_step(x[h], start, "f32")
        np.testing.assert_array_equal(s.chunks[0][h].codebook, cb)
        np.testing.assert_array_equal(s.chunks[0][h].ids, ids)
