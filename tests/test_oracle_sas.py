"""Pins for the oracle's k-means smoothing (CPU only).

QVG explainer, "Sommario tecnico" 2.A: k-means over the token axis, then the
group mean is subtracted.  Pins: brute force and a library distance routine
for the assignment, closed forms for C = 1 and for noiseless prototypes, and
the Lloyd objective invariants.
"""
from fractions import Fraction

import numpy as np
import pytest
from scipy.spatial.distance import cdist

from oracle import numerics, sas
import synth


def _bf16_data(rng, T, d, scale=1.0):
    return numerics.round_to_bf16(rng.standard_normal((T, d)) * scale)


@pytest.mark.parametrize("T,C,d", [(1, 1, 8), (5, 16, 8), (200, 7, 16), (513, 32, 64)])
def test_assign_matches_bruteforce_and_cdist(T, C, d):
    rng = np.random.default_rng(T * 31 + C)
    x = _bf16_data(rng, T, d)
    c = _bf16_data(rng, C, d)
    ids = sas.assign(x, c)
    np.testing.assert_array_equal(ids, sas.assign_bruteforce(x, c))
    ref = np.argmin(cdist(x.astype(np.float64), c.astype(np.float64), "sqeuclidean"), axis=1)
    # cdist may break exact-arithmetic ties differently only when distances tie;
    # with continuous data the minimiser is unique
    np.testing.assert_array_equal(ids, ref)


def test_assign_ties_go_to_lowest_index():
    x = np.array([[0.0, 0.0], [1.0, 1.0], [2.0, 0.0]], np.float32)
    c = np.array([[1.0, 0.0], [-1.0, 0.0], [0.0, 1.0], [1.0, 0.0]], np.float32)
    # token 0 is at distance 1 from c0, c1, c2 -> 0; token 1 ties c0, c2, c3 -> 0;
    # token 2 ties c0 and c3 (distance 1) -> 0
    np.testing.assert_array_equal(sas.assign(x, c), [0, 0, 0])
    c2 = c[[1, 2, 0, 3]]
    np.testing.assert_array_equal(sas.assign(x, c2), [0, 1, 2])


def test_assign_near_ties_decided_by_exact_distance():
    # Two centroids whose distances to x differ by one part in 1e12: the screening
    # must hand both to the exact distance, which picks the truly closer one.
    x = np.array([[1.0, 0.0, 0.0, 0.0]], np.float32)
    base = np.float32(0.5)
    c = np.array([[base, 0.0, 0.0, 0.0], [1.0, 0.5, 0.0, 0.0]], np.float32)
    assert sas.assign(x, c)[0] == 0       # exact tie: distance 0.25 each -> lowest index
    c[1, 1] = np.nextafter(np.float32(0.5), np.float32(0))
    assert sas.assign(x, c)[0] == 1       # now strictly closer
    # gaps of 2**-40 and 2**-38 against distances of 0.25: far inside the
    # screening window, decided by the exact distance
    c = np.array([[0.5, 0.0, 0.0, 0.0], [1.0, 0.5, 2.0 ** -20, 0.0]], np.float32)
    assert sas.assign(x, c)[0] == 0
    c[0, 2] = 2.0 ** -19
    assert sas.assign(x, c)[0] == 1


def test_distance_seq_is_channel_ordered_fp64():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((50, 37)).astype(np.float32)
    c = rng.standard_normal((50, 37)).astype(np.float32)
    D = sas.distance_seq(x, c)
    for t in range(50):
        acc = 0.0
        for j in range(37):
            diff = float(x[t, j]) - float(c[t, j])
            acc = acc + diff * diff
        assert D[t] == acc


def test_single_cluster_is_global_mean():
    rng = np.random.default_rng(6)
    x = _bf16_data(rng, 300, 16, 3.0)
    ids, c = sas.kmeans(x, 1, 3, "bf16")
    assert np.all(ids == 0)
    mean = [sum(Fraction(float(v)) for v in x[:, j]) / 300 for j in range(16)]
    # the fp64 mean rounded once to bf16 equals the exact mean rounded to bf16
    # unless the exact mean sits within fp64 error of a bf16 midpoint
    exp = numerics.round_to_bf16(np.array([float(m) for m in mean]))
    np.testing.assert_array_equal(c[0], exp)


def test_noiseless_prototypes_recovered_exactly():
    rng = np.random.default_rng(7)
    P = numerics.round_to_bf16(rng.standard_normal((8, 32)) * 4)
    labels = np.tile(np.arange(8), 50)
    x = P[labels]
    ids, c = sas.kmeans(x, 8, 1, "bf16", init=P[::-1].copy())
    np.testing.assert_array_equal(c[ids], x)
    assert sas.objective(x, c, ids) == 0.0
    r0 = sas.centroid_residual(x, c, ids)
    assert np.all(r0 == 0)


def test_strided_init_and_tiny_T():
    x = np.arange(4 * 3, dtype=np.float32).reshape(4, 3)
    c = sas.strided_init(x, 16)
    np.testing.assert_array_equal(c, x[(np.arange(16) * 4) // 16])
    ids, cb = sas.kmeans(x, 16, 5, "f32")
    # duplicated initial centroids: each token goes to the lowest copy of itself
    np.testing.assert_array_equal(ids, [0, 4, 8, 12])
    np.testing.assert_array_equal(cb[ids], x)


def test_empty_cluster_keeps_previous_centroid():
    x = np.array([[0.0, 0.0], [0.1, 0.0], [5.0, 5.0]], np.float32)
    init = np.array([[0.0, 0.0], [100.0, 100.0], [5.0, 5.0]], np.float32)
    ids, c = sas.kmeans(x, 3, 2, "f32", init=init)
    np.testing.assert_array_equal(c[1], init[1])
    np.testing.assert_array_equal(ids, [0, 0, 2])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_lloyd_objective_invariants(dtype):
    cfg = synth.scaled(synth.TINY, tokens=1024)
    x = synth.kv_tokens(cfg, 0, 0, 0, 1024)[0].float().numpy()
    if dtype == "bf16":
        x = numerics.round_to_bf16(x)
    trace = []
    sas.kmeans(x, 16, 6, dtype, trace=trace)
    prev_after = None
    for j_before, j_after, j_exact, c_next, counts in trace:
        # the exact mean minimises the within-cluster sum of squares
        assert j_exact <= j_before * (1 + 1e-12)
        # rounding the mean costs exactly sum_k n_k ||c_rnd - mean||^2
        assert j_after >= j_exact * (1 - 1e-12)
        # re-assignment never increases the objective
        if prev_after is not None:
            assert j_before <= prev_after * (1 + 1e-12)
        prev_after = j_after
    if dtype == "f32":
        # fp32 rounding of the means is negligible: monotone to 1e-6
        js = [t[0] for t in trace]
        assert all(b <= a * (1 + 1e-6) for a, b in zip(js, js[1:]))


def test_rounding_slack_identity():
    rng = np.random.default_rng(8)
    x = _bf16_data(rng, 400, 16, 2.0)
    trace = []
    sas.kmeans(x, 5, 1, "bf16", trace=trace)
    _, j_after, j_exact, c_next, counts = trace[0]
    ids = sas.assign(x, sas.strided_init(x, 5))
    x64 = x.astype(np.float64)
    slack = 0.0
    for k in range(5):
        if counts[k]:
            mean = x64[ids == k].mean(axis=0)
            slack += counts[k] * np.sum((c_next[k].astype(np.float64) - mean) ** 2)
    assert j_after == pytest.approx(j_exact + slack, rel=1e-10)


def test_update_sums_in_token_order():
    # sum order matters in fp64 for these values; the oracle adds in token order
    x = np.array([[1.0], [2.0 ** -60], [-1.0], [2.0 ** -60]], np.float32)
    ids = np.array([0, 0, 0, 0])
    c, _ = sas.update(x, ids, np.zeros((1, 1), np.float32), "f32")
    seq = ((1.0 + 2.0 ** -60) + -1.0) + 2.0 ** -60
    assert c[0, 0] == np.float32(seq / 4)
