"""Semantic-Aware Smoothing: k-means over the token axis (test infrastructure only).

QVG explainer, "Sommario tecnico" 2.A: tokens of one head are grouped with
k-means along the sequence-length axis by similarity in latent space; each
group's mean (centroid) is computed and subtracted from its tokens, leaving
small residuals concentrated near zero.  Section 3 adds centroid caching to
speed the clustering up.

Readings of what the page leaves open (one head, one tensor K or V):

* distance: squared Euclidean D(t, k) = sum_j (x[t, j] - c[k, j])**2, each
  term and each partial sum rounded to fp64, summed in channel order
  j = 0 .. d-1 (``distance_seq``).  Ties go to the lowest cluster index.
* initialisation: the stream's cached codebook when there is one (centroid
  caching); otherwise c[k] = x[floor(k * T / C)] for k = 0 .. C-1.
* Lloyd iterations: ``iters`` times (assign, then update), then a final
  assignment against the final codebook; those ids and that codebook are
  what gets stored.
* update: c[k] = round_to_dtype(S_k / n_k) where S_k is the fp64 sum of the
  member tokens taken in token order and the division is in fp64; the
  cache dtype is bf16 (or fp32 when the cache is fp32).  An empty cluster
  keeps its previous centroid.
* centroid subtraction: r0 = fl32(x - c[id]).
"""
import numpy as np

from .numerics import round_to_bf16


def strided_init(x, n_clusters):
    """Initial codebook: token floor(k*T/C) for cluster k (duplicates allowed)."""
    T = x.shape[0]
    rows = (np.arange(n_clusters, dtype=np.int64) * T) // n_clusters
    return x[rows].copy()


def distance_seq(x_rows, c_rows):
    """D for paired rows: fp64 squared differences accumulated in channel order."""
    x64 = np.asarray(x_rows, dtype=np.float64)
    c64 = np.asarray(c_rows, dtype=np.float64)
    D = np.zeros(x64.shape[0], dtype=np.float64)
    for j in range(x64.shape[1]):
        diff = x64[:, j] - c64[:, j]
        D = D + diff * diff
    return D


def assign_bruteforce(x, c):
    """argmin_k D(t, k) over every (t, k) pair; ties to the lowest k.

    Plain definition, O(T*C*d) Python-visible work; for small inputs.
    """
    T, C = x.shape[0], c.shape[0]
    tt = np.repeat(np.arange(T), C)
    kk = np.tile(np.arange(C), T)
    D = distance_seq(x[tt], c[kk]).reshape(T, C)
    return np.argmin(D, axis=1)   # np.argmin returns the first (lowest) minimum


def assign(x, c, block=8192):
    """Same result as ``assign_bruteforce`` at scale.

    A fp64 expanded-form score ||c||^2 - 2 x.c (BLAS) selects, per token, every
    cluster whose score is within 1e-9 * (||x||^2 + max ||c||^2) of the best;
    the BLAS error is below 1e-13 of that scale, so the exact minimiser of D is
    always among them.  ``distance_seq`` then decides among the candidates,
    ties to the lowest index.
    """
    x64 = np.asarray(x, dtype=np.float64)
    c64 = np.asarray(c, dtype=np.float64)
    T, C = x64.shape[0], c64.shape[0]
    cn = np.einsum("kd,kd->k", c64, c64)
    cmax = cn.max() if C else 0.0
    ids = np.empty(T, dtype=np.int64)
    for t0 in range(0, T, block):
        xb = x64[t0:t0 + block]
        s = cn[None, :] - 2.0 * (xb @ c64.T)
        xn = np.einsum("td,td->t", xb, xb)
        win = 1e-9 * (xn + cmax) + 1e-300
        smin = s.min(axis=1)
        cand_t, cand_k = np.nonzero(s <= (smin + 2.0 * win)[:, None])
        D = distance_seq(xb[cand_t], c64[cand_k])
        # lowest D per token, then lowest k among equal D: sort by (t, D, k)
        order = np.lexsort((cand_k, D, cand_t))
        first = np.ones(order.size, dtype=bool)
        first[1:] = cand_t[order][1:] != cand_t[order][:-1]
        sel = order[first]
        ids[t0 + cand_t[sel]] = cand_k[sel]
    return ids


def round_to_dtype(v64, dtype):
    """Round fp64 centroid means once to the cache dtype ('bf16' or 'f32')."""
    if dtype == "bf16":
        return round_to_bf16(v64)
    if dtype == "f32":
        return np.asarray(v64, dtype=np.float64).astype(np.float32)
    raise ValueError(dtype)


def update(x, ids, c_prev, dtype):
    """M-step: fp64 sum of members in token order, fp64 divide, one rounding.

    Empty clusters keep ``c_prev``.  Returns the new codebook (float32 array
    holding dtype-representable values) and the member counts.
    """
    x64 = np.asarray(x, dtype=np.float64)
    C = c_prev.shape[0]
    c_new = np.array(c_prev, dtype=np.float32, copy=True)
    counts = np.bincount(ids, minlength=C)
    order = np.argsort(ids, kind="stable")      # token order kept inside a cluster
    starts = np.concatenate([[0], np.cumsum(counts)])
    for k in range(C):
        n = counts[k]
        if n == 0:
            continue
        members = order[starts[k]:starts[k + 1]]
        s = np.cumsum(x64[members], axis=0)[-1]  # sequential accumulation, token order
        c_new[k] = round_to_dtype(s / np.float64(n), dtype)
    return c_new, counts


def objective(x, c, ids):
    """k-means objective J = sum_t D(t, id_t) in fp64."""
    return float(np.sum(distance_seq(x, c[ids])))


def kmeans(x, n_clusters, iters, dtype, init=None, trace=None):
    """Lloyd's k-means as read from the QVG explainer's SAS step.

    ``init`` is the cached codebook of this stream (warm start) or None for the
    strided initialisation.  Returns (ids, codebook).  When ``trace`` is a
    list, each iteration appends (J before update, J after update, J with the
    exact unrounded means) so the tests can check the objective.
    """
    x = np.asarray(x, dtype=np.float32)
    c = strided_init(x, n_clusters) if init is None else np.array(init, dtype=np.float32)
    if c.shape != (n_clusters, x.shape[1]):
        raise ValueError("codebook shape mismatch")
    for _ in range(iters):
        ids = assign(x, c)
        c_next, counts = update(x, ids, c, dtype)
        if trace is not None:
            x64 = x.astype(np.float64)
            exact = np.array(c, dtype=np.float64)
            for k in np.nonzero(counts)[0]:
                exact[k] = x64[ids == k].mean(axis=0)
            trace.append((objective(x, c, ids), objective(x, c_next, ids),
                          float(np.sum(distance_seq(x64, exact[ids]))), c_next, counts))
        c = c_next
    ids = assign(x, c)
    return ids, c


def centroid_residual(x, c, ids):
    """r0 = fl32(x - c[id]) (IEEE fp32 subtraction)."""
    return np.asarray(x, dtype=np.float32) - np.asarray(c, dtype=np.float32)[ids]
