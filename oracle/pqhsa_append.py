"""Float64 CPU oracle for appending new tokens to the IVF-PQ index.

TEST INFRASTRUCTURE.  Only the tests may import this module; the HIP path
shares no code with it.

What is computed, and where the pages say so.  The PQ-HSA page (rit.work
blog, "PQ-HSA long-context attention"), section "How approximate estimates
return the discarded context", sixth paragraph: once the prompt is processed
the index is built, and newer tokens are held outside it and added to it in
batches.  Section "Too early to change the architecture, a prototype can be
built", third paragraph: the cost of building and updating the index is one
of the things to measure.  The pages print no encoder; the reading taken here
is the standard IVF-PQ residual encoder that matches the key model the decode
step uses (k_hat = C[list] + concat_m B_m[code_m]):

  A1 list of token t  = argmin_c ||K_t - C_c||^2            (lowest c on ties)
  A2 code_m of token t = argmin_j ||r_t^(m) - B_m[j]||^2,    r_t = K_t - C[list_t]
                                                             (lowest j on ties)
  A3 the cluster mean over all indexed tokens of the cluster, updated
     incrementally: mu_c' = (n_c mu_c + sum of the new tokens' V) / (n_c + m_c)

Pins (tests/test_oracle_append_pins.py): brute force over explicit loops,
exact recovery of generating lists and codes for well-separated centroids
and zero-noise keys, the lower-index tie rule on planted equal distances, and
incremental means equal to the batch mean.
"""
from __future__ import annotations

import numpy as np

PQ_M = 16
PQ_DSUB = 8


def sq_dist(x: np.ndarray, c: np.ndarray) -> np.ndarray:
    """Squared Euclidean distances, x [n, d] against c [k, d] -> [n, k], float64."""
    x = np.asarray(x, np.float64)
    c = np.asarray(c, np.float64)
    # rows in batches, only to bound the [rows, k, d] temporary; every entry
    # is the same sum of squared differences
    out = np.empty((x.shape[0], c.shape[0]))
    rows = max(1, (1 << 23) // max(1, c.shape[0] * c.shape[1]))
    for r in range(0, x.shape[0], rows):
        out[r:r + rows] = ((x[r:r + rows, None, :] - c[None, :, :]) ** 2).sum(axis=-1)
    return out


def ivf_assign(K: np.ndarray, centroids: np.ndarray) -> np.ndarray:
    """A1: nearest centroid of each key (np.argmin returns the first minimum,
    i.e. the lowest cluster id on exact ties)."""
    return sq_dist(K, centroids).argmin(axis=1).astype(np.int64)


def pq_encode(R: np.ndarray, codebooks: np.ndarray) -> np.ndarray:
    """A2: per subspace m, the nearest codeword of the residual's m-th 8-dim
    slice (lowest codeword id on exact ties).  R [n, 128], codebooks [16, 256, 8]."""
    R = np.asarray(R, np.float64)
    n = R.shape[0]
    codes = np.zeros((n, PQ_M), np.int64)
    for m in range(PQ_M):
        codes[:, m] = sq_dist(R[:, m * PQ_DSUB:(m + 1) * PQ_DSUB], codebooks[m]).argmin(axis=1)
    return codes


def encode_tokens(K: np.ndarray, centroids: np.ndarray, codebooks: np.ndarray):
    """A1 then A2 for a batch of keys: (lists [n], codes [n, 16])."""
    K = np.asarray(K, np.float64)
    lists = ivf_assign(K, centroids)
    codes = pq_encode(K - np.asarray(centroids, np.float64)[lists], codebooks)
    return lists, codes


def append_means(mu_old: np.ndarray, n_old: np.ndarray, v_new: np.ndarray,
                 lists_new: np.ndarray, num_lists: int):
    """A3: incremental cluster means.  mu_old [L, d], n_old [L] counts,
    v_new [n, d] the new tokens' values, lists_new [n] their clusters.
    Returns (mu_new, n_new); empty clusters keep mean 0."""
    v_new = np.asarray(v_new, np.float64)
    add = np.zeros((num_lists, v_new.shape[1]))
    np.add.at(add, lists_new, v_new)
    m = np.bincount(lists_new, minlength=num_lists)
    n_new = n_old + m
    mu = np.zeros_like(add)
    nz = n_new > 0
    mu[nz] = (n_old[nz, None] * np.asarray(mu_old, np.float64)[nz] + add[nz]) / n_new[nz, None]
    return mu, n_new


def distance_gaps(K, centroids, codebooks, lists, codes):
    """For checking an encoder that decides in lower precision: how far the
    chosen list and codes are above the exact minimum distances (>= 0; 0 when
    the choice is an exact minimiser).  Returns (list_gap [n], code_gap [n, 16],
    list_min [n], code_min [n, 16])."""
    K = np.asarray(K, np.float64)
    dl = sq_dist(K, centroids)
    n = K.shape[0]
    lgap = dl[np.arange(n), lists] - dl.min(axis=1)
    R = K - np.asarray(centroids, np.float64)[lists]
    cgap = np.zeros((n, PQ_M))
    cmin = np.zeros((n, PQ_M))
    for m in range(PQ_M):
        dc = sq_dist(R[:, m * PQ_DSUB:(m + 1) * PQ_DSUB], codebooks[m])
        cgap[:, m] = dc[np.arange(n), codes[:, m]] - dc.min(axis=1)
        cmin[:, m] = dc.min(axis=1)
    return lgap, cgap, dl.min(axis=1), cmin


def bruteforce_encode(K, centroids, codebooks):
    """Pure-Python loops over every candidate, keeping the first minimum:
    the reference for the vectorised encoder on tiny inputs."""
    lists, codes = [], []
    for k in np.asarray(K, np.float64):
        best, bl = None, -1
        for c, cen in enumerate(np.asarray(centroids, np.float64)):
            dist = sum((float(a) - float(b)) ** 2 for a, b in zip(k, cen))
            if best is None or dist < best:
                best, bl = dist, c
        r = k - np.asarray(centroids, np.float64)[bl]
        code = []
        for m in range(len(codebooks)):
            sub = r[m * PQ_DSUB:(m + 1) * PQ_DSUB]
            bd, bj = None, -1
            for j, cw in enumerate(np.asarray(codebooks[m], np.float64)):
                dist = sum((float(a) - float(b)) ** 2 for a, b in zip(sub, cw))
                if bd is None or dist < bd:
                    bd, bj = dist, j
            code.append(bj)
        lists.append(bl)
        codes.append(code)
    return np.array(lists, np.int64), np.array(codes, np.int64)
