"""Pins of the index-append oracle (oracle/pqhsa_append.py) against facts that
do not depend on it: explicit loops, exact recovery of planted structure, the
tie rule, and the mean of all tokens at once."""
import numpy as np
import pytest

from oracle import pqhsa_append as ap
from pqhsa_synth.gen import draw_head


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_encoder_matches_bruteforce_loops(seed):
    rng = np.random.default_rng(seed)
    L, n = 6, 5
    C = rng.standard_normal((L, 128))
    B = rng.standard_normal((16, 256, 8)) * 0.3
    K = C[rng.integers(0, L, n)] + rng.standard_normal((n, 128)) * 0.4
    lists, codes = ap.encode_tokens(K, C, B)
    bl, bc = ap.bruteforce_encode(K, C, B)
    assert np.array_equal(lists, bl) and np.array_equal(codes, bc)


def test_zero_noise_keys_recover_their_lists_and_codes():
    # dyadic centroids far apart and small dyadic codewords: each key
    # C[l] + concat B[code] is nearest to its own centroid (the residual is
    # tiny next to the centroid spacing) and its residual equals its
    # codewords exactly (distance 0, codewords distinct)
    rng = np.random.default_rng(3)
    L, n = 16, 200
    C = rng.integers(-60, 61, (L, 128)).astype(np.float64) / 4.0
    B = np.stack([rng.permutation(256)[:, None] * 2.0 ** -9 + np.arange(8) * 2.0 ** -3
                  for _ in range(16)])
    lists = rng.integers(0, L, n)
    codes = rng.integers(0, 256, (n, 16))
    K = C[lists] + np.concatenate([B[m][codes[:, m]] for m in range(16)], axis=1)
    gl, gc = ap.encode_tokens(K, C, B)
    assert np.array_equal(gl, lists)
    assert np.array_equal(gc, codes)


def test_exact_ties_go_to_the_lower_index():
    C = np.zeros((4, 128))
    C[1, 0], C[3, 0] = 1.0, -1.0          # clusters 1 and 3 equidistant from the origin
    C[0, 0] = C[2, 0] = 5.0
    K = np.zeros((1, 128))
    assert ap.ivf_assign(K, C)[0] == 1
    B = np.zeros((16, 256, 8))
    B[:, 7, 0], B[:, 3, 0] = 2.0, -2.0    # codewords 3 and 7 equidistant, others farther
    B[:, [i for i in range(256) if i not in (3, 7)], 0] = 9.0
    codes = ap.pq_encode(np.zeros((1, 128)), B)
    assert np.all(codes == 3)


def test_incremental_means_equal_the_batch_mean():
    rng = np.random.default_rng(4)
    L, n0, n1 = 7, 300, 45
    V = rng.standard_normal((n0 + n1, 128))
    lists = rng.integers(0, L, n0 + n1)
    lists[:n0][lists[:n0] == 5] = 4            # cluster 5 empty before the append
    mu0 = np.zeros((L, 128))
    cnt0 = np.bincount(lists[:n0], minlength=L)
    for c in range(L):
        if cnt0[c]:
            mu0[c] = V[:n0][lists[:n0] == c].mean(axis=0)
    mu1, cnt1 = ap.append_means(mu0, cnt0, V[n0:], lists[n0:], L)
    for c in range(L):
        sel = lists == c
        ref = V[sel].mean(axis=0) if sel.any() else np.zeros(128)
        np.testing.assert_allclose(mu1[c], ref, atol=1e-12)
    assert np.array_equal(cnt1, np.bincount(lists, minlength=L))


def test_append_to_empty_cluster_set_is_the_batch_mean():
    rng = np.random.default_rng(5)
    V = rng.standard_normal((10, 128))
    lists = np.array([0, 2, 2, 0, 1, 1, 1, 0, 2, 0])
    mu, cnt = ap.append_means(np.zeros((4, 128)), np.zeros(4, np.int64), V, lists, 4)
    for c in range(3):
        np.testing.assert_allclose(mu[c], V[lists == c].mean(axis=0), atol=1e-12)
    assert np.all(mu[3] == 0) and cnt[3] == 0


def test_distance_gaps_are_zero_for_the_oracle_choice_and_positive_otherwise():
    d = draw_head(7, 0, 0, 64, 8)
    K = d.k_bits.astype(np.uint32) << 16
    K = K.view(np.float32).astype(np.float64)
    lists, codes = ap.encode_tokens(K, d.centroids, d.codebooks)
    lg, cg, _, _ = ap.distance_gaps(K, d.centroids, d.codebooks, lists, codes)
    assert np.all(lg == 0) and np.all(cg == 0)
    wrong = (lists + 1) % 8
    lg2, _, _, _ = ap.distance_gaps(K, d.centroids, d.codebooks, wrong, codes)
    assert np.all(lg2 > 0)


def test_synthetic_keys_mostly_recover_their_generating_lists():
    # the workload key model (centroid + codewords + small noise) keeps most
    # keys nearest to the centroid they were drawn from
    d = draw_head(0, 0, 0, 2000, 64)
    K = (d.k_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    lists = ap.ivf_assign(K, d.centroids)
    assert np.mean(lists == d.list_ids) > 0.9
