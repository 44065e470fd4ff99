"""Pins of the query-reuse oracle (oracle/pqhsa_reuse.py) against facts that
do not depend on it: full softmax attention from torch's own routine, the
prefix/suffix identity on exact and orthogonal reuse, planted distances for
the window, threshold and tie rules, explicit-loop search, and the ring's
replacement order."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import pqhsa_reuse as ru  # noqa: E402
from pqhsa_synth.gen import bf16_bits_to_f32, f32_to_bf16_bits  # noqa: E402

SCALE = 1.0 / np.sqrt(128.0)


def _bits(x):
    return f32_to_bf16_bits(np.asarray(x, np.float32))


def _kv(seed, B, Hkv, T, zero_dim=None, zero_upto=0):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((B, Hkv, T, 128)).astype(np.float32)
    V = rng.standard_normal((B, Hkv, T, 128)).astype(np.float32)
    if zero_dim is not None:
        K[:, :, :zero_upto, zero_dim] = 0.0
    return _bits(K), _bits(V)


def _sdpa(q_bits, k_bits, v_bits, T):
    """Full attention of one query over rows [0, T) through torch (float64)."""
    q = torch.from_numpy(bf16_bits_to_f32(q_bits).astype(np.float64))[None, None, None, :]
    K = torch.from_numpy(bf16_bits_to_f32(k_bits[:T]).astype(np.float64))[None, None]
    V = torch.from_numpy(bf16_bits_to_f32(v_bits[:T]).astype(np.float64))[None, None]
    O = torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=SCALE)[0, 0, 0].numpy()
    lse = torch.logsumexp(SCALE * (K[0, 0] @ q[0, 0, 0]), dim=0).item()
    return O, lse


def _q(seed, B, Hq):
    rng = np.random.default_rng(seed)
    return _bits(rng.standard_normal((B, Hq, 128))), _bits(rng.standard_normal((B, Hq, 128)))


def test_empty_buffer_falls_back_to_full_attention():
    B, Hq, Hkv = 2, 4, 2
    k, v = _kv(1, B, Hkv, 60)
    q, qs = _q(2, B, Hq)
    ctx = np.array([50, 37])
    buf = ru.new_buffer(B, Hq, 16)
    r = ru.reuse_step(buf, q, qs, k, v, ctx, SCALE, max_dist2=1e9)
    assert np.all(r["slot"] == -1) and np.all(np.isinf(r["d2"])) and np.all(r["start"] == 0)
    for b in range(B):
        for hq in range(Hq):
            O, lse = _sdpa(q[b, hq], k[b, hq // 2], v[b, hq // 2], ctx[b])
            np.testing.assert_allclose(r["O"][b, hq], O, rtol=1e-12, atol=1e-12)
            assert abs(r["lse"][b, hq] - lse) < 1e-12
    assert np.all(buf.cnt == 1) and np.all(buf.tj[:, :, 0] == ctx[:, None])


def test_identical_query_reuse_equals_full_attention():
    # an entry computed exactly at T1 and reused by the same query at T2
    # gives full attention over [0, T2): the prefix is [0, T1), the suffix
    # [T1, T2), with no token dropped or counted twice
    B, Hq, Hkv = 1, 2, 1
    k, v = _kv(3, B, Hkv, 80)
    q, qs = _q(4, B, Hq)
    buf = ru.new_buffer(B, Hq, 64)
    ru.reuse_step(buf, q, qs, k, v, np.array([41]), SCALE, max_dist2=0.0)
    r = ru.reuse_step(buf, q, qs, k, v, np.array([77]), SCALE, max_dist2=0.0)
    assert np.all(r["slot"] == 0) and np.all(r["d2"] == 0.0) and np.all(r["start"] == 41)
    for hq in range(Hq):
        O, lse = _sdpa(q[0, hq], k[0, 0], v[0, 0], 77)
        np.testing.assert_allclose(r["O"][0, hq], O, rtol=1e-12, atol=1e-12)
        assert abs(r["lse"][0, hq] - lse) < 1e-12


def test_chained_reuse_of_identical_queries_stays_exact():
    # each step reuses the previous step's entry, itself a reused state
    B, Hq, Hkv = 1, 2, 1
    k, v = _kv(5, B, Hkv, 90)
    q, qs = _q(6, B, Hq)
    buf = ru.new_buffer(B, Hq, 40)
    for i, T in enumerate([10, 11, 15, 30, 31, 62, 90]):
        r = ru.reuse_step(buf, q, qs, k, v, np.array([T]), SCALE, max_dist2=0.0)
        assert np.all(r["slot"] == (-1 if i == 0 else i - 1))
        for hq in range(Hq):
            O, _ = _sdpa(q[0, hq], k[0, 0], v[0, 0], T)
            np.testing.assert_allclose(r["O"][0, hq], O, rtol=1e-11, atol=1e-12)


def test_reuse_across_a_query_change_orthogonal_to_the_prefix_is_exact():
    # the old and new attention queries differ only in dim 5, where every
    # prefix key is 0: the prefix scores agree, so reuse is exact, while the
    # suffix (dim 5 non-zero) must be scored with the new query
    B, Hq, Hkv = 1, 1, 1
    T1, T2 = 33, 70
    k, v = _kv(7, B, Hkv, T2, zero_dim=5, zero_upto=T1)
    q1, qs = _q(8, B, Hq)
    q2 = q1.copy()
    q2[0, 0, 5:6] = _bits(bf16_bits_to_f32(q1[0, 0, 5:6]) + 1.5)
    buf = ru.new_buffer(B, Hq, 64)
    ru.reuse_step(buf, q1, qs, k, v, np.array([T1]), SCALE, max_dist2=0.0)
    r = ru.reuse_step(buf, q2, qs, k, v, np.array([T2]), SCALE, max_dist2=0.0)
    assert r["slot"][0, 0] == 0
    O, lse = _sdpa(q2[0, 0], k[0, 0], v[0, 0], T2)
    np.testing.assert_allclose(r["O"][0, 0], O, rtol=1e-12, atol=1e-12)
    assert abs(r["lse"][0, 0] - lse) < 1e-12
    # and the suffix really depends on the new query
    O_old, _ = _sdpa(q1[0, 0], k[0, 0], v[0, 0], T2)
    assert np.abs(O - O_old).max() > 1e-3


def _planted_buffer(W, entries):
    """Ring of one head with entries (slot, T_j, search vector)."""
    buf = ru.new_buffer(1, 1, W)
    for w, t, x in entries:
        buf.qs[0, 0, w] = x
        buf.tj[0, 0, w] = t
        buf.m[0, 0, w], buf.Dn[0, 0, w] = 0.0, 1.0
    buf.cnt[0, 0] = len(entries)
    return buf


def test_threshold_decides_between_reuse_and_full_attention():
    x = np.zeros(128)
    y = x.copy()
    y[:4] = 0.5                                       # d2 = 4 * 0.25 = 1 exactly
    k, v = _kv(9, 1, 1, 40)
    q = _bits(np.random.default_rng(10).standard_normal((1, 1, 128)))
    for thr, expect in [(0.999, -1), (1.0, 0)]:
        buf = _planted_buffer(8, [(0, 25, y)])
        r = ru.reuse_step(buf, q, _bits(x[None, None]), k, v, np.array([30]), SCALE, thr)
        assert r["d2"][0, 0] == 1.0 and r["slot"][0, 0] == expect
        if expect < 0:
            O, _ = _sdpa(q[0, 0], k[0, 0], v[0, 0], 30)
            np.testing.assert_allclose(r["O"][0, 0], O, rtol=1e-12, atol=1e-12)
        else:
            assert r["start"][0, 0] == 25


def test_window_and_position_rules():
    x = np.zeros(128)
    near, mid, far = x.copy(), x.copy(), x.copy()
    near[0], mid[0], far[0] = 0.25, 0.5, 1.0
    # at T = 30 with W = 8: T_j = 23 is the oldest eligible (30 - 23 < 8);
    # T_j = 22 is outside the window; T_j = 31 lies ahead of T; 0 is empty
    buf = _planted_buffer(8, [(0, 22, near), (1, 31, near), (2, 23, far), (3, 29, mid)])
    assert ru.nearest_entry(buf, 0, 0, x, 30) == (3, 0.25)
    buf.tj[0, 0, 3] = 0
    assert ru.nearest_entry(buf, 0, 0, x, 30) == (2, 1.0)
    buf.tj[0, 0, 2] = 0
    assert ru.nearest_entry(buf, 0, 0, x, 30) == (-1, np.inf)
    assert ru.nearest_entry(buf, 0, 0, x, 31) == (1, 0.0625)   # T_j = T is eligible
    assert ru.nearest_entry(buf, 0, 0, x, 28) == (0, 0.0625)


def test_ties_prefer_the_more_recent_entry_then_the_lower_slot():
    x = np.zeros(128)
    y = x.copy()
    y[7] = 0.5
    buf = _planted_buffer(8, [(0, 20, y), (1, 25, y), (2, 25, y), (5, 24, y)])
    assert ru.nearest_entry(buf, 0, 0, x, 30) == (1, 0.25)
    buf.tj[0, 0, 1] = 0
    assert ru.nearest_entry(buf, 0, 0, x, 30) == (2, 0.25)


@pytest.mark.parametrize("seed", range(6))
def test_search_matches_explicit_loops(seed):
    rng = np.random.default_rng(seed)
    W, T = 7, 40
    buf = ru.new_buffer(1, 1, W)
    base = rng.integers(-4, 5, (3, 128)) / 4.0        # few distinct vectors: exact ties
    for w in range(W):
        buf.qs[0, 0, w] = base[rng.integers(0, 3)]
        buf.tj[0, 0, w] = rng.choice([0, 30, 34, 34, 39, 40, 41])
    for _ in range(5):
        x = base[rng.integers(0, 3)] + rng.integers(-1, 2, 128) / 4.0
        assert ru.nearest_entry(buf, 0, 0, x, T) == ru.bruteforce_nearest(
            buf.qs[0, 0], buf.tj[0, 0], W, x, T)


def test_ring_replaces_the_oldest_entry():
    B, Hq, Hkv, W = 1, 1, 1, 3
    k, v = _kv(11, B, Hkv, 20)
    buf = ru.new_buffer(B, Hq, W)
    rng = np.random.default_rng(12)
    Ts = [5, 8, 9, 13, 17]
    for T in Ts:
        q = _bits(rng.standard_normal((1, 1, 128)))
        ru.reuse_step(buf, q, q, k, v, np.array([T]), SCALE, max_dist2=-1.0)
    assert buf.cnt[0, 0] == 5
    assert list(buf.tj[0, 0]) == [13, 17, 9]
