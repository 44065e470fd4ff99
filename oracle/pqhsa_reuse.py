"""Float64 CPU oracle for decode attention with query reuse.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the HIP path shares no code with it.

What is computed, and where the pages say so.  "The query-reuse post" is the
quant_prune_distill Telegram post on reusing attention across close queries.

  * Opening paragraph: split the context into a prefix P and a suffix S; the
    attention output is O = (N_P + N_S) / (D_P + D_S), N the unnormalised
    numerator and D the denominator.  When an earlier query is close enough
    to the current one, the numerator and denominator precomputed for that
    query are reused, and only the terms between that query's position and
    the current position are computed.
  * Section "Important practical considerations": a small sliding buffer of
    queries is kept (a full query cache would cost more than the KV cache
    under GQA and MLA; reuse pays more the closer the reused query is in
    position).  Closeness is the L2 distance between pre-RoPE vectors; when
    the smallest distance is above a threshold, standard attention is
    computed instead.
  * Section "Experiments": the nearest query is searched among the last 1024
    tokens; the threshold was tuned by hand (no value is given).

Readings where the post is silent or ambiguous (each a choice, stated once):
  Q1 the compared vectors: the post speaks of pre-RoPE keys while comparing
     queries; the reading is the current query's pre-RoPE vector against the
     buffered queries' pre-RoPE vectors.  The caller passes it as q_search,
     separately from the attention query q.
  Q2 every query head keeps its own ring of entries and decides on its own.
  Q3 a ring has W slots, one entry per step; an entry inserted at context
     length T_j is eligible at context length T when 1 <= T_j <= T and
     T - T_j < W (it is the query of one of the last W tokens).
  Q4 an entry's state covers the context it was computed on, [0, T_j); the
     suffix computed now is [T_j, T).
  Q5 closeness is the squared L2 distance d2; reuse when the smallest d2 is
     <= max_dist2, a caller parameter.
  Q6 equal distances go to the more recent entry (larger T_j, more reuse),
     then to the lower slot.
  Q7 every step inserts its search vector and the state it produced (reused
     or full) into slot (count mod W) of its head's ring, replacing the
     oldest entry.

States are kept as (m, N, D) with natural-log maxima: N = sum_t e^{s_t - m} V_t,
D = sum_t e^{s_t - m}, s_t = scale * q . K_t; O = N / D, lse = m + ln D.

Pins (tests/test_oracle_reuse_pins.py): full attention through an independent
library routine when nothing is reused; exact reuse of an identical earlier
query equals full attention (the prefix/suffix identity); reuse across a
query change orthogonal to every prefix key is exact; window, threshold and
tie rules on planted entries; brute-force search by explicit loops; the
ring's replacement order.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .pqhsa_oracle import bf16_to_f64, partial_attention


@dataclass
class ReuseBuffer:
    """Per (sequence, query head) rings of W entries (Q2, Q3, Q7)."""
    W: int
    qs: np.ndarray     # [B, Hq, W, D]   search vectors
    m: np.ndarray      # [B, Hq, W]      state maxima (natural log)
    N: np.ndarray      # [B, Hq, W, D]   state numerators
    Dn: np.ndarray     # [B, Hq, W]      state denominators
    tj: np.ndarray     # [B, Hq, W]      context length at insertion, 0 = empty
    cnt: np.ndarray    # [B, Hq]         entries inserted so far


def new_buffer(batch: int, num_q_heads: int, window: int, head_dim: int = 128) -> ReuseBuffer:
    return ReuseBuffer(window,
                       np.zeros((batch, num_q_heads, window, head_dim)),
                       np.full((batch, num_q_heads, window), -np.inf),
                       np.zeros((batch, num_q_heads, window, head_dim)),
                       np.zeros((batch, num_q_heads, window)),
                       np.zeros((batch, num_q_heads, window), np.int64),
                       np.zeros((batch, num_q_heads), np.int64))


def eligible(buf: ReuseBuffer, b: int, hq: int, T: int) -> np.ndarray:
    """Q3: slots whose entry may be reused at context length T."""
    tj = buf.tj[b, hq]
    return np.nonzero((tj >= 1) & (tj <= T) & (T - tj < buf.W))[0]


def sq_dists(buf: ReuseBuffer, b: int, hq: int, q_search: np.ndarray) -> np.ndarray:
    """Q5: squared L2 distance of q_search to every slot's search vector."""
    return ((buf.qs[b, hq] - np.asarray(q_search, np.float64)[None, :]) ** 2).sum(axis=1)


def nearest_entry(buf: ReuseBuffer, b: int, hq: int, q_search: np.ndarray, T: int):
    """The closest eligible entry: (slot, d2), or (-1, inf) when none is
    eligible.  Ties go to the larger T_j, then to the lower slot (Q6)."""
    cand = eligible(buf, b, hq, T)
    if cand.size == 0:
        return -1, np.inf
    d2 = sq_dists(buf, b, hq, q_search)[cand]
    order = np.lexsort((cand, -buf.tj[b, hq, cand], d2))
    best = cand[order[0]]
    return int(best), float(d2[order[0]])


def merge_states(parts):
    """(m, N, D) parts -> one (m, N, D): the prefix/suffix law generalised,
    N = sum_i e^{m_i - M} N_i, D = sum_i e^{m_i - M} D_i with M = max_i m_i.
    Empty parts (m = -inf) contribute nothing."""
    M = max(p[0] for p in parts)
    if M == -np.inf:
        return -np.inf, np.zeros_like(parts[0][1]), 0.0
    N = sum(np.exp(p[0] - M) * p[1] for p in parts if p[0] != -np.inf)
    D = sum(np.exp(p[0] - M) * p[2] for p in parts if p[0] != -np.inf)
    return M, N, D


def reuse_step(buf: ReuseBuffer, q_bits, qs_bits, k_bits, v_bits, context_lens, scale: float,
               max_dist2: float, choices=None, insert: bool = True):
    """One decode step with query reuse for a batch; updates buf in place.

    q_bits, qs_bits: [B, Hq, D] bf16 bits of the attention and search vectors;
    k_bits, v_bits: [B, Hkv, Tmax, D] bf16 bits of the logical K/V rows;
    context_lens: [B].  choices (optional) [B, Hq] overrides the slot each
    head reuses (-1: none); the tests pass the device's decision where it sits
    within float32 rounding of a tie or of the threshold.

    Returns dict(O [B, Hq, D], lse [B, Hq], slot [B, Hq], d2 [B, Hq],
    start [B, Hq]) where slot is the reused slot or -1, d2 the smallest
    eligible squared distance (inf if none) and start the first position
    computed at this step.
    """
    q = bf16_to_f64(q_bits)
    qs = bf16_to_f64(qs_bits)
    B, Hq, D = q.shape
    Hkv = k_bits.shape[1]
    G = Hq // Hkv
    O = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    slot = np.full((B, Hq), -1, np.int64)
    d2 = np.full((B, Hq), np.inf)
    start = np.zeros((B, Hq), np.int64)
    new_states = []
    for b in range(B):
        T = int(context_lens[b])
        for hq in range(Hq):
            h = hq // G
            j, dj = nearest_entry(buf, b, hq, qs[b, hq], T)
            d2[b, hq] = dj
            if choices is not None:
                j = int(choices[b, hq])
            elif not (j >= 0 and dj <= max_dist2):
                j = -1
            slot[b, hq] = j
            s0 = int(buf.tj[b, hq, j]) if j >= 0 else 0
            start[b, hq] = s0
            K = bf16_to_f64(k_bits[b, h, s0:T])
            V = bf16_to_f64(v_bits[b, h, s0:T])
            m_s, N_s, D_s = partial_attention(q[b, hq][None, :], K, V, scale)
            parts = [(float(m_s[0]), N_s[0], float(D_s[0]))]
            if j >= 0:
                parts.append((float(buf.m[b, hq, j]), buf.N[b, hq, j].copy(),
                              float(buf.Dn[b, hq, j])))
            M, N, Dn = merge_states(parts)
            O[b, hq] = N / Dn if Dn > 0 else 0.0
            lse[b, hq] = M + np.log(Dn) if Dn > 0 else -np.inf
            new_states.append((b, hq, T, M, N, Dn))
    if insert:
        for b, hq, T, M, N, Dn in new_states:
            w = int(buf.cnt[b, hq] % buf.W)
            buf.qs[b, hq, w] = qs[b, hq]
            buf.m[b, hq, w], buf.N[b, hq, w], buf.Dn[b, hq, w] = M, N, Dn
            buf.tj[b, hq, w] = T
            buf.cnt[b, hq] += 1
    return dict(O=O, lse=lse, slot=slot, d2=d2, start=start)


def bruteforce_nearest(qs_ring, tj_ring, W: int, q_search, T: int):
    """Explicit loops over one ring: the first slot with the strictly smallest
    distance, preferring the larger T_j on equal distances (tiny inputs)."""
    best, best_d, best_t = -1, None, None
    for w in range(len(tj_ring)):
        t = int(tj_ring[w])
        if not (1 <= t <= T and T - t < W):
            continue
        d = 0.0
        for x, y in zip(q_search, qs_ring[w]):
            d += (float(x) - float(y)) ** 2
        if best_d is None or d < best_d or (d == best_d and t > best_t):
            best, best_d, best_t = w, d, t
    return best, (np.inf if best_d is None else best_d)
