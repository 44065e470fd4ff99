"""Seeded synthetic workloads shaped like the PQ-HSA evaluation setups.

The PQ-HSA page (rit.work blog, "PQ-HSA long-context attention") measures on
Llama-3.1-8B-Instruct and Qwen3-30B-A3B (section "The background contribution
kept accuracy, and length gave the speed-up").  No weights or datasets are
used here: the workloads below copy those models' attention shapes (query
heads, KV heads, head_dim 128, paged bf16 cache with 16-token pages) and fill
them with seeded random data whose keys follow an IVF-PQ key model, so that
the index and the cache agree the way an index built after prefill would.

Recipe for one (sequence b, KV head h), rng = default_rng([workload_id, b, h]):
  centroids  C  = 0.5 * N(0,1) of shape (L, 128), float32
  codebooks  B  = 0.3 * N(0,1) of shape (16, 256, 8), float32
  list ids      = uniform integers in [0, L), shape (T,)
  codes         = uniform integers in [0, 256), shape (T, 16), uint8
  keys       K  = bf16( C[list_t] + concat_m B[m, code_t,m] + noise * N(0,1) )
  values     V  = bf16( N(0,1) ), shape (T, 128)
Query for sequence b, rng = default_rng([workload_id, b]):
  planted positions: one uniform draw in each of n_planted equal strata of
  [n_sink, T - max(n_recent, n_tail)); then for h = 0..Hkv-1 and each of the
  G query heads g of that KV head:
  q_g = bf16( N(0,1)^128 + 3 * sum_p K_h[p] / ||K_h[p]|| ).
Physical pages: a seeded permutation of the page pool fills the block table.
Draws are float32 (standard_normal(dtype=float32) times the stated sigma).
All of a sequence's T tokens get lists and codes; only the first n_indexed
of them are handed to the index, the rest form the unindexed tail.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

HEAD_DIM = 128
PAGE_SIZE = 16
PQ_M = 16
PQ_KSUB = 256
PQ_DSUB = HEAD_DIM // PQ_M

# Workloads: attention shapes of the pages' models at their context lengths.
WORKLOADS = {
    0: dict(name="tiny-8k", batch=1, num_q_heads=4, num_kv_heads=1, context=8192,
            num_lists=64, n_sink=4, n_recent=64, n_tail=0, budget_bp=100, n_planted=4),
    1: dict(name="llama3.1-8b-32k", batch=1, num_q_heads=32, num_kv_heads=8, context=32768,
            num_lists=256, n_sink=4, n_recent=128, n_tail=256, budget_bp=100, n_planted=16),
    2: dict(name="llama3.1-8b-128k", batch=1, num_q_heads=32, num_kv_heads=8, context=131072,
            num_lists=512, n_sink=4, n_recent=128, n_tail=256, budget_bp=100, n_planted=16),
    3: dict(name="llama3.1-8b-128k-batch16", batch=16, num_q_heads=32, num_kv_heads=8,
            context=131072, num_lists=512, n_sink=4, n_recent=128, n_tail=256, budget_bp=100,
            n_planted=16),
    4: dict(name="qwen3-30b-a3b-512k", batch=1, num_q_heads=32, num_kv_heads=4, context=524288,
            num_lists=1024, n_sink=4, n_recent=256, n_tail=512, budget_bp=100, n_planted=64),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class HeadDraw:
    """Random draws of one (sequence, KV head)."""
    centroids: np.ndarray   # (L, 128) float32
    codebooks: np.ndarray   # (16, 256, 8) float32
    list_ids: np.ndarray    # (T,) int32
    codes: np.ndarray       # (T, 16) uint8
    k_bits: np.ndarray      # (T, 128) uint16 (bf16)
    v_bits: np.ndarray      # (T, 128) uint16 (bf16)


def draw_head(workload_id: int, b: int, h: int, T: int, L: int, *, noise: float = 0.02,
              dyadic: bool = False, constant_v: float | None = None,
              one_token_per_list: bool = False) -> HeadDraw:
    """Draw the index parameters, codes and K/V rows of one (sequence, KV head).

    dyadic=True draws centroids and codewords as multiples of 1/16 with magnitude
    below 4 and uses no noise, so every key C[list]+concat(B[code]) has at most
    8 significant bits and is exactly representable in bf16.
    one_token_per_list=True draws the list ids as a permutation of [0, L)
    (L >= T), so every token sits alone in its list.
    """
    rng = np.random.default_rng([workload_id, b, h])
    if dyadic:
        C = (rng.integers(-63, 64, (L, HEAD_DIM)) / 16.0).astype(np.float32)
        B = (rng.integers(-63, 64, (PQ_M, PQ_KSUB, PQ_DSUB)) / 16.0).astype(np.float32)
    else:
        C = rng.standard_normal((L, HEAD_DIM), dtype=np.float32) * np.float32(0.5)
        B = rng.standard_normal((PQ_M, PQ_KSUB, PQ_DSUB), dtype=np.float32) * np.float32(0.3)
    if one_token_per_list:
        lists = rng.permutation(L)[:T].astype(np.int32)
    else:
        lists = rng.integers(0, L, T, dtype=np.int32)
    codes = rng.integers(0, PQ_KSUB, (T, PQ_M), dtype=np.uint8)
    keys = C[lists]
    keys += B[np.arange(PQ_M)[None, :], codes].reshape(T, HEAD_DIM)
    if not dyadic and noise > 0:
        keys += np.float32(noise) * rng.standard_normal((T, HEAD_DIM), dtype=np.float32)
    k_bits = f32_to_bf16_bits(keys)
    del keys
    if constant_v is not None:
        v_bits = np.full((T, HEAD_DIM), f32_to_bf16_bits(np.float32(constant_v)), np.uint16)
    else:
        v_bits = f32_to_bf16_bits(rng.standard_normal((T, HEAD_DIM), dtype=np.float32))
    return HeadDraw(C, B, lists, codes, k_bits, v_bits)


@dataclass
class StepInputs:
    """Logical (unpaged) inputs of one decode step for a batch.

    Per-token arrays are padded to the longest sequence, Tmax; only the first
    context_lens[b] rows of sequence b are meaningful, and only the first
    n_indexed[b] of its lists/codes belong to the index.
    """
    q_bits: np.ndarray          # (B, Hq, 128) uint16
    k_bits: np.ndarray          # (B, Hkv, Tmax, 128) uint16
    v_bits: np.ndarray          # (B, Hkv, Tmax, 128) uint16
    centroids: np.ndarray       # (B, Hkv, L, 128) float32
    codebooks: np.ndarray       # (B, Hkv, 16, 256, 8) float32
    list_ids: np.ndarray        # (B, Hkv, Tmax) int32
    codes: np.ndarray           # (B, Hkv, Tmax, 16) uint8
    context_lens: np.ndarray    # (B,) int32
    n_indexed: np.ndarray       # (B,) int32
    num_lists: int
    n_sink: int
    n_recent: int
    budget_bp: int
    scale: float = 1.0 / np.sqrt(HEAD_DIM)
    planted: list = field(default_factory=list)

    @property
    def batch(self):
        return self.q_bits.shape[0]

    @property
    def num_q_heads(self):
        return self.q_bits.shape[1]

    @property
    def num_kv_heads(self):
        return self.k_bits.shape[1]


def make_step_inputs(workload: int | dict, *, workload_id: int | None = None,
                     context_lens=None, n_tail=None, n_planted=None, noise: float = 0.02,
                     dyadic: bool = False, constant_v: float | None = None,
                     planted_strength: float = 3.0, one_token_per_list: bool = False,
                     workers: int | None = None, **overrides) -> StepInputs:
    """Build one decode step's inputs from a workload (an id in WORKLOADS or a dict).

    Any workload field may be overridden by keyword (num_lists, budget_bp, ...).
    context_lens may give a per-sequence length; n_tail is the unindexed tail
    length of every sequence (clamped to its length).  Large inputs are drawn
    by up to `workers` threads (default: the CPU count, at most 16); the
    result does not depend on the thread count.
    """
    if isinstance(workload, int):
        wid = workload if workload_id is None else workload_id
        w = dict(WORKLOADS[workload])
    else:
        wid = 100 if workload_id is None else workload_id
        w = dict(workload)
    w.update(overrides)
    B, Hq, Hkv, L = w["batch"], w["num_q_heads"], w["num_kv_heads"], w["num_lists"]
    G = Hq // Hkv
    if context_lens is None:
        context_lens = [w["context"]] * B
    context_lens = np.asarray(context_lens, dtype=np.int32)
    tail = w["n_tail"] if n_tail is None else n_tail
    n_indexed = np.maximum(context_lens - tail, 0).astype(np.int32)
    planted_n = w["n_planted"] if n_planted is None else n_planted
    Tmax = int(context_lens.max())

    q_bits = np.zeros((B, Hq, HEAD_DIM), np.uint16)
    k_bits = np.zeros((B, Hkv, Tmax, HEAD_DIM), np.uint16)
    v_bits = np.zeros((B, Hkv, Tmax, HEAD_DIM), np.uint16)
    cents = np.zeros((B, Hkv, L, HEAD_DIM), np.float32)
    books = np.zeros((B, Hkv, PQ_M, PQ_KSUB, PQ_DSUB), np.float32)
    lists = np.zeros((B, Hkv, Tmax), np.int32)
    codes = np.zeros((B, Hkv, Tmax, PQ_M), np.uint8)
    planted_all = []

    def fill(bh):
        # every (b, h) has its own generator, so the draws do not depend on
        # the order in which worker threads run
        b, h = divmod(bh, Hkv)
        T = int(context_lens[b])
        d = draw_head(wid, b, h, T, L, noise=noise, dyadic=dyadic, constant_v=constant_v,
                      one_token_per_list=one_token_per_list)
        cents[b, h], books[b, h] = d.centroids, d.codebooks
        lists[b, h, :T], codes[b, h, :T] = d.list_ids, d.codes
        k_bits[b, h, :T], v_bits[b, h, :T] = d.k_bits, d.v_bits

    n_workers = max(1, min(workers or os.cpu_count() or 1, 16, B * Hkv))
    if n_workers == 1 or int(context_lens.sum()) * Hkv < (1 << 20):
        for bh in range(B * Hkv):
            fill(bh)
    else:
        with ThreadPoolExecutor(n_workers) as ex:
            list(ex.map(fill, range(B * Hkv)))
    for b in range(B):
        T = int(context_lens[b])
        rng = np.random.default_rng([wid, b])
        lo = min(w["n_sink"], T)
        hi = max(T - max(w["n_recent"], T - int(n_indexed[b])), lo)
        pos = []
        if planted_n > 0 and hi > lo:
            edges = np.linspace(lo, hi, planted_n + 1)
            for i in range(planted_n):
                a, e = int(edges[i]), max(int(edges[i + 1]), int(edges[i]) + 1)
                pos.append(int(rng.integers(a, min(e, hi))))
        planted_all.append(pos)
        for h in range(Hkv):
            z = rng.standard_normal((G, HEAD_DIM), dtype=np.float32)
            if pos:
                kp = bf16_bits_to_f32(k_bits[b, h, pos]).astype(np.float32)
                dirs = kp / np.maximum(np.linalg.norm(kp, axis=1, keepdims=True), 1e-30)
                z = z + np.float32(planted_strength) * dirs.sum(axis=0, dtype=np.float32)
            q_bits[b, h * G:(h + 1) * G] = f32_to_bf16_bits(z)
    return StepInputs(q_bits, k_bits, v_bits, cents, books, lists, codes, context_lens,
                      n_indexed, L, w["n_sink"], w["n_recent"], w["budget_bp"],
                      planted=planted_all)


def page_layout(context_lens, page_size: int = PAGE_SIZE, seed: int = 0, spare_pages: int = 0):
    """Block table from a seeded permutation of the page pool.

    Returns (block_table (B, max_pages) int32, num_pages).  Unused table slots
    hold -1.
    """
    context_lens = np.asarray(context_lens)
    need = [(int(t) + page_size - 1) // page_size for t in context_lens]
    num_pages = int(sum(need)) + spare_pages
    max_pages = max(max(need), 1)
    perm = np.random.default_rng([seed, 7]).permutation(num_pages).astype(np.int32)
    table = np.full((len(context_lens), max_pages), -1, np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += n
    return table, num_pages


def to_paged(rows_bits: np.ndarray, context_lens, block_table: np.ndarray, num_pages: int,
             page_size: int = PAGE_SIZE) -> np.ndarray:
    """Scatter logical rows (B, Hkv, Tmax, D) into a paged cache (num_pages, page, Hkv, D)."""
    B, Hkv, _, D = rows_bits.shape
    cache = np.zeros((num_pages, page_size, Hkv, D), rows_bits.dtype)
    for b in range(B):
        T = int(context_lens[b])
        n = (T + page_size - 1) // page_size
        pad = n * page_size
        blk = np.zeros((Hkv, pad, D), rows_bits.dtype)
        blk[:, :T] = rows_bits[b, :, :T]
        blk = blk.reshape(Hkv, n, page_size, D).transpose(1, 2, 0, 3)
        cache[block_table[b, :n]] = blk
    return cache


def make_query_stream(workload_id: int, batch: int, num_q_heads: int, n_steps: int, *,
                      n_topics: int = 4, p_stay: float = 0.8, spread: float = 1.0,
                      jitter: float = 0.05, separate_search: bool = True):
    """Seeded queries of consecutive decode steps, with repeats to reuse.

    Recipe per (sequence b, query head hq), rng = default_rng([workload_id, b, hq, 11]):
      topic centres  Z  = spread * N(0,1) of shape (n_topics, 128)
      attention offsets Zq = spread * N(0,1) of shape (n_topics, 128)
      topic of step 0 uniform in [0, n_topics); each later step keeps the
      previous topic with probability p_stay, else draws it uniformly
      search vector  q_search[t] = bf16( Z[topic_t] + jitter * N(0,1)^128 )
      attention query q[t] = bf16( Zq[topic_t] + jitter * N(0,1)^128 ) when
      separate_search, else q_search[t]
    Returns (q_bits, qs_bits) of shape (n_steps, B, Hq, 128) uint16 and
    topics (n_steps, B, Hq) int32.
    """
    q = np.zeros((n_steps, batch, num_q_heads, HEAD_DIM), np.uint16)
    qs = np.zeros_like(q)
    topics = np.zeros((n_steps, batch, num_q_heads), np.int32)
    for b in range(batch):
        for hq in range(num_q_heads):
            rng = np.random.default_rng([workload_id, b, hq, 11])
            Z = np.float32(spread) * rng.standard_normal((n_topics, HEAD_DIM), dtype=np.float32)
            Zq = np.float32(spread) * rng.standard_normal((n_topics, HEAD_DIM), dtype=np.float32)
            stay = rng.random(n_steps)
            draw = rng.integers(0, n_topics, n_steps)
            noise_s = rng.standard_normal((n_steps, HEAD_DIM), dtype=np.float32)
            noise_q = rng.standard_normal((n_steps, HEAD_DIM), dtype=np.float32)
            t = int(draw[0])
            for i in range(n_steps):
                if i > 0 and stay[i] >= p_stay:
                    t = int(draw[i])
                topics[i, b, hq] = t
                qs[i, b, hq] = f32_to_bf16_bits(Z[t] + np.float32(jitter) * noise_s[i])
                if separate_search:
                    q[i, b, hq] = f32_to_bf16_bits(Zq[t] + np.float32(jitter) * noise_q[i])
                else:
                    q[i, b, hq] = qs[i, b, hq]
    return q, qs, topics
