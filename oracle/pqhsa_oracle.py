"""Plain float64 CPU oracle for one decode step of PQ-HSA attention.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The product path (the HIP library
and its Python binding) never imports, calls or links it, and it shares no
code with that path; both receive their inputs from the seeded generator.

What is computed, and where the pages say so.  "The PQ-HSA page" is the
rit.work blog article "PQ-HSA long-context attention"; "section A" is its
section "How approximate estimates return the discarded context".  "The
query-reuse post" is the quant_prune_distill Telegram post on reusing a
prefix's attention numerator and denominator.

  * Keys of each KV head are indexed with IVF-PQ: grouped into clusters with
    compressed codes kept per token; every indexed token gets an approximate
    attention logit from the index (PQ-HSA page, section A, third paragraph).
    The logit formula is not printed; the reading taken here is the standard
    IVF-PQ residual model s_hat = scale * q . (C[list] + concat_m B_m[code_m]),
    evaluated through per-query tables (lut_tables / approx_logits).
  * One stream of estimates does two jobs: a budget of tokens picked by it is
    read from the original KV cache and computed exactly; the other tokens
    enter the shared normalisation with their approximate logits (section A,
    fourth paragraph).
  * The unread tokens' numerator is their weight summed per cluster times the
    cluster's mean value; main budget 1 % (section A, fifth paragraph).
  * The first tokens and the recent window stay exact; tokens arriving after
    the index was built stay outside it and are read exactly (section A,
    sixth paragraph).
  * O = (N_P + N_S) / (D_P + D_S) for a split of the context into two parts
    (query-reuse post, opening paragraph): the merge law used by lse_merge.

Readings where the pages are silent (each is a choice, stated once here):
  R1 logit model and scale: as above, scale = 1/sqrt(head_dim) on both the
     approximate and the exact logits.
  R2 one top-k per KV head; the selection key of a token is the largest
     approximate logit over the query heads sharing that KV head.
  R3 forced-exact set F = first n_sink tokens  U  last max(n_recent, n_tail)
     tokens, where n_tail = T - n_indexed (recent window and tail both count
     back from the end, so they overlap).  Candidates C = indexed tokens not
     in F.
  R4 budget k = min(ceil(T * budget_bp / 10000), |C|), T the full context.
  R5 ties in the selection key go to the lower token position.
  R6 cluster mean mu_c = mean of V over all indexed tokens of cluster c
     (0 for an empty cluster).
  R7 background weight of an unselected candidate t is exp(s_hat_t - m) with
     the same max m as the exact part: one shared normalisation.

Every function here has a pin in tests/test_oracle_pins.py (dense limit at
budget 100 %, the prefix/suffix merge identity, zero-noise dyadic keys,
one-token clusters, brute force on tiny inputs, closed forms and
invariants).
"""
from __future__ import annotations

import math

import numpy as np


# --------------------------------------------------------------------------
# small helpers
# --------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """Exact upcast of bfloat16 bit patterns (uint16) to float64."""
    w = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return w.view(np.float32).astype(np.float64)


def partition(T: int, n_indexed: int, n_sink: int, n_recent: int):
    """Forced-exact positions F and index candidates C of one sequence (R3).

    PQ-HSA page, section A, sixth paragraph: first tokens and the recent
    window stay exact, new tokens are held outside the index.  Returns two
    ascending int64 arrays (F, C).
    """
    pos = np.arange(T)
    keep_from = T - max(n_recent, T - n_indexed)
    forced = (pos < n_sink) | (pos >= keep_from)
    cand = (~forced) & (pos < n_indexed)
    return np.nonzero(forced)[0], np.nonzero(cand)[0]


def budget_k(T: int, budget_bp: int, n_cand: int) -> int:
    """Top-k size: ceil(T * budget_bp / 10000) capped at |C| (R4), in integers."""
    return min((T * budget_bp + 9999) // 10000, n_cand)


# --------------------------------------------------------------------------
# approximate logits from the IVF-PQ index (PQ-HSA page, section A, 3rd para)
# --------------------------------------------------------------------------
def lut_tables(q_group: np.ndarray, centroids: np.ndarray, codebooks: np.ndarray,
               scale: float):
    """Per-query tables of the IVF-PQ logit (R1).

    q_group (G, D), centroids (L, D), codebooks (M, ksub, D/M)  ->
      qc  (G, L):        qc[g, c]     = scale * q_g . C_c
      lut (G, M, ksub):  lut[g, m, j] = scale * q_g^(m) . B_m[j]
    where q_g^(m) is the m-th D/M-dimensional slice of q_g.
    """
    G, D = q_group.shape
    M, ksub, dsub = codebooks.shape
    qc = scale * (q_group @ centroids.T)
    qm = q_group.reshape(G, M, dsub)
    lut = scale * np.einsum("gmd,mjd->gmj", qm, codebooks)
    return qc, lut


def approx_logits(qc: np.ndarray, lut: np.ndarray, list_ids: np.ndarray,
                  codes: np.ndarray) -> np.ndarray:
    """s_hat[g, t] = qc[g, list_t] + sum_m lut[g, m, code_{t,m}] for indexed t."""
    s = qc[:, list_ids].copy()
    for m in range(lut.shape[1]):
        s += lut[:, m, codes[:, m]]
    return s


def select_topk(kappa: np.ndarray, candidates: np.ndarray, k: int) -> np.ndarray:
    """The k candidates with the largest key, ties to the lower position (R5).

    Returned in ascending position order.
    """
    if k <= 0 or candidates.size == 0:
        return np.zeros(0, np.int64)
    order = np.lexsort((candidates, -kappa[candidates]))
    return np.sort(candidates[order[:k]])


def cluster_means(v_indexed: np.ndarray, list_ids: np.ndarray, num_lists: int) -> np.ndarray:
    """mu_c = mean of V_t over indexed t with list_t = c; 0 if c is empty (R6).

    PQ-HSA page, section A, fifth paragraph ("mean value of this group").
    """
    D = v_indexed.shape[1]
    counts = np.bincount(list_ids, minlength=num_lists).astype(np.float64)
    sums = np.zeros((num_lists, D))
    for d in range(D):
        sums[:, d] = np.bincount(list_ids, weights=v_indexed[:, d], minlength=num_lists)
    mu = np.zeros((num_lists, D))
    nz = counts > 0
    mu[nz] = sums[nz] / counts[nz, None]
    return mu


# --------------------------------------------------------------------------
# the decode step for one KV head and its query-head group
# --------------------------------------------------------------------------
def head_group_step(q_group, K, V, T, n_indexed, centroids, codebooks, list_ids, codes,
                    scale, n_sink, n_recent, budget_bp, selected=None, background=True):
    """One decode step of PQ-HSA for one KV head and the G query heads on it.

    q_group (G, D) float64; K, V (>=T, D) float64 logical rows; the index
    covers positions [0, n_indexed).  If `selected` is given it replaces the
    top-k set (used to recompute the output for another valid selection).
    background=False drops the background term (plain sparse attention, the
    baseline the PQ-HSA page contrasts with in section A, second paragraph).

    Returns a dict with O (G, D), selected (ascending), m (G,) the shared
    max, denom (G,) the total softmax denominator D_exact + D_bg relative to
    m, kappa (n_indexed,), s_hat (G, n_indexed), k, forced, candidates.
    """
    G, Dh = q_group.shape
    L = centroids.shape[0]
    forced, cand = partition(T, n_indexed, n_sink, n_recent)
    qc, lut = lut_tables(q_group, centroids, codebooks, scale)
    s_hat = approx_logits(qc, lut, list_ids[:n_indexed], codes[:n_indexed])
    kappa = s_hat.max(axis=0) if G > 0 else np.zeros(n_indexed)
    k = budget_k(T, budget_bp, cand.size)
    if selected is None:
        S = select_topk(kappa, cand, k)
    else:
        S = np.unique(np.asarray(selected, dtype=np.int64))
        if not np.all(np.isin(S, cand)):
            raise ValueError("selected set must lie inside the candidates")
    exact = np.union1d(forced, S)
    bg = np.setdiff1d(cand, S, assume_unique=True) if background else np.zeros(0, np.int64)

    Ke, Ve = K[exact], V[exact]
    s_ex = scale * (q_group @ Ke.T)                       # (G, |F u S|)
    mu = cluster_means(V[:n_indexed], list_ids[:n_indexed], L)
    s_bg = s_hat[:, bg]                                   # (G, |Bg|)

    m = np.full(G, -np.inf)
    if exact.size:
        m = np.maximum(m, s_ex.max(axis=1))
    if bg.size:
        m = np.maximum(m, s_bg.max(axis=1))

    O = np.zeros((G, Dh))
    denom = np.zeros(G)
    for g in range(G):
        if not np.isfinite(m[g]):
            continue
        p_ex = np.exp(s_ex[g] - m[g])
        d_ex = p_ex.sum()
        n_ex = p_ex @ Ve
        w = np.bincount(list_ids[bg], weights=np.exp(s_bg[g] - m[g]), minlength=L)
        d_bg = w.sum()
        n_bg = w @ mu
        denom[g] = d_ex + d_bg
        O[g] = (n_ex + n_bg) / denom[g]
    return dict(O=O, selected=S, m=m, denom=denom, kappa=kappa, s_hat=s_hat, k=k,
                forced=forced, candidates=cand, means=mu)


def decode_step(inp, selected=None, background=True, heads=None):
    """PQ-HSA decode step over a batch of `pqhsa_synth.StepInputs`.

    selected: optional dict {(b, h): positions} overriding the top-k of those
    heads.  heads: optional iterable of (b, h) to compute (others left 0).
    Returns dict with O (B, Hq, D), selected {(b, h): array}, m and denom
    (B, Hq), k {(b, h): int}.
    """
    B, Hq, Hkv = inp.batch, inp.num_q_heads, inp.num_kv_heads
    G = Hq // Hkv
    D = inp.q_bits.shape[-1]
    O = np.zeros((B, Hq, D))
    m = np.full((B, Hq), -np.inf)
    den = np.zeros((B, Hq))
    sel, ks = {}, {}
    todo = [(b, h) for b in range(B) for h in range(Hkv)] if heads is None else list(heads)
    for b, h in todo:
        T, Ti = int(inp.context_lens[b]), int(inp.n_indexed[b])
        q = bf16_to_f64(inp.q_bits[b, h * G:(h + 1) * G])
        K = bf16_to_f64(inp.k_bits[b, h, :T])
        V = bf16_to_f64(inp.v_bits[b, h, :T])
        r = head_group_step(q, K, V, T, Ti, inp.centroids[b, h].astype(np.float64),
                            inp.codebooks[b, h].astype(np.float64), inp.list_ids[b, h, :T],
                            inp.codes[b, h, :T], inp.scale, inp.n_sink, inp.n_recent,
                            inp.budget_bp,
                            selected=None if selected is None else selected.get((b, h)),
                            background=background)
        O[b, h * G:(h + 1) * G] = r["O"]
        m[b, h * G:(h + 1) * G] = r["m"]
        den[b, h * G:(h + 1) * G] = r["denom"]
        sel[(b, h)], ks[(b, h)] = r["selected"], r["k"]
    return dict(O=O, selected=sel, m=m, denom=den, k=ks)


# --------------------------------------------------------------------------
# dense attention and the prefix/suffix merge law
# --------------------------------------------------------------------------
def dense_attention(q_group: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Plain softmax attention of G queries over all rows of K, V.

    Returns (O (G, D), m (G,), denom (G,)) with denom relative to m.
    """
    s = scale * (q_group @ K.T)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    den = p.sum(axis=1)
    return (p @ V) / den[:, None], m, den


def dense_step(inp):
    """Dense decode attention over each sequence's full context, (B, Hq, D)."""
    B, Hq, Hkv = inp.batch, inp.num_q_heads, inp.num_kv_heads
    G = Hq // Hkv
    O = np.zeros((B, Hq, inp.q_bits.shape[-1]))
    for b in range(B):
        T = int(inp.context_lens[b])
        for h in range(Hkv):
            q = bf16_to_f64(inp.q_bits[b, h * G:(h + 1) * G])
            O[b, h * G:(h + 1) * G] = dense_attention(
                q, bf16_to_f64(inp.k_bits[b, h, :T]), bf16_to_f64(inp.v_bits[b, h, :T]),
                inp.scale)[0]
    return O


def partial_attention(q_group, K, V, scale):
    """Unnormalised parts of attention over a block of rows: (m, N, D).

    N = sum_t exp(s_t - m) V_t and D = sum_t exp(s_t - m): the numerator and
    denominator of the query-reuse post's O = (N_P + N_S)/(D_P + D_S).
    An empty block gives m = -inf, N = 0, D = 0.
    """
    G = q_group.shape[0]
    if K.shape[0] == 0:
        return np.full(G, -np.inf), np.zeros((G, V.shape[1])), np.zeros(G)
    s = scale * (q_group @ K.T)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    return m, p @ V, p.sum(axis=1)


def lse_merge(parts):
    """Merge (m, N, D) parts into O: O = sum_i e^{m_i-M} N_i / sum_i e^{m_i-M} D_i."""
    ms = np.stack([p[0] for p in parts])
    M = ms.max(axis=0)
    w = np.where(np.isfinite(ms), np.exp(ms - M), 0.0)
    num = sum(w[i][:, None] * parts[i][1] for i in range(len(parts)))
    den = sum(w[i] * parts[i][2] for i in range(len(parts)))
    return num / den[:, None]


# --------------------------------------------------------------------------
# brute force for tiny inputs: an independent route through the same reading
# --------------------------------------------------------------------------
def bruteforce_head_group(q_group, K, V, T, n_indexed, centroids, codebooks, list_ids, codes,
                          scale, n_sink, n_recent, budget_bp):
    """Token-by-token version of head_group_step for tiny inputs.

    Reconstructs every key from its cluster centroid and codewords instead of
    using lookup tables, sorts with Python's sort, and sums the background
    token by token (weight times the mean of the token's cluster) instead of
    through per-cluster bins.  Pure Python loops: keep T <= a few hundred.
    """
    G, Dh = len(q_group), len(q_group[0])
    M = len(codebooks)
    dsub = Dh // M
    L = len(centroids)
    khat = []
    for t in range(n_indexed):
        c = int(list_ids[t])
        vec = []
        for m in range(M):
            vec.extend(float(x) for x in codebooks[m][int(codes[t][m])])
        khat.append([float(centroids[c][i]) + vec[i] for i in range(Dh)])
    s_hat = [[scale * sum(float(q_group[g][i]) * khat[t][i] for i in range(Dh))
              for t in range(n_indexed)] for g in range(G)]
    kappa = [max(s_hat[g][t] for g in range(G)) for t in range(n_indexed)]
    keep_from = T - max(n_recent, T - n_indexed)
    forced = [t for t in range(T) if t < n_sink or t >= keep_from]
    cand = [t for t in range(n_indexed) if t not in forced]
    k = min(math.ceil(T * budget_bp / 10000), len(cand))
    chosen = sorted(cand, key=lambda t: (-kappa[t], t))[:k]
    S = sorted(chosen)
    bgset = [t for t in cand if t not in chosen]
    # cluster means from all indexed tokens
    sums = [[0.0] * Dh for _ in range(L)]
    cnt = [0] * L
    for t in range(n_indexed):
        c = int(list_ids[t])
        cnt[c] += 1
        for i in range(Dh):
            sums[c][i] += float(V[t][i])
    mu = [[sums[c][i] / cnt[c] if cnt[c] else 0.0 for i in range(Dh)] for c in range(L)]
    exact = sorted(set(forced) | set(S))
    O = []
    for g in range(G):
        s_ex = {t: scale * sum(float(q_group[g][i]) * float(K[t][i]) for i in range(Dh))
                for t in exact}
        vals = list(s_ex.values()) + [s_hat[g][t] for t in bgset]
        mx = max(vals)
        num = [0.0] * Dh
        den = 0.0
        for t in exact:
            w = math.exp(s_ex[t] - mx)
            den += w
            for i in range(Dh):
                num[i] += w * float(V[t][i])
        for t in bgset:
            w = math.exp(s_hat[g][t] - mx)
            den += w
            c = int(list_ids[t])
            for i in range(Dh):
                num[i] += w * mu[c][i]
        O.append([x / den for x in num])
    del dsub
    return dict(O=np.array(O), selected=np.array(S, dtype=np.int64), kappa=np.array(kappa), k=k)
