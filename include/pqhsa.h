/*
 * pqhsa.h -- C ABI of libpqhsa: one decode step of PQ-HSA attention on an
 * AMD Instinct MI355X (gfx950).
 *
 * The method (rit.work blog, "PQ-HSA long-context attention", section "How
 * approximate estimates return the discarded context"): every KV head's keys
 * are indexed with IVF-PQ (clusters plus compressed codes); each indexed
 * token gets an approximate attention logit from the index; a budget of the
 * best tokens, the first tokens, the recent window and the not-yet-indexed
 * tail are attended exactly from the paged KV cache; every other token stays
 * in the softmax through its approximate weight, and its numerator is that
 * weight summed per cluster times the cluster's mean value:
 *     O = (N_exact + N_bg) / (D_exact + D_bg).
 * The last identity is the prefix/suffix merge of the quant_prune_distill
 * post on query reuse (opening paragraph), applied to more than two parts.
 *
 * Conventions shared by every entry point
 *   - Every array pointer is a DEVICE pointer (hipMalloc'd or a torch CUDA
 *     tensor), owned by the caller.  The library never allocates, frees or
 *     synchronises; scratch memory comes in through `workspace`.
 *   - Work is enqueued on `stream`; results are ready when the stream is.
 *   - Arguments are validated on the host before anything is launched; an
 *     invalid call returns a status and enqueues nothing.  PQHSA_ERR_HIP means
 *     a launch failed.  Faults inside kernels surface at the caller's next
 *     synchronisation.
 *   - Values that live on the device (context lengths, n_indexed, block
 *     table entries) are range-checked inside the kernels: out-of-range
 *     values are clamped so that no access leaves its buffer, and the output
 *     is then unspecified.  Documented preconditions below say what is valid.
 *   - bf16 data are passed as uint16_t bit patterns.
 *   - No global state: concurrent calls on different streams with disjoint
 *     workspaces are safe.  Calls sharing a workspace must be ordered.
 *
 * Supported shapes: head_dim 128, page_size 16, pq_m 16 (8-dim subspaces),
 * pq_ksub 256, G = num_q_heads / num_kv_heads in {1, 2, 4, 8},
 * 1 <= num_lists <= 16384.  Query head i uses KV head i / G.
 */
#ifndef PQHSA_H
#define PQHSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pqhsa_status {
  PQHSA_OK = 0,
  PQHSA_ERR_INVALID_ARG = 1,     /* null pointer, inconsistent or out-of-range shape field */
  PQHSA_ERR_UNSUPPORTED = 2,     /* a valid shape these kernels are not built for */
  PQHSA_ERR_BUFFER_TOO_SMALL = 3,/* index_buf or workspace smaller than the query functions say */
  PQHSA_ERR_HIP = 4              /* a HIP launch or copy failed */
} pqhsa_status;

/* Shape and method parameters.  All fields are host values. */
typedef struct pqhsa_shape {
  int32_t batch;              /* B >= 1 sequences */
  int32_t num_q_heads;        /* Hq */
  int32_t num_kv_heads;       /* Hkv, Hq % Hkv == 0 */
  int32_t head_dim;           /* 128 */
  int32_t page_size;          /* tokens per cache page, 16 */
  int32_t num_pages;          /* pages in each of the K and V caches */
  int32_t max_pages_per_seq;  /* columns of the block table */
  int32_t num_lists;          /* L, IVF clusters per (sequence, KV head) */
  int32_t pq_m;               /* PQ subspaces, 16 */
  int32_t pq_ksub;            /* codewords per subspace, 256 */
  int32_t max_context;        /* bound on every context length and index capacity;
                                 <= max_pages_per_seq * page_size */
  int32_t n_sink;             /* first tokens always attended exactly, >= 0 */
  int32_t n_recent;           /* last tokens always attended exactly, >= 0 */
  int32_t budget_bp;          /* top-k budget in basis points of the context, 0..10000 */
  float scale;                /* logit scale, normally 1/sqrt(head_dim); > 0 */
  int32_t exact_only;         /* 0: PQ-HSA (exact part + background term);
                                 1: drop the background term, i.e. plain top-k
                                 sparse attention over sink, selected and recent
                                 tokens, the comparison of section B of the
                                 PQ-HSA page; other values are invalid */
} pqhsa_shape;

/* Number of entry points computed per step (exact partial splits etc.) are
 * chosen by the library from the shape; these report the buffer sizes. */

/* Bytes of the index buffer for `shape` (0 if the shape is invalid). */
size_t pqhsa_index_bytes(const pqhsa_shape* shape);

/* Bytes of scratch workspace for pqhsa_upload_index (0 if invalid). */
size_t pqhsa_upload_workspace_bytes(const pqhsa_shape* shape);

/* Bytes of scratch workspace for one decode step; dense != 0 sizes it for
 * pqhsa_dense_decode_step instead.  0 if the shape is invalid.  A decode-step
 * workspace must be zero-filled before its first use (it holds per-head
 * counters and a histogram that every step leaves cleared for the next one);
 * it needs no further clearing while it is used for one shape. */
size_t pqhsa_workspace_bytes(const pqhsa_shape* shape, int dense);

/* Capacity of the optional `selected` output per (sequence, KV head):
 * min(ceil(max_context * budget_bp / 10000), max_context). */
int32_t pqhsa_max_selected(const pqhsa_shape* shape);

/*
 * Build the per-step index from an IVF-PQ index built after prefill
 * (PQ-HSA page, section "How approximate estimates return the discarded
 * context", sixth paragraph: the index is built after the prompt is filled,
 * newer tokens stay outside it).  Not part of the per-step path.
 *
 *   centroids   float [B][Hkv][L][128]          IVF cluster centres
 *   codebooks   float [B][Hkv][16][256][8]      PQ codewords, shared by the L lists
 *   list_ids    int32 [B][Hkv][max_context]     cluster of token t (first n_indexed used)
 *   codes       uint8 [B][Hkv][max_context][16] PQ code of token t's key
 *   n_indexed   int32 [B]                       indexed prefix length of each sequence;
 *                                               must be <= max_context
 *   v_cache     bf16  [num_pages][16][Hkv][128] paged values (for the cluster means)
 *   block_table int32 [B][max_pages_per_seq]    logical page -> physical page
 *
 * Writes into index_buf: the centroids and codebooks, the codes regrouped
 * by cluster (stable: token order kept inside a cluster) with each entry's
 * token position, and each cluster's mean value vector over its indexed
 * tokens (section A, fifth paragraph: the group's mean value; 0 for an
 * empty cluster).  Tokens whose list id lies outside [0, L) are left out of
 * the index and counted; pqhsa_index_dropped() reports the count.
 * index_buf must stay alive and unchanged while decode steps use it.
 */
pqhsa_status pqhsa_upload_index(const pqhsa_shape* shape, const float* centroids,
                                const float* codebooks, const int32_t* list_ids,
                                const uint8_t* codes, const int32_t* n_indexed,
                                const uint16_t* v_cache, const int32_t* block_table,
                                void* index_buf, size_t index_bytes, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* Bytes of scratch workspace for pqhsa_append_tokens (0 if invalid). */
size_t pqhsa_append_workspace_bytes(const pqhsa_shape* shape);

/*
 * Add tokens [n_indexed_b, new_n_indexed[b]) of each sequence to an uploaded
 * index: the tokens held outside the index are added to it in batches
 * (PQ-HSA page, section A, sixth paragraph; section C lists the update cost
 * among the things to measure).
 *
 *   index_buf      an index written by pqhsa_upload_index (and possibly
 *                  earlier appends) for `shape`; updated in place
 *   k_cache, v_cache, block_table   as in pqhsa_decode_step; the new tokens'
 *                  keys and values must be in the cache
 *   new_n_indexed  int32 [B] device; new_n_indexed[b] >= the index's current
 *                  n_indexed[b] and <= max_context
 *   max_new        host bound on new_n_indexed[b] - n_indexed[b] over b
 *                  (sizes the grid).  At most max_new tokens of a sequence
 *                  are added: its n_indexed becomes
 *                  min(new_n_indexed[b], n_indexed_b + max_new), and any
 *                  further tokens stay in the exact tail.
 *   list_ids       int32 [B][Hkv][max_context], the token-order list ids the
 *                  index was uploaded from; entries of the new tokens are
 *                  written, all indexed entries are read
 *   codes          uint8 [B][Hkv][max_context][16], likewise
 *
 * For each new token t of (b, h), with K_t its key from the cache:
 *   list_t   = argmin_c ||K_t - C_c||^2                  (lowest c on ties)
 *   code_t,m = argmin_j ||(K_t - C[list_t])^(m) - B_m[j]||^2  (lowest j on ties)
 * in fp32 (the residual IVF-PQ encoder matching the decode step's key model;
 * the pages print no encoder).  The index is then regrouped by cluster over
 * all indexed tokens (token order kept inside a cluster) and every cluster
 * mean becomes (n_old * mean + sum of the new members' V) / n_new.  Finally
 * the index's n_indexed becomes new_n_indexed.  Asynchronous on `stream`.
 */
pqhsa_status pqhsa_append_tokens(const pqhsa_shape* shape, void* index_buf,
                                 const uint16_t* k_cache, const uint16_t* v_cache,
                                 const int32_t* block_table, const int32_t* new_n_indexed,
                                 int32_t max_new, int32_t* list_ids, uint8_t* codes,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Copy the count of dropped (out-of-range list id) tokens of an uploaded
 * index to *dropped.  Synchronises `stream`; meant for tests and tooling. */
pqhsa_status pqhsa_index_dropped(const pqhsa_shape* shape, const void* index_buf,
                                 int64_t* dropped, hipStream_t stream);

/*
 * One PQ-HSA decode step for every (sequence, query head).
 *
 *   q            bf16  [B][Hq][128]                 current queries
 *   k_cache      bf16  [num_pages][16][Hkv][128]    paged keys (vLLM layout)
 *   v_cache      bf16  [num_pages][16][Hkv][128]    paged values
 *   block_table  int32 [B][max_pages_per_seq]
 *   context_lens int32 [B]    T_b, 1..max_context, >= n_indexed of the index
 *   out          float [B][Hq][128]                 attention output O
 *   selected     int32 [B][Hkv][pqhsa_max_selected] optional (may be NULL):
 *                the top-k positions in ascending order, -1 padded
 *   lse          float [B][Hq]                      optional (may be NULL):
 *                natural log of the full softmax denominator, m + log(D)
 *
 * Per (sequence b, KV head h), with T = T_b and n_tail = T - n_indexed:
 *   forced F  = [0, n_sink) U [T - max(n_recent, n_tail), T)
 *   candidates C = indexed tokens not in F
 *   s_hat_g,t = scale * (q_g . C[list_t] + sum_m q_g^(m) . B_m[code_t,m])
 *   key_t     = max over the G query heads g of s_hat_g,t
 *   S         = the k = min(ceil(T*budget_bp/10000), |C|) candidates with the
 *               largest key, ties to the lower position
 *   exact logits for F U S from the paged cache; for every other candidate
 *   the weight exp(s_hat - m) is summed per cluster and multiplied by the
 *   cluster's mean value; one shared normalisation gives O.
 * (Section A of the PQ-HSA page, paragraphs three to six.  Taking the max
 * over the group's query heads, the overlap of the recent window with the
 * tail, and the tie rule are readings where the page is silent.)
 */
/* Execution: when its whole grid fits on the device at once, the step
 * runs as one kernel whose blocks of a KV head share that head's clusters and
 * meet at two barriers (fused step); otherwise as the six kernels listed
 * below (staged step).  Both compute the same quantities.  The fused step
 * assumes its blocks can all be resident together: on a device whose CUs are
 * partly withheld (CU masking, long-running concurrent kernels) a barrier wait
 * may run out after about 2 s.  The call still returns PQHSA_OK (it cannot
 * wait for the device), the affected KV head's `out` and `lse` entries are NaN,
 * and bit 0 of the workspace flags is set.  Checking that flag with
 * pqhsa_step_flags is the caller's duty wherever CUs may be withheld; once it
 * is set, the workspace must be cleared (pqhsa_step_flags with clear != 0)
 * before the next step.  The staged variant of pqhsa_decode_step_profiled has
 * no residency requirement. */
pqhsa_status pqhsa_decode_step(const pqhsa_shape* shape, const void* index_buf,
                               const uint16_t* q, const uint16_t* k_cache,
                               const uint16_t* v_cache, const int32_t* block_table,
                               const int32_t* context_lens, float* out, int32_t* selected,
                               float* lse, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * pqhsa_decode_step without a workspace argument, for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments (minus workspace), same results and
 * same kernels as pqhsa_decode_step, plus one small kernel that clears the
 * step's counters first.  Scratch comes from a fixed array of
 * PQHSA_NOALLOC_SCRATCH_BYTES in the library, one per device, held until the
 * process ends; nothing is allocated or freed.  Shapes whose workspace
 * (pqhsa_workspace_bytes(shape, 0)) exceeds it return
 * PQHSA_ERR_BUFFER_TOO_SMALL and enqueue nothing (128 MiB covers, e.g., one
 * sequence of 131072 tokens with 8 KV heads; not 16 such sequences).
 * Every call on a device shares that device's array: calls that overlap on
 * one device (other streams, other threads) race and must be ordered by the
 * caller.  A barrier wait that runs out leaves NaN outputs as in
 * pqhsa_decode_step; the next call starts from cleared counters.  Errors: as
 * pqhsa_decode_step; PQHSA_ERR_HIP also if the array's address cannot be
 * found.
 */
#define PQHSA_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
pqhsa_status pqhsa_decode_step_noalloc(const pqhsa_shape* shape, const void* index_buf,
                                       const uint16_t* q, const uint16_t* k_cache,
                                       const uint16_t* v_cache, const int32_t* block_table,
                                       const int32_t* context_lens, float* out,
                                       int32_t* selected, float* lse, hipStream_t stream);

/*
 * Dense split-K decode attention over each sequence's whole context, through
 * the same exact-attention row tiles (16-row MFMA tiles, online softmax) as
 * pqhsa_decode_step, and the staged step's log-sum-exp merge kernel.  This is
 * the honest baseline: the activation/KV-sparsity crossover article
 * (rit.work blog, section "Why one method gives different speed-ups") runs
 * dense and sparse modes through one split-K kernel, because a slower dense
 * kernel inflates the measured speed-up.  index_buf is not needed.
 * Arguments as in pqhsa_decode_step; budget, sink, recent and list fields of
 * the shape are ignored.
 */
pqhsa_status pqhsa_dense_decode_step(const pqhsa_shape* shape, const uint16_t* q,
                                     const uint16_t* k_cache, const uint16_t* v_cache,
                                     const int32_t* block_table, const int32_t* context_lens,
                                     float* out, float* lse, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/* Kernels of the staged decode step, in launch order, for profiling. */
enum {
  PQHSA_STAGE_TABLES = 0,     /* per-query lookup tables */
  PQHSA_STAGE_SCAN = 1,       /* code scan: approximate logits, keys, cluster bins */
  PQHSA_STAGE_COLLECT = 2,    /* top-k: threshold bucket, collection, selected weights */
  PQHSA_STAGE_SELECT = 3,     /* top-k: exact threshold, ascending row list */
  PQHSA_STAGE_ATTEND = 4,     /* paged split-K exact attention and background partials */
  PQHSA_STAGE_MERGE = 5,      /* log-sum-exp merge into O */
  PQHSA_NUM_STAGES = 6
};

/* Variants of pqhsa_decode_step_profiled. */
enum {
  PQHSA_VARIANT_DEFAULT = 0,  /* exactly what pqhsa_decode_step runs */
  PQHSA_VARIANT_STAGED = 1,   /* the six staged kernels, whatever the shape */
  PQHSA_VARIANT_DENSE = 2,    /* pqhsa_dense_decode_step (index_buf unused) */
  PQHSA_VARIANT_BARRIER_TEST = 3, /* test only: the fused step with barriers that
                                     wait for one block more than there are and
                                     give up after 20 us, so that every wait runs
                                     out (every kernel still ends normally): all
                                     outputs NaN, flags bit 0 set.  Returns
                                     PQHSA_ERR_UNSUPPORTED where the fused step
                                     cannot run the shape. */
  PQHSA_VARIANT_KEYS_OUT = 4      /* test only: the fused step, which then also
                                     writes every entry's 16-bit key code into
                                     the workspace's keys region (by default it
                                     passes them from its scan to its selection
                                     in LDS where a block's entries fit).
                                     Returns PQHSA_ERR_UNSUPPORTED where the
                                     fused step cannot run the shape. */
};

/* A decode step that also times its kernels.  events holds 2 * PQHSA_NUM_STAGES
 * events created by the caller; kernel i of the step gets events[2i] (start)
 * and events[2i+1] (end), and *n_kernels (if not NULL) is set to the number
 * of kernels launched.  Kernels are launched with hipExtLaunchKernel, whose
 * events stamp each kernel's own start and end.  Results are those of the
 * untimed call of the same variant. */
pqhsa_status pqhsa_decode_step_profiled(const pqhsa_shape* shape, const void* index_buf,
                                        const uint16_t* q, const uint16_t* k_cache,
                                        const uint16_t* v_cache, const int32_t* block_table,
                                        const int32_t* context_lens, float* out,
                                        int32_t* selected, float* lse, void* workspace,
                                        size_t workspace_bytes, int variant,
                                        hipEvent_t* events, int32_t* n_kernels,
                                        hipStream_t stream);

/* Byte offsets of the intermediate arrays inside the decode workspace, so
 * tests can check each stage.  Layouts (bh = b * Hkv + h):
 *   lut     float [B*Hkv][16][256][G]  scale*log2(e) * q_g^(m) . B_m[j]
 *   qc      float [B*Hkv][L][G]        scale*log2(e) * q_g . C_c
 *   keys    uint32 [B*Hkv][max_context] order-preserving bits of each index
 *           entry's key (cluster order; 0 for non-candidates)
 *   bins    float [B*Hkv][L][G][2]     per cluster: max and sum of exp2 of
 *           the candidates' base-2 logits relative to that max
 *   rows    int32 [B*Hkv][max_context] exact rows: sink, selected, recent/tail
 *   n_rows  int32 [B*Hkv]
 *   partials float [B][Hq][n_parts][132]: (m in base 2, l, pad, pad, acc[128])
 *   flags   uint32: bit 0 set if a barrier wait of the fused step ever timed
 *           out (its results are then not valid)
 * The staged step fills lut, qc, keys, bins, rows, n_rows and partials; the
 * fused step fills qc and bins of every cluster and n_rows; rows only for
 * blocks whose share of the exact rows exceeds one LDS staging (in a
 * per-block order); and, under PQHSA_VARIANT_KEYS_OUT or for blocks whose
 * entries exceed their LDS key cache, at the start of keys a 16-bit code of
 * each key as uint16 [B*Hkv][max_context]: the order key's sign, its binary
 * exponent clamped to the 16 binades of [2^-7, 2^9) (the same field range in
 * both halves), then 11 mantissa bits, at least 1 (0 for non-candidates). */
/* Also: hist (uint32 [B*Hkv][5120]: each (b, h)'s 4096-bin key histogram
 * followed by 1024 unused words, hist_bytes long) and
 * counters (the fused step's per-head barrier counters and flags, the flags
 * word and per-block counts, counters_bytes long): the regions a step expects
 * to find cleared; total = pqhsa_workspace_bytes. */
typedef struct pqhsa_ws_layout {
  size_t lut, qc, keys, bins, rows, n_rows, partials, flags;
  int32_t n_exact_splits, n_bg_splits, n_parts;
  size_t hist, hist_bytes, counters, counters_bytes, total;
} pqhsa_ws_layout;
pqhsa_status pqhsa_workspace_layout(const pqhsa_shape* shape, int dense, pqhsa_ws_layout* out);

/* Status word of a decode-step workspace: *flags gets the flags word (bit 0:
 * a barrier wait of the fused step ran out since the workspace was last
 * cleared, so the outputs of the heads involved were written as NaN).  With
 * clear != 0 the workspace's counters, flags and histogram are then zeroed,
 * which makes it ready for the next step.  Synchronises `stream` (meant for
 * error handling and tests, not for every step).  Errors: shape errors as in
 * pqhsa_decode_step; PQHSA_ERR_INVALID_ARG for a NULL pointer;
 * PQHSA_ERR_BUFFER_TOO_SMALL for a short workspace; PQHSA_ERR_HIP. */
pqhsa_status pqhsa_step_flags(const pqhsa_shape* shape, void* workspace, size_t workspace_bytes,
                              int clear, uint32_t* flags, hipStream_t stream);

/* Byte offsets of the index arrays inside index_buf (bh = b * Hkv + h):
 *   centroids float [B*Hkv][L][128], codebooks float [B*Hkv][16][256][8],
 *   list_off int32 [B*Hkv][L+1] (entries of cluster c are [list_off[c], list_off[c+1])),
 *   codes uint8 [B*Hkv][max_context][16], pos int32 [B*Hkv][max_context],
 *   means float [B*Hkv][L][128], n_indexed int32 [B]. */
typedef struct pqhsa_index_layout {
  size_t centroids, codebooks, list_off, codes, pos, means, n_indexed, dropped;
} pqhsa_index_layout;
pqhsa_status pqhsa_index_layout_of(const pqhsa_shape* shape, pqhsa_index_layout* out);

/*
 * ------------------------------------------------------------------ query reuse
 * Dense decode attention that reuses the prefix numerator and denominator of a
 * close earlier query (the quant_prune_distill post on query reuse, opening
 * paragraph and sections "Important practical considerations" and
 * "Experiments"): O = (N_P + N_S) / (D_P + D_S), where the prefix terms come
 * from the earlier query's stored state and only the suffix is computed.
 *
 * Every query head of every sequence keeps a ring of `window` entries (1 to
 * 8192; the post searches the last 1024 tokens), one per step: the step's
 * search vector (bf16, 128 values), the state its attention produced (base-2
 * maximum m, sum l and unnormalised acc[128], fp32) and the context length T_j
 * it was computed at.  At context length T, head (b, hq):
 *   eligible  = entries with 1 <= T_j <= T and T - T_j < window
 *   d2_j      = sum_i (q_search[b][hq][i] - search_j[i])^2, fp32 from bf16
 *   choice    = the eligible entry with the smallest d2, then the larger T_j,
 *               then the lower slot
 *   reuse     when a choice exists and d2 <= max_dist2
 *   O         = attention of q[b][hq] over [T_j, T) merged with the entry's
 *               state (reuse), or over [0, T) (no reuse)
 * and the step's state is written to slot (count mod window) of the head's
 * ring, with T_j = T, replacing the oldest entry.  (Comparing the pre-RoPE
 * query vectors, one ring per query head, the window counted in steps, the
 * squared distance and the tie order are readings where the post is silent:
 * it names keys where it compares queries and gives no threshold.)
 *
 * Arguments as in pqhsa_dense_decode_step, plus:
 *   window        ring slots per query head, 1..8192
 *   max_dist2     reuse threshold on the squared distance (a negative value
 *                 never reuses; NaN is invalid)
 *   q_search      uint16 (bf16) [B][Hq][128] pre-RoPE vectors compared across
 *                 steps (may equal q)
 *   reuse_buf     device buffer of pqhsa_reuse_buffer_bytes(shape, window)
 *                 bytes, owned by the caller and kept across steps; zero-filled
 *                 or cleared with pqhsa_reuse_clear before its first step
 *   reused_slot   int32 [B][Hq] optional: slot reused, -1 when none
 *   min_dist2     float [B][Hq] optional: smallest eligible d2 (inf if none)
 *   workspace     pqhsa_reuse_workspace_bytes(shape, window) bytes of scratch
 * Steps on one reuse_buf must be ordered (same stream or synchronised); the
 * step runs three kernels: search, split-K attention, merge and insert.
 * Errors: PQHSA_ERR_INVALID_ARG for a NULL required pointer, a window out of
 * range or a NaN threshold; PQHSA_ERR_BUFFER_TOO_SMALL for short buffers;
 * shape errors as in pqhsa_dense_decode_step.
 */
size_t pqhsa_reuse_buffer_bytes(const pqhsa_shape* shape, int32_t window);
size_t pqhsa_reuse_workspace_bytes(const pqhsa_shape* shape, int32_t window);

/* Byte offsets of the rings inside reuse_buf: search [B*Hq][window][128] bf16,
 * states [B*Hq][window][132] fp32 (m, l, 0, 0, acc[128]), context
 * [B*Hq][window] int32 (T_j, 0 = empty) and count [B*Hq] int32. */
typedef struct pqhsa_reuse_layout {
  size_t search, states, context, count, total;
} pqhsa_reuse_layout;
pqhsa_status pqhsa_reuse_layout_of(const pqhsa_shape* shape, int32_t window,
                                   pqhsa_reuse_layout* out);

/* Empty the rings of sequences [seq_begin, seq_end) (for a new request in
 * those batch slots).  Asynchronous on `stream`. */
pqhsa_status pqhsa_reuse_clear(const pqhsa_shape* shape, int32_t window, void* reuse_buf,
                               size_t reuse_bytes, int32_t seq_begin, int32_t seq_end,
                               hipStream_t stream);

pqhsa_status pqhsa_reuse_decode_step(const pqhsa_shape* shape, int32_t window, float max_dist2,
                                     const uint16_t* q, const uint16_t* q_search,
                                     const uint16_t* k_cache, const uint16_t* v_cache,
                                     const int32_t* block_table, const int32_t* context_lens,
                                     void* reuse_buf, size_t reuse_bytes, float* out, float* lse,
                                     int32_t* reused_slot, float* min_dist2, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/* pqhsa_reuse_decode_step with its three kernels timed: events holds 6 events
 * created by the caller, kernel i stamps events[2i] and events[2i+1]. */
pqhsa_status pqhsa_reuse_decode_step_profiled(
    const pqhsa_shape* shape, int32_t window, float max_dist2, const uint16_t* q,
    const uint16_t* q_search, const uint16_t* k_cache, const uint16_t* v_cache,
    const int32_t* block_table, const int32_t* context_lens, void* reuse_buf, size_t reuse_bytes,
    float* out, float* lse, int32_t* reused_slot, float* min_dist2, void* workspace,
    size_t workspace_bytes, hipEvent_t* events, int32_t* n_kernels, hipStream_t stream);

/* Static description of a status code. */
const char* pqhsa_status_string(pqhsa_status status);

#ifdef __cplusplus
}
#endif
#endif /* PQHSA_H */
