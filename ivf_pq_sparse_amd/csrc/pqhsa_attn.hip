// Exact split-K attention over paged bf16 K/V, the per-cluster background
// term, and the log-sum-exp merge.
//
// PQ-HSA page (rit.work blog), section "How approximate estimates return the
// discarded context": selected, first and recent tokens are read from the
// original (paged) KV cache and computed exactly (fourth and sixth
// paragraphs); unread tokens contribute their approximate weight summed per
// cluster times the cluster mean (fifth paragraph).  The merge is the
// prefix/suffix law O = (N_P + N_S)/(D_P + D_S) of the quant_prune_distill
// post on query reuse, over all partials.  Dense and sparse exact attention
// run through the same row-tile MFMA code (pqhsa_internal.hpp: tile_logits,
// tile_accumulate), as the activation/KV-sparsity crossover article (rit.work
// blog, section "Why one method gives different speed-ups") requires of an
// honest baseline: the dense step's tiles are the pages of the context, the
// sparse steps' tiles are gathered from their row lists.  The same code also
// serves query reuse: each query head starts at the context length of the
// earlier query whose prefix state it reuses (0 when it reuses none), and the
// reused state joins the merge as one more partial.
//
// Split-K block: 4 waves.  The block stages the cache offsets of up to 256
// rows in LDS (row list and block table read once, in parallel); wave w takes
// the staged row tiles w, w + 4, ... with the next tile's K and V in flight.
// The 4 waves merge through LDS and the block writes one partial
// (m, l, acc[128]) per query head.
#include "pqhsa_internal.hpp"

namespace pqhsa {

// LDS of one attend block: staged row offsets, then the merge of 4 waves x G
// heads x (m, l, acc[128]).
template <int G>
struct AttendLds {
  long long row_off[kPhaseRows];
  float ml[4][G][2];
  float acc[4][G][kD];
  int rstart[G];   // query reuse: first position computed for head g
  int rslot[G];    // query reuse: reused slot of head g, or -1
};

// Where the rows of a split-K block come from.
enum RowSource {
  kRowsIndex = 0,   // the step's exact-row list (sink, selected, recent)
  kRowsReuse = 2    // [start_g, T) per query head g, after the reuse decision
};

// Reuse decision of the G query heads of (b, h): the best candidate over the
// head's search slabs, ordered by (distance, larger T_j, lower slot); the
// head reuses it when its distance is within the threshold.  Fills
// sh.rstart / sh.rslot; with `report`, also writes the optional outputs.
template <int G>
__device__ void reuse_decide(const StepArgs& a, int b, int h, bool report, AttendLds<G>& sh) {
  const ReusePtrs& r = a.ru;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int g = wave; g < G; g += 4) {
    const int bq = b * a.d.Hq + h * G + g;
    uint32_t khi = 0xffffffffu, klo = 0xffffffffu;
    int sl = -1;
    if (lane < r.S) {
      const int4 c = r.cand[(size_t)bq * r.S + lane];
      khi = (uint32_t)c.x;
      klo = ~(uint32_t)c.y;
      sl = c.z;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const uint32_t ohi = __shfl_xor(khi, o), olo = __shfl_xor(klo, o);
      const int os = __shfl_xor(sl, o);
      const bool take = ohi < khi || (ohi == khi && (olo < klo || (olo == klo &&
                                                                   (uint32_t)os < (uint32_t)sl)));
      if (take) { khi = ohi; klo = olo; sl = os; }
    }
    if (lane == 0) {
      const float d2 = __uint_as_float(khi);
      const bool reuse = sl >= 0 && d2 <= r.max_d2;
      sh.rslot[g] = reuse ? sl : -1;
      sh.rstart[g] = reuse ? (int)~klo : 0;
      if (report) {
        if (r.slot_out) r.slot_out[bq] = reuse ? sl : -1;
        if (r.d2_out) r.d2_out[bq] = sl >= 0 ? d2 : INFINITY;
      }
    }
  }
  __syncthreads();
}

// Merge the per-wave states held in LDS (ml, acc) and store one partial per
// query head at `slot`.
template <int G>
__device__ void block_merge_store(AttendLds<G>& sh, float* part_base, int n_parts, int slot) {
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * kD; idx += blockDim.x) {
    const int g = idx / kD, dim = idx % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sh.ml[w][g][0]);
    float L = 0.0f, A = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = sh.ml[w][g][0];
        const float f = (mw == -INFINITY) ? 0.0f : exp2f(mw - M);
        L = fmaf(f, sh.ml[w][g][1], L);
        A = fmaf(f, sh.acc[w][g][dim], A);
      }
    }
    float* out = part_base + ((size_t)g * n_parts + slot) * kPart;
    out[4 + dim] = A;
    if (dim == 0) { out[0] = M; out[1] = L; out[2] = 0.0f; out[3] = 0.0f; }
  }
}

// A wave's row-tile state into the block's LDS slot `wave`.
template <int G>
__device__ void tile_state_to_lds(const RowTileState& st, int wave, int col, int j,
                                  AttendLds<G>& sh) {
  if (col < G) {
    if (j == 0) {
      sh.ml[wave][col][0] = st.m;
      sh.ml[wave][col][1] = st.l;
    }
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) sh.acc[wave][col][32 * j + 8 * i + c] = st.acc[c][i];
  }
}


// Split-K exact attention for one (b, h, split): its share of the rows of the
// source SRC (see RowSource).  With kRowsReuse the rows [base, T) (base the
// smallest start of the G heads) go to splits of equal size (at least
// kReuseMinRows rows), and only the n_act splits that have rows run; split 0
// also places each head's
// reused state (or an empty one) in partial n_act and records n_act + 1, the
// number of partials the merge reads.
template <int G, int SRC>
__device__ void exact_block(const StepArgs& a, int bh, int split, AttendLds<G>& sh) {
  const Dims& d = a.d;
  const int b = bh / d.Hkv, h = bh % d.Hkv;
  int n_rows, base = 0, split_rows = 0;
  int s0[G] = {};
  if constexpr (SRC == kRowsIndex) {
    n_rows = min(max(a.ws.n_rows[bh], 0), d.cap);
  } else {
    const int T = min(max(a.ctx[b], 0), d.cap);
    if constexpr (SRC == kRowsReuse) {
      reuse_decide<G>(a, b, h, split == 0, sh);
      base = T;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        s0[g] = min(sh.rstart[g], T);
        base = min(base, s0[g]);
      }
      // short suffixes still spread over several blocks: at least
      // kReuseMinRows rows per split, at most the grid's splits
      const int n_sfx = T - base;
      const int rows = max(kReuseMinRows, (n_sfx + d.n_exact_splits - 1) / d.n_exact_splits);
      const int n_act = (n_sfx + rows - 1) / rows;
      split_rows = rows;
      if (split == 0) {
        const ReusePtrs& r = a.ru;
        float* pb = a.ws.partials + ((size_t)b * d.Hq + h * G) * d.n_parts * kPart;
        for (int i = threadIdx.x; i < G * kPart; i += blockDim.x) {
          const int g = i / kPart, e = i % kPart;
          const int sl = sh.rslot[g];
          float v = e == 0 ? -INFINITY : 0.0f;
          if (sl >= 0) v = r.st[((size_t)(b * d.Hq + h * G + g) * r.W + sl) * kPart + e];
          pb[((size_t)g * d.n_parts + n_act) * kPart + e] = v;
        }
        if (threadIdx.x == 0) a.ws.n_rows[bh] = n_act + 1;
      }
      if (split >= n_act) return;   // no rows for this split (uniform per block)
    }
    n_rows = T - base;
  }
  int r0, r1;
  if constexpr (SRC == kRowsReuse) {
    r0 = base + split * split_rows;
    r1 = min(base + n_rows, r0 + split_rows);
  } else {
    const int chunk = (n_rows + d.n_exact_splits - 1) / d.n_exact_splits;
    r0 = base + min(n_rows, split * chunk);
    r1 = base + min(n_rows, split * chunk + chunk);
  }
  // row tiles: the rows of a phase are staged as cache offsets in LDS; wave
  // w takes the phase's tiles w, w + 4, ..., the next tile's loads in flight
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15, j = lane >> 4;
  // the first position this lane's column (query head) attends to: a head
  // that reuses a prefix starts after it
  int start = 0;
  if constexpr (SRC == kRowsReuse) {
#pragma unroll
    for (int g = 0; g < G; ++g)
      if (col == g) start = s0[g];
  }
  bf16x8 qb[4];
  tile_query<G>(a.q + ((size_t)b * d.Hq + h * G) * kD, col, j, qb);
  RowTileState st;
  tile_init(st);
  const int32_t* tab = a.table + (size_t)b * d.max_pages;
  const int32_t* rows = a.ws.rows + (size_t)bh * d.cap;
  for (int ph = r0; ph < r1; ph += kPhaseRows) {
    const int n = min(kPhaseRows, r1 - ph);
    if ((int)threadIdx.x < n) {
      const int p = SRC != kRowsIndex ? ph + (int)threadIdx.x
                                      : min(max(rows[ph + threadIdx.x], 0), d.cap - 1);
      int page = tab[p >> 4];
      page = min(max(page, 0), d.num_pages - 1);
      sh.row_off[threadIdx.x] =
          ((long long)(page * kPage + (p & (kPage - 1))) * d.Hkv + h) * kD;
    }
    __syncthreads();
    const int nt = (n + 15) / 16;
    // K[row col] 64 bytes at 32j, V[row 4j + i] 16 bytes at 8 col; rows past
    // the phase load nothing
    auto load_tile = [&](int t, uint4 (&kb)[4], uint4 (&vb)[4]) {
      const int rk = 16 * t + col;
      if (rk < n) {
        const uint16_t* kr = a.kc + sh.row_off[rk] + 32 * j;
#pragma unroll
        for (int c = 0; c < 4; ++c) kb[c] = *reinterpret_cast<const uint4*>(kr + 8 * c);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) kb[c] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rv = 16 * t + 4 * j + i;
        vb[i] = rv < n ? *reinterpret_cast<const uint4*>(a.vc + sh.row_off[rv] + 8 * col)
                       : make_uint4(0, 0, 0, 0);
      }
    };
    uint4 kb[2][4], vb[2][4];
    int t = wave;
    if (t < nt) load_tile(t, kb[0], vb[0]);
    auto step = [&](uint4 (&kc)[4], uint4 (&vc)[4], uint4 (&kn)[4], uint4 (&vn)[4]) {
      if (t + 4 < nt) load_tile(t + 4, kn, vn);
      const f32x4 sv = tile_logits(qb, kc, d.scale_log2);
      float s[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rv = 16 * t + 4 * j + i;
        // the logit of row 4j + i for query head `col`: kept if the head
        // takes the row (past its reused prefix, if any); the V slice
        // (dims 8 col ..) serves every head, rows past the phase hold zeros
        const bool ok = rv < n && (SRC != kRowsReuse || ph + rv >= start);
        s[i] = ok ? sv[i] : -INFINITY;
      }
      tile_accumulate(st, s, vc);
      t += 4;
    };
    while (t < nt) {
      step(kb[0], vb[0], kb[1], vb[1]);
      if (t >= nt) break;
      step(kb[1], vb[1], kb[0], vb[0]);
    }
    __syncthreads();
  }
  tile_finish(st);
  tile_state_to_lds<G>(st, wave, col, j, sh);
  float* part_base = a.ws.partials + ((size_t)b * d.Hq + h * G) * d.n_parts * kPart;
  block_merge_store<G>(sh, part_base, d.n_parts, split);
}

// Background partial for the clusters of one (b, h, split): per cluster the
// candidates' summed weight minus the selected ones', times the cluster mean.
// Wave w handles bg_per_wave consecutive clusters in batches of 4 whose loads
// are issued together.
template <int G>
__device__ void background_block(const StepArgs& a, int bh, int split, AttendLds<G>& sh) {
  constexpr int NB = kBgBatch;
  const Dims& d = a.d;
  const int b = bh / d.Hkv, h = bh % d.Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int cw0 = (split * kBgWaves + wave) * d.bg_per_wave;
  // without the background term every background partial is empty
  const int cw1 = d.exact_only ? cw0 : min(d.L, cw0 + d.bg_per_wave);
  float M[G], Lw[G], acc[G][2];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    M[g] = -INFINITY;
    Lw[g] = 0.0f;
    acc[g][0] = acc[g][1] = 0.0f;
  }
  for (int cb = cw0; cb < cw1; cb += NB) {
    float2 mu[NB];
    float Mc[NB][G], Wc[NB][G];
    unsigned long long Ws[NB][G];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int c = cb + i;
      mu[i] = make_float2(0.0f, 0.0f);
#pragma unroll
      for (int g = 0; g < G; ++g) { Mc[i][g] = -INFINITY; Wc[i][g] = 0.0f; Ws[i][g] = 0ull; }
      if (c < cw1) {
        mu[i] = *reinterpret_cast<const float2*>(a.ix.means + ((size_t)bh * d.L + c) * kD + 2 * lane);
        const float* bin = a.ws.bins + ((size_t)bh * d.L + c) * G * 2;
        const unsigned long long* ws = a.ws.wsel + ((size_t)bh * d.L + c) * G;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          Mc[i][g] = bin[2 * g];
          Wc[i][g] = bin[2 * g + 1];
          Ws[i][g] = ws[g];
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const float wb = fmaxf(Wc[i][g] - (float)Ws[i][g] * kFixInv, 0.0f);
        if (wb > 0.0f) {
          float Mn, f0, f1;
          lse_factors(M[g], Mc[i][g], &Mn, &f0, &f1);
          const float w = f1 * wb;
          Lw[g] = fmaf(Lw[g], f0, w);
          acc[g][0] = fmaf(acc[g][0], f0, w * mu[i].x);
          acc[g][1] = fmaf(acc[g][1], f0, w * mu[i].y);
          M[g] = Mn;
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (lane == 0) { sh.ml[wave][g][0] = M[g]; sh.ml[wave][g][1] = Lw[g]; }
    sh.acc[wave][g][2 * lane] = acc[g][0];
    sh.acc[wave][g][2 * lane + 1] = acc[g][1];
  }
  float* part_base = a.ws.partials + ((size_t)b * d.Hq + h * G) * d.n_parts * kPart;
  block_merge_store<G>(sh, part_base, d.n_parts, d.n_exact_splits + split);
}

// ---------------------------------------------------------------- dense split-K
// Dense decode attention of one (b, h), split over the context: the head's
// W = 4 * splits waves (4 per block) take its pages (16 tokens each, one row
// tile) in turn, wave w the pages w, w + W, w + 2W, ..., so that at any moment
// the head's waves read neighbouring pages, and with every head progressing
// alike the heads' rows of a page (interleaved in the cache) are read at about
// the same time.  Each wave keeps the next page's K and V in flight while the
// row-tile MFMAs compute the current; K is read in 64-byte runs per lane, V in
// whole 256-byte rows per 16 lanes.  The block merges its four waves into one
// partial per query head.
template <int G>
__global__ __launch_bounds__(256) void k_dense_mfma(StepArgs a) {
  __shared__ AttendLds<G> sh;
  const Dims& d = a.d;
  const int BH = d.B * d.Hkv;
  int bh, split;
  xcd_map(blockIdx.x, BH, d.n_exact_splits, &bh, &split);
  const int b = bh / d.Hkv, h = bh % d.Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, j = lane >> 4;
  const int T = min(max(a.ctx[b], 0), d.cap);
  const int n_tiles = (T + kPage - 1) / kPage;
  const int nwh = d.n_exact_splits * 4;   // waves of the head
  bf16x8 qb[4];
  tile_query<G>(a.q + ((size_t)b * d.Hq + h * G) * kD, col, j, qb);
  const int32_t* tab = a.table + (size_t)b * d.max_pages;
  const size_t rstride = (size_t)d.Hkv * kD;   // elements between a page's token rows
  // a page's loads: K[slot col][32j .. 32j + 32) and V[slot 4j + i][8 col .. + 8]
  auto load_tile = [&](int tile, uint4 (&kb)[4], uint4 (&vb)[4]) {
    const int page = min(max(tab[tile], 0), d.num_pages - 1);
    const uint16_t* kr = a.kc + ((size_t)page * kPage + col) * rstride + (size_t)h * kD + 32 * j;
#pragma unroll
    for (int c = 0; c < 4; ++c) kb[c] = *reinterpret_cast<const uint4*>(kr + 8 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      vb[i] = *reinterpret_cast<const uint4*>(
          a.vc + ((size_t)page * kPage + 4 * j + i) * rstride + (size_t)h * kD + 8 * col);
  };
  RowTileState st;
  tile_init(st);
  uint4 kb[2][4], vb[2][4];
  int tile = split * 4 + wave;
  if (tile < n_tiles) load_tile(tile, kb[0], vb[0]);
  auto step = [&](uint4 (&kc)[4], uint4 (&vc)[4], uint4 (&kn)[4], uint4 (&vn)[4]) {
    const int next = tile + nwh;
    if (next < n_tiles) load_tile(next, kn, vn);
    const f32x4 sv = tile_logits(qb, kc, d.scale_log2);
    const int tok0 = tile * kPage + 4 * j;
    float s[4], v[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // rows past the context hold whatever the page does
      const bool ok = tok0 + i < T;
      s[i] = ok ? sv[i] : -INFINITY;
      bf16x8_to_f32(ok ? vc[i] : make_uint4(0, 0, 0, 0), v[i]);
    }
    tile_accumulate_fp32mfma(st, s, v);
    tile = next;
  };
  while (tile < n_tiles) {
    step(kb[0], vb[0], kb[1], vb[1]);
    if (tile >= n_tiles) break;
    step(kb[1], vb[1], kb[0], vb[0]);
  }
  tile_finish(st);
  tile_state_to_lds<G>(st, wave, col, j, sh);
  float* part_base = a.ws.partials + ((size_t)b * d.Hq + h * G) * d.n_parts * kPart;
  block_merge_store<G>(sh, part_base, d.n_parts, split);
}

// One launch for both: blocks [0, BH*n_exact) do split-K, the rest background.
template <int G, int SRC>
__global__ __launch_bounds__(256) void k_attend(StepArgs a) {
  __shared__ AttendLds<G> sh;
  const int BH = a.d.B * a.d.Hkv;
  const int n_exact_blocks = BH * a.d.n_exact_splits;
  const int blk = blockIdx.x;
  int bh, sub;
  if (blk < n_exact_blocks) {
    xcd_map(blk, BH, a.d.n_exact_splits, &bh, &sub);
    exact_block<G, SRC>(a, bh, sub, sh);
  } else if constexpr (SRC == kRowsIndex) {
    xcd_map(blk - n_exact_blocks, BH, a.d.n_bg_splits, &bh, &sub);
    background_block<G>(a, bh, sub, sh);
  }
}

// Log-sum-exp merge of one query head's n_parts partials into O and the
// log-sum-exp.  grid (B*Hq), 128 x NG threads = NG groups of the parts (2, 4
// or 8, more for more parts) x 128 dims.  The parts' maxima and sums are
// staged in LDS; each thread then sums its dim over its group's parts,
// issuing 16 loads before using any, and the groups' sums add pairwise.
template <int NG>
__global__ __launch_bounds__(128 * NG) void k_merge(StepArgs a) {
  constexpr int NW = 2 * NG;
  extern __shared__ float mlds[];   // [np] weights, [np] sums, [NG][128] the groups' sums
  __shared__ float red[2 * NW];
  const int G = a.d.G;
  int bh, g;
  xcd_map(blockIdx.x, a.d.B * a.d.Hkv, G, &bh, &g);
  // query reuse merges only the partials its attention wrote
  const int np = a.ru.st ? min(max(a.ws.n_rows[bh], 1), a.d.n_parts) : a.d.n_parts;
  const int bq = (bh / a.d.Hkv) * a.d.Hq + (bh % a.d.Hkv) * G + g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* part = a.ws.partials + (size_t)bq * a.d.n_parts * kPart;
  float* wts = mlds;
  float* ls = mlds + np;
  float* gsum = mlds + 2 * np;
  // this thread's output dim of its group's first kPre partials is loaded
  // right after the (m, l) pairs, before anything waits on them, so that
  // the merge takes one round of loads (two where a group has more)
  constexpr int kPre = 32;
  const int dim = tid & (kD - 1), grp = tid >> 7;
  const int hp = (np + NG - 1) / NG;
  const int i0 = grp * hp, i1 = min(np, i0 + hp);
  const float* pd = part + 4 + dim;
  float mv = -INFINITY, lv = 0.0f;
  const bool has_ml = tid < np;
  if (has_ml) {
    mv = part[(size_t)tid * kPart];
    lv = part[(size_t)tid * kPart + 1];
  }
  float xp[kPre];
#pragma unroll
  for (int u = 0; u < kPre; ++u) xp[u] = (i0 + u < i1) ? pd[(size_t)(i0 + u) * kPart] : 0.0f;
  float mx = -INFINITY;
  if (has_ml) {
    wts[tid] = mv;
    ls[tid] = lv;
    mx = mv;
  }
  for (int i = tid + blockDim.x; i < np; i += blockDim.x) {
    const float m = part[(size_t)i * kPart];
    wts[i] = m;
    ls[i] = part[(size_t)i * kPart + 1];
    mx = fmaxf(mx, m);
  }
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, red[w]);
  float lsum = 0.0f;
  for (int i = tid; i < np; i += blockDim.x) {
    const float m = wts[i];
    const float f = (m == -INFINITY || M == -INFINITY) ? 0.0f : exp2f(m - M);
    wts[i] = f;
    lsum = fmaf(f, ls[i], lsum);
  }
  lsum = wave_sum(lsum);
  __syncthreads();
  if (lane == 0) red[NW + wave] = lsum;
  __syncthreads();
  // pairwise over the waves, neighbours first
  float t[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) t[w] = red[NW + w];
#pragma unroll
  for (int n = NW; n > 1; n >>= 1)
#pragma unroll
    for (int w = 0; w < n / 2; ++w) t[w] = t[2 * w] + t[2 * w + 1];
  const float L = t[0];
  float A[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < kPre; ++u)
    if (i0 + u < i1) A[u & 3] = fmaf(wts[i0 + u], xp[u], A[u & 3]);
  for (int i = i0 + kPre; i < i1; i += 16) {
    float x[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) x[u] = (i + u < i1) ? pd[(size_t)(i + u) * kPart] : 0.0f;
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (i + u < i1) A[u & 3] = fmaf(wts[i + u], x[u], A[u & 3]);
  }
  gsum[grp * kD + dim] = (A[0] + A[1]) + (A[2] + A[3]);
  __syncthreads();
  if (grp == 0) {
#pragma unroll
    for (int n = NG; n > 1; n >>= 1)
#pragma unroll
      for (int k = 0; k < n / 2; ++k) gsum[k * kD + dim] += gsum[(k + n / 2) * kD + dim];
    const float tot = gsum[dim];
    // no rows at all: O = 0, lse = -inf; a NaN sum stays NaN (never hidden)
    a.out[(size_t)bq * kD + dim] = L != 0.0f ? tot / L : 0.0f;
    if (dim == 0 && a.lse) a.lse[bq] = L != 0.0f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
    if (a.ru.st) {
      // query reuse: this step's state goes into the head's ring
      const int w = (int)((uint32_t)a.ru.cnt[bq] % (uint32_t)a.ru.W);
      float* dst = a.ru.st + ((size_t)bq * a.ru.W + w) * kPart;
      dst[4 + dim] = tot;
      if (dim == 0) { dst[0] = M; dst[1] = L; dst[2] = 0.0f; dst[3] = 0.0f; }
      if (dim < kD / 8)
        *reinterpret_cast<uint4*>(a.ru.qs + ((size_t)bq * a.ru.W + w) * kD + dim * 8) =
            *reinterpret_cast<const uint4*>(a.ru.q_search + (size_t)bq * kD + dim * 8);
    }
  }
  if (a.ru.st) {
    __syncthreads();   // every thread has read the count
    if (tid == 0) {
      const int c = a.ru.cnt[bq];
      const int b = bh / a.d.Hkv;
      a.ru.tj[(size_t)bq * a.ru.W + (uint32_t)c % (uint32_t)a.ru.W] =
          min(max(a.ctx[b], 0), a.d.cap);
      a.ru.cnt[bq] = c + 1;
    }
  }
}

template <int G>
static hipError_t attend_g(const StepArgs& a, bool dense, const Launch& l) {
  const int BH = a.d.B * a.d.Hkv;
  if (dense)
    return launch_kernel(k_dense_mfma<G>, dim3(BH * a.d.n_exact_splits), dim3(256), 0, l, a);
  return launch_kernel(k_attend<G, kRowsIndex>, dim3(BH * (a.d.n_exact_splits + a.d.n_bg_splits)),
                       dim3(256), 0, l, a);
}

template <int G>
static hipError_t attend_reuse_g(const StepArgs& a, const Launch& l) {
  const int BH = a.d.B * a.d.Hkv;
  return launch_kernel(k_attend<G, kRowsReuse>, dim3(BH * a.d.n_exact_splits), dim3(256), 0, l, a);
}

#define PQHSA_G_DISPATCH2(fn, ...)                  \
  switch (a.d.G) {                                  \
    case 1: return fn<1>(__VA_ARGS__);              \
    case 2: return fn<2>(__VA_ARGS__);              \
    case 4: return fn<4>(__VA_ARGS__);              \
    case 8: return fn<8>(__VA_ARGS__);              \
  }                                                 \
  return hipErrorInvalidValue;

hipError_t launch_exact_and_background(const StepArgs& a, bool dense, const Launch& l) {
  PQHSA_G_DISPATCH2(attend_g, a, dense, l)
}

hipError_t launch_exact_reuse(const StepArgs& a, const Launch& l) {
  PQHSA_G_DISPATCH2(attend_reuse_g, a, l)
}

hipError_t launch_merge(const StepArgs& a, const Launch& l) {
  // groups of the parts: at most 32 parts per thread
  const int ng = a.d.n_parts <= 64 ? 2 : a.d.n_parts <= 128 ? 4 : 8;
  const size_t lds = ((size_t)2 * a.d.n_parts + (size_t)ng * kD) * sizeof(float);
  auto kern = ng == 2 ? k_merge<2> : ng == 4 ? k_merge<4> : k_merge<8>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  return launch_kernel(kern, dim3(a.d.B * a.d.Hq), dim3(kD * ng), lds, l, a);
}

}  // namespace pqhsa
