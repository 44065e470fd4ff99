// Exact split-K attention over paged bf16 K/V, the per-cluster background
// term, and the log-sum-exp merge.
//
// PQ-HSA page (rit.work blog), section "How approximate estimates return the
// discarded context": selected, first and recent tokens are read from the
// original (paged) KV cache and computed exactly (fourth and sixth
// paragraphs); unread tokens contribute their approximate weight summed per
// cluster times the cluster mean (fifth paragraph).  The merge is the
// prefix/suffix law O = (N_P + N_S)/(D_P + D_S) of the quant_prune_distill
// post on query reuse, over all partials.  Dense and sparse modes share the
// split-K kernel, as the activation/KV-sparsity crossover article (rit.work
// blog, section "Why one method gives different speed-ups") requires of an
// honest baseline.  The same split-K kernel also serves query reuse: each
// query head starts at the context length of the earlier query whose prefix
// state it reuses (0 when it reuses none), and the reused state joins the
// merge as one more partial.
//
// Split-K block: 256 threads = 16 row groups of 16 lanes (one DPP row each).
// The block first stages the cache offsets of up to 256 rows in LDS (row list
// and block table read once, in parallel); each row group then streams its
// rows with the next two rows' K and V (16 B per lane, 256 B per row) in
// flight while it computes the current two: the G dot products use a 16-lane
// DPP reduction, and an online base-2 softmax (max, sum, acc[8 dims]) is kept
// per query head.  Row groups of a wave merge through lane shuffles, the 4
// waves through LDS, and the block writes one partial (m, l, acc[128]) per
// query head.
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
  kRowsDense = 1,   // the whole context [0, T)
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
  const int l16 = threadIdx.x & 15;
  const int rg = threadIdx.x >> 4;
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
  // heads that take row `p` (all of them unless some reuse a prefix)
  auto act = [&](int p) -> uint32_t {
    if constexpr (SRC != kRowsReuse) return 0xffu;
    uint32_t m = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) m |= (uint32_t)(p >= s0[g]) << g;
    return m;
  };

  float qv[G][8];
  {
    const uint16_t* q = a.q + ((size_t)b * d.Hq + h * G) * kD + l16 * 8;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint4 w = *reinterpret_cast<const uint4*>(q + g * kD);
      const float f[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                          bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[g][i] = f[i] * d.scale_log2;
    }
  }
  AttnState<G> st;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.m[g] = -INFINITY;
    st.l[g] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) st.acc[g][i] = 0.0f;
  }
  const int32_t* tab = a.table + (size_t)b * d.max_pages;
  const int32_t* rows = a.ws.rows + (size_t)bh * d.cap;
  const uint16_t* kc = a.kc + l16 * 8;
  const uint16_t* vc = a.vc + l16 * 8;
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
    // rows j and j + 16 of the group per pair; two pairs' buffers alternate
    // (the loop is unrolled by two so that no buffer is copied), the next
    // pair's loads in flight while a pair is computed.  A row past the
    // phase's end loads the phase's last row instead (finite values, weight
    // zero), so that no register needs clearing.
    auto load_pair = [&](int j, uint4 (&kv)[4]) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const long long o = sh.row_off[min(j + 16 * r, n - 1)];
        kv[2 * r] = *reinterpret_cast<const uint4*>(kc + o);
        kv[2 * r + 1] = *reinterpret_cast<const uint4*>(vc + o);
      }
    };
    auto run_pair = [&](int j, const uint4 (&kv)[4]) {
      attend_rows2<G>(st, qv, kv[0], kv[1], kv[2], kv[3], act(ph + j),
                      j + 16 < n ? act(ph + j + 16) : 0u);
    };
    uint4 pa[4], pb[4];
    int j = rg;
    if (j < n) load_pair(j, pa);
    while (j < n) {
      if (j + 32 < n) load_pair(j + 32, pb);
      run_pair(j, pa);
      if (j + 32 >= n) break;
      if (j + 64 < n) load_pair(j + 64, pa);
      run_pair(j + 32, pb);
      j += 64;
    }
    __syncthreads();
  }
  // merge the wave's 4 row groups (lanes l, l^16, l^32, l^48 hold the same dims)
#pragma unroll
  for (int o = 16; o <= 32; o <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(st.m[g], o);
      const float lo = __shfl_xor(st.l[g], o);
      float M, a0, a1;
      lse_factors(st.m[g], mo, &M, &a0, &a1);
      st.l[g] = st.l[g] * a0 + lo * a1;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float ao = __shfl_xor(st.acc[g][i], o);
        st.acc[g][i] = st.acc[g][i] * a0 + ao * a1;
      }
      st.m[g] = M;
    }
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) < 16) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (l16 == 0) { sh.ml[wave][g][0] = st.m[g]; sh.ml[wave][g][1] = st.l[g]; }
#pragma unroll
      for (int i = 0; i < 8; ++i) sh.acc[wave][g][l16 * 8 + i] = st.acc[g][i];
    }
  }
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
// log-sum-exp.  grid (B*Hq), 256 threads = 2 halves of the parts x 128 dims.
// The parts' maxima and sums are staged in LDS; each thread then sums its dim
// over its half of the parts, issuing 16 loads before using any.
__global__ __launch_bounds__(256) void k_merge(StepArgs a) {
  extern __shared__ float mlds[];   // [np] weights, [np] sums, [128] second half's sums
  __shared__ float red[8];
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
  float* half1 = mlds + 2 * np;
  float mx = -INFINITY;
  for (int i = tid; i < np; i += blockDim.x) {
    const float m = part[(size_t)i * kPart];
    wts[i] = m;
    ls[i] = part[(size_t)i * kPart + 1];
    mx = fmaxf(mx, m);
  }
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float lsum = 0.0f;
  for (int i = tid; i < np; i += blockDim.x) {
    const float m = wts[i];
    const float f = (m == -INFINITY || M == -INFINITY) ? 0.0f : exp2f(m - M);
    wts[i] = f;
    lsum = fmaf(f, ls[i], lsum);
  }
  lsum = wave_sum(lsum);
  __syncthreads();
  if (lane == 0) red[4 + wave] = lsum;
  __syncthreads();
  const float L = (red[4] + red[5]) + (red[6] + red[7]);
  const int dim = tid & (kD - 1), half = tid >> 7;
  const int hp = (np + 1) / 2;
  const int i0 = half * hp, i1 = min(np, i0 + hp);
  const float* pd = part + 4 + dim;
  float A[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int i = i0; i < i1; i += 16) {
    float x[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) x[u] = (i + u < i1) ? pd[(size_t)(i + u) * kPart] : 0.0f;
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (i + u < i1) A[u & 3] = fmaf(wts[i + u], x[u], A[u & 3]);
  }
  const float sum = (A[0] + A[1]) + (A[2] + A[3]);
  if (half == 1) half1[dim] = sum;
  __syncthreads();
  if (half == 0) {
    const float tot = sum + half1[dim];
    a.out[(size_t)bq * kD + dim] = L > 0.0f ? tot / L : 0.0f;
    if (dim == 0 && a.lse) a.lse[bq] = L > 0.0f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
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
    return launch_kernel(k_attend<G, kRowsDense>, dim3(BH * a.d.n_exact_splits), dim3(256), 0, l,
                         a);
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
  const size_t lds = ((size_t)2 * a.d.n_parts + kD) * sizeof(float);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_merge),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  return launch_kernel(k_merge, dim3(a.d.B * a.d.Hq), dim3(256), lds, l, a);
}

}  // namespace pqhsa
