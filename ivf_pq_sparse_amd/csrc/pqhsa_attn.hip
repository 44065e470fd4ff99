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
// honest baseline.
//
// Split-K block: 256 threads = 16 row groups of 16 lanes (one DPP row each).
// A row group reads one token's K and V rows (16 B per lane, 256 B per row),
// forms the G dot products with a 16-lane DPP reduction and keeps an online
// base-2 softmax (max, sum, acc[8 dims]) per query head.  Row groups of a
// wave merge through lane shuffles, the 4 waves through LDS, and the block
// writes one partial (m, l, acc[128]) per query head.
#include "pqhsa_internal.hpp"

namespace pqhsa {

template <int G>
struct AttnState {
  float m[G], l[G], acc[G][8];
};

template <int G>
__device__ __forceinline__ void attend_row(AttnState<G>& st, const float (&qv)[G][8], uint4 kw,
                                           uint4 vw) {
  const float kf[8] = {bf16_lo(kw.x), bf16_hi(kw.x), bf16_lo(kw.y), bf16_hi(kw.y),
                       bf16_lo(kw.z), bf16_hi(kw.z), bf16_lo(kw.w), bf16_hi(kw.w)};
  const float vf[8] = {bf16_lo(vw.x), bf16_hi(vw.x), bf16_lo(vw.y), bf16_hi(vw.y),
                       bf16_lo(vw.z), bf16_hi(vw.z), bf16_lo(vw.w), bf16_hi(vw.w)};
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float s = qv[g][0] * kf[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) s = fmaf(qv[g][i], kf[i], s);
    s = row16_sum(s);
    const float mn = fmaxf(st.m[g], s);
    const float al = exp2f(st.m[g] - mn);
    const float p = exp2f(s - mn);
    st.l[g] = fmaf(st.l[g], al, p);
#pragma unroll
    for (int i = 0; i < 8; ++i) st.acc[g][i] = fmaf(st.acc[g][i], al, p * vf[i]);
    st.m[g] = mn;
  }
}

// Merge (m1, w1) into (m0, w0) style states: returns the two scale factors.
__device__ __forceinline__ void lse_factors(float m0, float m1, float* M, float* a0, float* a1) {
  *M = fmaxf(m0, m1);
  *a0 = (m0 == -INFINITY) ? 0.0f : exp2f(m0 - *M);
  *a1 = (m1 == -INFINITY) ? 0.0f : exp2f(m1 - *M);
}

// LDS scratch of the block-level merge: 4 waves x G heads x (m, l, acc[128]).
template <int G>
struct MergeLds {
  float ml[4][G][2];
  float acc[4][G][kD];
};

// Write (m, l, acc) of the 4 waves' lanes 0..15 (8 dims each) to LDS, merge
// and store one partial per query head at `slot`.
template <int G>
__device__ void block_merge_store(MergeLds<G>& sh, const float* m, const float* l,
                                  const float (*acc)[8], int l16, bool writer, float* part_base,
                                  int n_parts, int slot) {
  const int wave = threadIdx.x >> 6;
  if (writer) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (l16 == 0) { sh.ml[wave][g][0] = m[g]; sh.ml[wave][g][1] = l[g]; }
#pragma unroll
      for (int i = 0; i < 8; ++i) sh.acc[wave][g][l16 * 8 + i] = acc[g][i];
    }
  }
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

// Split-K exact attention for one (b, h, split): rows [r0, r1) of either the
// index-list row array (DENSE = false) or the whole context (DENSE = true).
template <int G, bool DENSE>
__device__ void exact_block(const StepArgs& a, int bh, int split, MergeLds<G>& sh) {
  const Dims& d = a.d;
  const int b = bh / d.Hkv, h = bh % d.Hkv;
  const int l16 = threadIdx.x & 15;
  const int rg = threadIdx.x >> 4;
  int n_rows;
  if constexpr (DENSE) n_rows = min(max(a.ctx[b], 0), d.cap);
  else n_rows = a.ws.n_rows[bh];
  const int chunk = (n_rows + d.n_exact_splits - 1) / d.n_exact_splits;
  const int r0 = min(n_rows, split * chunk);
  const int r1 = min(n_rows, r0 + chunk);

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
  const int32_t* rows = DENSE ? nullptr : a.ws.rows + (size_t)bh * d.cap;
  auto row_offset = [&](int r) -> size_t {
    const int p = DENSE ? r : rows[r];
    int page = tab[p >> 4];
    page = min(max(page, 0), d.num_pages - 1);
    return ((size_t)(page * kPage + (p & (kPage - 1))) * d.Hkv + h) * kD + l16 * 8;
  };
  int r = r0 + rg;
  // two rows per step so that four 16-byte loads per lane are in flight
  for (; r + 16 < r1; r += 32) {
    const size_t o0 = row_offset(r), o1 = row_offset(r + 16);
    const uint4 k0 = *reinterpret_cast<const uint4*>(a.kc + o0);
    const uint4 v0 = *reinterpret_cast<const uint4*>(a.vc + o0);
    const uint4 k1 = *reinterpret_cast<const uint4*>(a.kc + o1);
    const uint4 v1 = *reinterpret_cast<const uint4*>(a.vc + o1);
    attend_row<G>(st, qv, k0, v0);
    attend_row<G>(st, qv, k1, v1);
  }
  if (r < r1) {
    const size_t o0 = row_offset(r);
    const uint4 k0 = *reinterpret_cast<const uint4*>(a.kc + o0);
    const uint4 v0 = *reinterpret_cast<const uint4*>(a.vc + o0);
    attend_row<G>(st, qv, k0, v0);
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
  float* part_base = a.ws.partials + ((size_t)b * d.Hq + h * G) * d.n_parts * kPart;
  block_merge_store<G>(sh, st.m, st.l, st.acc, l16, (threadIdx.x & 63) < 16, part_base,
                       d.n_parts, split);
}

// Background partial for clusters [c0, c1) of (b, h): per cluster the
// candidates' summed weight minus the selected ones' weight, times the mean.
template <int G>
__device__ void background_block(const StepArgs& a, int bh, int split, MergeLds<G>& sh) {
  const Dims& d = a.d;
  const int b = bh / d.Hkv, h = bh % d.Hkv;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int per = (d.L + d.n_bg_splits - 1) / d.n_bg_splits;
  const int c0 = min(d.L, split * per), c1 = min(d.L, c0 + per);
  const int32_t* off = a.ix.list_off + (size_t)bh * (d.L + 1);
  const uint4* codes = reinterpret_cast<const uint4*>(a.ix.codes + (size_t)bh * d.cap * kM);
  const uint32_t* sel_e = a.ws.sel_e + (size_t)bh * d.nwords;
  const float* lut = a.ws.lut + (size_t)bh * kM * kKsub * G;
  float M[G], Lw[G], acc[G][2];
#pragma unroll
  for (int g = 0; g < G; ++g) { M[g] = -INFINITY; Lw[g] = 0.0f; acc[g][0] = acc[g][1] = 0.0f; }
  for (int c = c0 + wave; c < c1; c += 4) {
    const float* bin = a.ws.bins + ((size_t)bh * d.L + c) * G * 2;
    float Mc[G], Wc[G], qc[G];
    bool any = false;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      Mc[g] = bin[2 * g];
      Wc[g] = bin[2 * g + 1];
      qc[g] = a.ws.qc[((size_t)bh * d.L + c) * G + g];
      any |= Wc[g] > 0.0f;
    }
    if (!any) continue;
    const int e1 = min(off[c + 1], d.cap), e0 = min(max(off[c], 0), e1);
    float wsel[G];
#pragma unroll
    for (int g = 0; g < G; ++g) wsel[g] = 0.0f;
    for (int eb = e0; eb < e1; eb += 64) {
      const int e = eb + lane;
      bool sel = false;
      if (e < e1) sel = (sel_e[e >> 5] >> (e & 31)) & 1u;
      if (sel) {
        float s[G];
        entry_logits<G>(lut, qc, codes[e], s);
#pragma unroll
        for (int g = 0; g < G; ++g) wsel[g] += exp2f(s[g] - Mc[g]);
      }
    }
    const float2 mu = *reinterpret_cast<const float2*>(a.ix.means + ((size_t)bh * d.L + c) * kD + 2 * lane);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float wb = fmaxf(Wc[g] - wave_sum(wsel[g]), 0.0f);
      if (wb > 0.0f) {
        float Mn, f0, f1;
        lse_factors(M[g], Mc[g], &Mn, &f0, &f1);
        const float w = f1 * wb;
        Lw[g] = fmaf(Lw[g], f0, w);
        acc[g][0] = fmaf(acc[g][0], f0, w * mu.x);
        acc[g][1] = fmaf(acc[g][1], f0, w * mu.y);
        M[g] = Mn;
      }
    }
  }
  // store through the same LDS merge: lanes hold dims (2*lane, 2*lane+1)
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (lane == 0) { sh.ml[wave][g][0] = M[g]; sh.ml[wave][g][1] = Lw[g]; }
    sh.acc[wave][g][2 * lane] = acc[g][0];
    sh.acc[wave][g][2 * lane + 1] = acc[g][1];
  }
  float* part_base = a.ws.partials + ((size_t)b * d.Hq + h * G) * d.n_parts * kPart;
  // writer=false: LDS already filled above
  const float dummy_acc[G][8] = {};
  block_merge_store<G>(sh, M, Lw, dummy_acc, 0, false, part_base, d.n_parts,
                       d.n_exact_splits + split);
}

// One launch for both: blocks [0, BH*n_exact) do split-K, the rest background.
template <int G, bool DENSE>
__global__ __launch_bounds__(256) void k_attend(StepArgs a) {
  __shared__ MergeLds<G> sh;
  const int BH = a.d.B * a.d.Hkv;
  const int n_exact_blocks = BH * a.d.n_exact_splits;
  const int blk = blockIdx.x;
  if (blk < n_exact_blocks) {
    exact_block<G, DENSE>(a, blk / a.d.n_exact_splits, blk % a.d.n_exact_splits, sh);
  } else if constexpr (!DENSE) {
    const int i = blk - n_exact_blocks;
    background_block<G>(a, i / a.d.n_bg_splits, i % a.d.n_bg_splits, sh);
  }
}

// grid (B*Hq), 128 threads (one per output dim).
__global__ __launch_bounds__(128) void k_merge(StepArgs a) {
  const int bq = blockIdx.x;
  const int dim = threadIdx.x;
  const int np = a.d.n_parts;
  const float* p = a.ws.partials + (size_t)bq * np * kPart;
  float M = -INFINITY;
  for (int i = 0; i < np; ++i) M = fmaxf(M, p[(size_t)i * kPart]);
  float L = 0.0f, A = 0.0f;
  if (M != -INFINITY) {
#pragma unroll 4
    for (int i = 0; i < np; ++i) {
      const float mi = p[(size_t)i * kPart];
      const float f = (mi == -INFINITY) ? 0.0f : exp2f(mi - M);
      L = fmaf(f, p[(size_t)i * kPart + 1], L);
      A = fmaf(f, p[(size_t)i * kPart + 4 + dim], A);
    }
  }
  a.out[(size_t)bq * kD + dim] = L > 0.0f ? A / L : 0.0f;
  if (dim == 0 && a.lse) a.lse[bq] = L > 0.0f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
}

template <int G>
static hipError_t attend_g(const StepArgs& a, bool dense, hipStream_t st) {
  const int BH = a.d.B * a.d.Hkv;
  if (dense) {
    hipLaunchKernelGGL((k_attend<G, true>), dim3(BH * a.d.n_exact_splits), dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((k_attend<G, false>),
                       dim3(BH * (a.d.n_exact_splits + a.d.n_bg_splits)), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_exact_and_background(const StepArgs& a, bool dense, hipStream_t st) {
  switch (a.d.G) {
    case 1: return attend_g<1>(a, dense, st);
    case 2: return attend_g<2>(a, dense, st);
    case 4: return attend_g<4>(a, dense, st);
    case 8: return attend_g<8>(a, dense, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const StepArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_merge, dim3(a.d.B * a.d.Hq), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace pqhsa
