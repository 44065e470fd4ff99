// Per-step PQ-HSA kernels before the exact attention: lookup tables, code
// scan, and the two stages of the budgeted top-k.
//
// PQ-HSA page (rit.work blog), section "How approximate estimates return the
// discarded context": the IVF-PQ index gives an approximate attention logit
// for every indexed token (third paragraph); the same estimates pick the
// tokens read exactly and weight the unread ones (fourth paragraph).  Section
// "The background contribution kept accuracy, and length gave the speed-up"
// names the fixed costs these kernels are: building tables, scanning
// compressed codes, choosing candidates.
//
// Every kernel here is written for latency: the step moves tens of MB, so a
// kernel costs a few dependent memory round trips, and the code issues each
// round's loads together before using any of them.
#include "pqhsa_internal.hpp"

namespace pqhsa {

// ---------------------------------------------------------------- tables
// grid (B*Hkv, 16 + ceil(L/16)), 256 threads.
//   y < 16 : lut[m = y][j = thread][g] = scale*log2e * q_g^(m) . B_m[j]
//   y >= 16: qc[c][g] = scale*log2e * q_g . C_c, one 16-lane row per cluster
// The blocks also clear the step's histogram.
template <int G>
__global__ __launch_bounds__(256) void k_tables(StepArgs a) {
  const Dims& d = a.d;
  const int bh = blockIdx.x;
  const int b = bh / d.Hkv, h = bh % d.Hkv;
  const uint16_t* q = a.q + ((size_t)b * d.Hq + h * G) * kD;
  {
    const int nb = gridDim.y;
    for (int i = blockIdx.y * blockDim.x + threadIdx.x; i < kHistBins; i += nb * blockDim.x)
      a.ws.hist[(size_t)bh * kHistStride + i] = 0;
  }
  if (blockIdx.y < kM) {
    const int m = blockIdx.y;
    const int j = threadIdx.x;
    const float* cw = a.ix.codebooks + (((size_t)bh * kM + m) * kKsub + j) * kDsub;
    const float4 c0 = *reinterpret_cast<const float4*>(cw);
    const float4 c1 = *reinterpret_cast<const float4*>(cw + 4);
    const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    float* out = a.ws.lut + (((size_t)bh * kM + m) * kKsub + j) * G;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint4 w = *reinterpret_cast<const uint4*>(q + g * kD + m * kDsub);
      const float qs[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                           bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
      float s = (qs[0] * d.scale_log2) * cv[0];
#pragma unroll
      for (int i = 1; i < kDsub; ++i) s = fmaf(qs[i] * d.scale_log2, cv[i], s);
      out[g] = s;
    }
  } else {
    const int l16 = threadIdx.x & 15;
    const int c = (blockIdx.y - kM) * 16 + (threadIdx.x >> 4);
    float cv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (c < d.L) {
      const float* cp = a.ix.centroids + ((size_t)bh * d.L + c) * kD + l16 * 8;
      const float4 c0 = *reinterpret_cast<const float4*>(cp);
      const float4 c1 = *reinterpret_cast<const float4*>(cp + 4);
      cv[0] = c0.x; cv[1] = c0.y; cv[2] = c0.z; cv[3] = c0.w;
      cv[4] = c1.x; cv[5] = c1.y; cv[6] = c1.z; cv[7] = c1.w;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint4 w = *reinterpret_cast<const uint4*>(q + g * kD + l16 * 8);
      const float qs[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                           bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
      float s = (qs[0] * d.scale_log2) * cv[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) s = fmaf(qs[i] * d.scale_log2, cv[i], s);
      s = row16_sum(s);
      if (c < d.L && l16 == g) a.ws.qc[((size_t)bh * d.L + c) * G + g] = s;
    }
  }
}

// ---------------------------------------------------------------- scan
// grid (B*Hkv*scan_blocks), 1024 threads, LDS = LUT (16*256*G floats) + 4096
// histogram bins.  A block owns scan_lists consecutive clusters of one (b, h);
// wave w takes clusters w, w+16, ... whole, so a cluster's qc is wave-uniform
// and its bin needs no atomics.  A wave walks its clusters as one stream of
// rounds of P 64-entry tiles, with two register buffers in ping-pong: the
// next round's codes and positions are in flight while the current one is
// computed.  The LUT copy's loads are issued first, then the first round.
// For every entry: base-2 approximate logits of the G query heads, key = max
// over heads in order-preserving bits (0 for non-candidates), one histogram
// count on the key's top 12 bits.  Per round and head the lane keeps a
// running (max, sum of exp2) over candidates: one max over the round, then
// one exp2 per value; the cluster's (max, sum) is reduced over the wave.

template <int G, int P>
struct ScanRound {
  uint4 cw[P];
  int pp[P];
};

template <int G>
__global__ __launch_bounds__(kScanThreads) void k_scan(StepArgs a) {
  // tiles in flight per wave; fewer at G >= 4 to stay within 128 VGPRs
  constexpr int P = G >= 4 ? 2 : 4;
  extern __shared__ float4 smem4[];
  float* lut = reinterpret_cast<float*>(smem4);
  uint32_t* hist = reinterpret_cast<uint32_t*>(lut + kM * kKsub * G);
  const Dims& d = a.d;
  int bh, blk;
  xcd_map(blockIdx.x, d.B * d.Hkv, d.scan_blocks, &bh, &blk);
  const int b = bh / d.Hkv;
  const int lane = threadIdx.x & 63;
  // the wave id as a scalar: all cluster-level control flow is wave-uniform,
  // so the cross-lane reductions below always see every lane
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c_end = min(d.L, (blk + 1) * d.scan_lists);
  const int32_t* off = a.ix.list_off + (size_t)bh * (d.L + 1);
  const uint4* codes = reinterpret_cast<const uint4*>(a.ix.codes + (size_t)bh * d.cap * kM);
  const int32_t* pos = a.ix.pos + (size_t)bh * d.cap;
  uint32_t* keys = a.ws.keys + (size_t)bh * d.cap;
  const float* qcg = a.ws.qc + (size_t)bh * d.L * G;

  auto issue = [&](ScanRound<G, P>& r, int base, int e1) {
#pragma unroll
    for (int t = 0; t < P; ++t) {
      const int e = base + t * 64 + lane;
      r.pp[t] = -1;
      if (e < e1) {
        r.cw[t] = codes[e];
        r.pp[t] = pos[e];
      }
    }
  };

  // LUT copy: its loads go out first, then the cluster offsets and the first
  // round of codes; the LDS writes wait for the LUT only
  constexpr int kPer = kM * kKsub * G / 4 / kScanThreads;
  {
    float4 tmp[kPer];
    const float4* src = reinterpret_cast<const float4*>(a.ws.lut + (size_t)bh * kM * kKsub * G);
#pragma unroll
    for (int i = 0; i < kPer; ++i) tmp[i] = src[i * kScanThreads + threadIdx.x];
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) hist[i] = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) smem4[i * kScanThreads + threadIdx.x] = tmp[i];
  }
  // stream position: cluster c, round base, cluster bounds and qc
  int c = blk * d.scan_lists + wave;
  int e0 = 0, e1 = 0;
  float qc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) qc[g] = 0.0f;
  ScanRound<G, P> rb[2];
  if (c < c_end) {
    e1 = min(off[c + 1], d.cap);
    e0 = min(max(off[c], 0), e1);
#pragma unroll
    for (int g = 0; g < G; ++g) qc[g] = qcg[c * G + g];
    issue(rb[0], e0, e1);
  }
  __syncthreads();
  const SeqInfo si = seq_info(d, a.ctx, a.ix.n_indexed, b);

  float mx[G], sm[G];
#pragma unroll
  for (int g = 0; g < G; ++g) { mx[g] = -INFINITY; sm[g] = 0.0f; }
  int base = e0;
  int cur = 0;
  // one round; returns false when the wave's stream has ended
  auto round = [&](ScanRound<G, P>& now, ScanRound<G, P>& nxt) {
    // the next round: more of this cluster, or the first round of the next one
    int nc = c, nbase = base + 64 * P, ne0 = e0, ne1 = e1;
    float nqc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) nqc[g] = qc[g];
    const bool last = nbase >= e1;
    if (last) {
      nc = c + kScanWaves;
      if (nc < c_end) {
        ne1 = min(off[nc + 1], d.cap);
        ne0 = min(max(off[nc], 0), ne1);
#pragma unroll
        for (int g = 0; g < G; ++g) nqc[g] = qcg[nc * G + g];
      }
      nbase = ne0;
    }
    if (nc < c_end) issue(nxt, nbase, ne1);

    float s[P][G];
#pragma unroll
    for (int t = 0; t < P; ++t) {
      const int p = now.pp[t];
      const int e = base + t * 64 + lane;
#pragma unroll
      for (int g = 0; g < G; ++g) s[t][g] = -INFINITY;
      if (p >= 0) {
        float v[G];
        entry_logits_lds<G>(lut, qc, now.cw[t], v);
        float kappa = v[0];
#pragma unroll
        for (int g = 1; g < G; ++g) kappa = fmaxf(kappa, v[g]);
        const bool cand = p >= si.cand_beg && p < si.cand_end;
        uint32_t key = 0;
        if (cand) {
          key = order_key(kappa);
          atomicAdd(&hist[key >> (32 - kHistBits)], 1u);
#pragma unroll
          for (int g = 0; g < G; ++g) s[t][g] = v[g];
        }
        keys[e] = key;
      }
    }
    // running (max, sum of exp2) per head: one max over the round, then
    // one exp2 per value
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float rm = s[0][g];
#pragma unroll
      for (int t = 1; t < P; ++t) rm = fmaxf(rm, s[t][g]);
      const float Mn = fmaxf(mx[g], rm);
      if (Mn != -INFINITY) {
        float acc = sm[g] * __builtin_amdgcn_exp2f(mx[g] - Mn);
#pragma unroll
        for (int t = 0; t < P; ++t) acc += __builtin_amdgcn_exp2f(s[t][g] - Mn);
        sm[g] = acc;
        mx[g] = Mn;
      }
    }
    if (last) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float M = wave_max(mx[g]);
        const float part = (mx[g] == -INFINITY) ? 0.0f : sm[g] * __builtin_amdgcn_exp2f(mx[g] - M);
        const float S = wave_sum(part);
        if (lane == 0) {
          float* bin = a.ws.bins + (((size_t)bh * d.L + c) * G + g) * 2;
          bin[0] = M;
          bin[1] = S;
        }
        mx[g] = -INFINITY;
        sm[g] = 0.0f;
      }
    }
    c = nc;
    base = nbase;
    e0 = ne0;
    e1 = ne1;
#pragma unroll
    for (int g = 0; g < G; ++g) qc[g] = nqc[g];
  };
  // rounds alternate between the two buffers (no register copies)
  while (c < c_end) {
    round(rb[0], rb[1]);
    if (!(c < c_end)) break;
    round(rb[1], rb[0]);
  }
  (void)cur;
  __syncthreads();
  uint32_t* gh = a.ws.hist + (size_t)bh * kHistStride;
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) {
    const uint32_t v = hist[i];
    if (v) atomicAdd(&gh[i], v);
  }
}

// Approximate base-2 weights of an index entry relative to its cluster's
// max (<= 1 for candidates: the max was taken over them in the scan).
template <int G>
__device__ __forceinline__ void entry_weights(const StepArgs& a, int bh, int e, int c, float* w) {
  const Dims& d = a.d;
  const uint4 cw = reinterpret_cast<const uint4*>(a.ix.codes + (size_t)bh * d.cap * kM)[e];
  float qc[G], s[G];
#pragma unroll
  for (int g = 0; g < G; ++g) qc[g] = a.ws.qc[((size_t)bh * d.L + c) * G + g];
  entry_logits<G>(a.ws.lut + (size_t)bh * kM * kKsub * G, qc, cw, s);
  const float* bin = a.ws.bins + ((size_t)bh * d.L + c) * G * 2;
#pragma unroll
  for (int g = 0; g < G; ++g) w[g] = exp2f(s[g] - bin[2 * g]);
}

// Add weights to a cluster's fixed-point sums of selected weights (integer
// adds: the sums do not depend on the order in which entries arrive).  `ws`
// is the LDS or global array [L][G].
template <int G>
__device__ __forceinline__ void add_fixed(unsigned long long* ws, int c, const float* w) {
#pragma unroll
  for (int g = 0; g < G; ++g)
    atomicAdd(&ws[c * G + g], (unsigned long long)(w[g] * kFixScale + 0.5f));
}

__device__ __forceinline__ int entry_cluster(const StepArgs& a, int bh, int e) {
  return min(max(a.ix.ent_list[(size_t)bh * a.d.cap + e], 0), a.d.L - 1);
}

// ---------------------------------------------------------------- select
// One block per (b, h), after the collect kernel.  Marks the
// above-threshold positions in an LDS bitmap over positions, resolves the
// threshold bucket exactly with an 8-bit radix select over 52-bit composites
// (the key's low 20 bits, then the bit-inverted position, so equal keys prefer
// the lower position), adds the tie winners' precomputed weights to their
// clusters, then compacts the bitmap into the ascending exact-row list: sink
// rows, selected rows, recent/tail rows.
constexpr int kWinCap = 2048;   // tie winners listed in LDS before their weight updates
constexpr size_t kWselLdsBytes = 64 * 1024;   // per-cluster selected weights kept in LDS up to this

struct SelectLds {
  int sh[8];
  uint32_t rh[256];
  int res[3];
  int n_win;
  int pre_a[kMaxSparseContext / kCollectEntries + 1];
  int pre_t[kMaxSparseContext / kCollectEntries + 1];
};

template <int G>
__device__ void select_head(const StepArgs& a, int bh, const SeqInfo& si, unsigned char* dyn,
                            SelectLds& L) {
  const Dims& d = a.d;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int nw = d.nwords;
  uint32_t* pbit = reinterpret_cast<uint32_t*>(dyn);
  uint2* win = reinterpret_cast<uint2*>(dyn + ((size_t)nw * 4 + 15) / 16 * 16);
  // selected weights per cluster: accumulated in LDS when they fit, else in
  // the global array (cleared here first)
  const int nwsel = d.L * G;
  const bool wsel_lds = (size_t)nwsel * 8 <= kWselLdsBytes;
  unsigned long long* wacc =
      wsel_lds ? reinterpret_cast<unsigned long long*>(reinterpret_cast<unsigned char*>(win) +
                                                        kWinCap * sizeof(uint2))
               : a.ws.wsel + (size_t)bh * nwsel;
  for (int i = tid; i < nw; i += nthr) pbit[i] = 0u;
  for (int i = tid; i < nwsel; i += nthr) wacc[i] = 0ull;
  if (tid == 0) L.n_win = 0;
  if (!wsel_lds) __threadfence_block();
  // k is reached by the above-bucket keys plus some of the threshold
  // bucket's; with fewer candidates than k (dropped entries) all are taken
  int ksel = 0;
  if (si.k > 0) {
    const int nseg = d.collect_slices;
    // exclusive prefix over the collect segments (at most 256: one wave, 4 per lane)
    if (tid < 64) {
      int ca[4], ct[4], sa = 0, st = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int sgi = tid * 4 + i;
        ca[i] = ct[i] = 0;
        if (sgi < nseg) {
          const int2 cnt = *reinterpret_cast<const int2*>(
              a.ws.seg_cnt + ((size_t)bh * d.collect_slices + sgi) * 2);
          ca[i] = cnt.x;
          ct[i] = cnt.y;
        }
        sa += ca[i];
        st += ct[i];
      }
      int xa = sa, xt = st;
      for (int o = 1; o < 64; o <<= 1) {
        const int ya = __shfl_up(xa, o), yt = __shfl_up(xt, o);
        if (tid >= o) { xa += ya; xt += yt; }
      }
      int ra = xa - sa, rt = xt - st;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int sgi = tid * 4 + i;
        if (sgi < nseg) { L.pre_a[sgi] = ra; L.pre_t[sgi] = rt; }
        ra += ca[i];
        rt += ct[i];
      }
      if (tid == 63) { L.pre_a[nseg] = xa; L.pre_t[nseg] = xt; }   // the totals
    }
    __syncthreads();
    const int n_above = L.pre_a[nseg];
    const int n_tie = L.pre_t[nseg];
    ksel = min(si.k, n_above + n_tie);
    const int r = ksel - n_above;
    const int2* seg_a = a.ws.seg_above + (size_t)bh * d.cap;
    const float* seg_aw = a.ws.seg_aw + (size_t)bh * d.cap * G;
    const uint4* seg_t = a.ws.seg_tie + (size_t)bh * d.cap;
    const float* seg_w = a.ws.seg_w + (size_t)bh * d.cap * G;
    // above-bucket entries: all of a thread's loads first, then the updates
    for (int i0 = tid; i0 < n_above; i0 += 4 * nthr) {
      int2 pc[4];
      float w[4][G];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * nthr;
        pc[u] = make_int2(-1, 0);
        if (i < n_above) {
          const int sgi = seg_of(L.pre_a, nseg, i);
          const int slot = sgi * kCollectEntries + (i - L.pre_a[sgi]);
          pc[u] = seg_a[slot];
#pragma unroll
          for (int g = 0; g < G; ++g) w[u][g] = seg_aw[(size_t)slot * G + g];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (pc[u].x >= 0) {
          atomicOr(&pbit[pc[u].x >> 5], 1u << (pc[u].x & 31));
          add_fixed<G>(wacc, pc[u].y, w[u]);
        }
      }
    }
    if (r > 0) {
      // candidates of the threshold bucket (with their storage slot in .w),
      // cached in registers when they fit
      constexpr int kReg = 4;
      uint4 cr[kReg];
#pragma unroll
      for (int qi = 0; qi < kReg; ++qi) {
        const int i = tid + qi * nthr;
        cr[qi] = make_uint4(0, 0, 0, 0);
        if (i < n_tie) {
          const int sgi = seg_of(L.pre_t, nseg, i);
          const int slot = sgi * kCollectEntries + (i - L.pre_t[sgi]);
          cr[qi] = seg_t[slot];
          cr[qi].z = (uint32_t)slot;
        }
      }
      const bool cached = n_tie <= kReg * nthr;
      auto load_tie = [&](int i) -> uint4 {
        const int sgi = seg_of(L.pre_t, nseg, i);
        const int slot = sgi * kCollectEntries + (i - L.pre_t[sgi]);
        uint4 v = seg_t[slot];
        v.z = (uint32_t)slot;
        return v;
      };
// BODY runs with `cv` bound to each candidate of the threshold bucket: from
// registers when they were cached there, else from the segments.
#define PQHSA_FOR_EACH_TIE(BODY)                                   \
  if (cached) {                                                    \
    _Pragma("unroll") for (int qi = 0; qi < kReg; ++qi) {          \
      if (tid + qi * nthr < n_tie) {                               \
        const uint4 cv = cr[qi];                                   \
        BODY                                                       \
      }                                                            \
    }                                                              \
  } else {                                                         \
    for (int i = tid; i < n_tie; i += nthr) {                      \
      const uint4 cv = load_tie(i);                                \
      BODY                                                         \
    }                                                              \
  }
      unsigned long long prefix = 0, mask = 0;
      const bool all = r >= n_tie;
      if (!all) {
        int need = r;
        for (int shift = 44; ; shift -= 8) {
          const int s = shift > 0 ? shift : 0;
          const unsigned long long dm = shift >= 0 ? 0xffull : 0xfull;
          for (int i = tid; i < 256; i += nthr) L.rh[i] = 0;
          __syncthreads();
          PQHSA_FOR_EACH_TIE({
            const unsigned long long c = composite52(cv);
            if ((c & mask) == prefix) atomicAdd(&L.rh[(c >> s) & dm], 1u);
          })
          __syncthreads();
          if (tid < 64) {
            // digit whose suffix count crosses `need` (bins scanned from the top)
            int v4[4], sl = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int bin = 255 - (tid * 4 + i);
              v4[i] = bin <= (int)dm ? (int)L.rh[bin] : 0;
              sl += v4[i];
            }
            int x = sl;
            for (int o = 1; o < 64; o <<= 1) {
              const int y = __shfl_up(x, o);
              if (tid >= o) x += y;
            }
            int run = x - sl;
            if (run < need && run + sl >= need) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                if (run < need && run + v4[i] >= need) {
                  L.res[0] = 255 - (tid * 4 + i);
                  L.res[1] = run;
                  L.res[2] = v4[i];
                }
                run += v4[i];
              }
            }
          }
          __syncthreads();
          const int dig = L.res[0];
          need -= L.res[1];
          prefix |= (unsigned long long)dig << s;
          mask |= dm << s;
          const bool done = L.res[2] == need || s == 0;
          __syncthreads();
          if (done) break;
        }
      }
      // winners: positions into the bitmap; (cluster, slot) listed for the
      // weight updates, which then run one per lane
      if (r <= kWinCap) {
        PQHSA_FOR_EACH_TIE({
          if (all || (composite52(cv) & mask) >= prefix) {
            atomicOr(&pbit[cv.y >> 5], 1u << (cv.y & 31));
            win[atomicAdd(&L.n_win, 1)] = make_uint2(cv.w, cv.z);
          }
        })
        __syncthreads();
        for (int i = tid; i < L.n_win; i += nthr) {
          const uint2 cs = win[i];
          float w[G];
#pragma unroll
          for (int g = 0; g < G; ++g) w[g] = seg_w[(size_t)cs.y * G + g];
          add_fixed<G>(wacc, (int)cs.x, w);
        }
      } else {
        for (int i = tid; i < n_tie; i += nthr) {
          const uint4 cv = load_tie(i);
          if (all || (composite52(cv) & mask) >= prefix) {
            atomicOr(&pbit[cv.y >> 5], 1u << (cv.y & 31));
            float w[G];
#pragma unroll
            for (int g = 0; g < G; ++g) w[g] = seg_w[(size_t)cv.z * G + g];
            add_fixed<G>(wacc, (int)cv.w, w);
          }
        }
      }
    }
  }
  __syncthreads();
  // compaction of the position bitmap into ascending rows
  int32_t* rows = a.ws.rows + (size_t)bh * d.cap;
  for (int i = tid; i < si.ns; i += nthr) rows[i] = i;
  const int per = (nw + nthr - 1) / nthr;
  const int w0 = min(nw, tid * per), w1 = min(nw, w0 + per);
  int cnt = 0;
  if (ksel > 0)
    for (int w = w0; w < w1; ++w) cnt += __popc(pbit[w]);
  const int lane = tid & 63, wave = tid >> 6, nwv = nthr >> 6;
  int x = cnt;
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) L.sh[wave] = x;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < nwv; ++w) { int v = L.sh[w]; L.sh[w] = run; run += v; }
    L.sh[nwv] = run;
  }
  __syncthreads();
  int at = si.ns + L.sh[wave] + x - cnt;
  const int nsel = L.sh[nwv];
  int32_t* selout = a.selected ? a.selected + (size_t)bh * a.max_sel : nullptr;
  if (ksel > 0) {
    for (int w = w0; w < w1; ++w) {
      uint32_t bits = pbit[w];
      while (bits) {
        const int bit = __ffs(bits) - 1;
        bits &= bits - 1;
        const int p = w * 32 + bit;
        if (selout && at - si.ns < a.max_sel) selout[at - si.ns] = p;
        rows[at++] = p;
      }
    }
  }
  const int rb = si.recent_beg;
  const int base_r = si.ns + nsel;
  for (int i = tid; i < si.T - rb; i += nthr) rows[base_r + i] = rb + i;
  if (selout)
    for (int i = nsel + tid; i < a.max_sel; i += nthr) selout[i] = -1;
  if (tid == 0) a.ws.n_rows[bh] = base_r + (si.T - rb);
  // every collect block has read the histogram: leave it cleared (the fused
  // step expects a zero histogram)
  for (int i = tid; i < kHistBins; i += nthr) a.ws.hist[(size_t)bh * kHistStride + i] = 0u;
  if (wsel_lds) {
    unsigned long long* out = a.ws.wsel + (size_t)bh * nwsel;
    for (int i = tid; i < nwsel; i += nthr) out[i] = wacc[i];
  }
}

#undef PQHSA_FOR_EACH_TIE

// grid (B*Hkv), kSelectThreads threads: the selection of one (b, h), after
// the collect kernel has filled the segments.
template <int G>
__global__ __launch_bounds__(kSelectThreads) void k_select(StepArgs a) {
  extern __shared__ __align__(16) unsigned char dyn[];
  __shared__ SelectLds L;
  const int bh = blockIdx.x;
  const SeqInfo si = seq_info(a.d, a.ctx, a.ix.n_indexed, bh / a.d.Hkv);
  select_head<G>(a, bh, si, dyn, L);
}

// ---------------------------------------------------------------- collect
// grid (B*Hkv*collect_slices), 256 threads, 4096 entries per block (16 per
// thread, all loaded before the threshold search).  Keys in buckets above the
// threshold bucket are selected: their positions, clusters and weights go to
// this block's segment.  Keys in the threshold bucket go
// to the block's tie segment together with their weights, for the exact pass.
// The few such entries are first compacted into an LDS list (block scan of
// per-thread counts) so that their dependent loads run once, one entry per
// lane.
template <int G>
__global__ __launch_bounds__(kCollectThreads) void k_collect(StepArgs a) {
  extern __shared__ __align__(16) unsigned char dyn[];
  __shared__ SelectLds L;
  __shared__ int scan_a[kCollectThreads / 64 + 1], scan_t[kCollectThreads / 64 + 1];
  const Dims& d = a.d;
  int bh, slice;
  xcd_map(blockIdx.x, d.B * d.Hkv, d.collect_slices, &bh, &slice);
  const int b = bh / d.Hkv;
  const int tid = threadIdx.x;
  const SeqInfo si = seq_info(d, a.ctx, a.ix.n_indexed, b);
  const int n_entries = min(a.ix.list_off[(size_t)bh * (d.L + 1) + d.L], d.cap);
  const int e0 = slice * kCollectEntries;
  if (si.k <= 0 || e0 >= n_entries) {
    // an idle slice: empty segments, so the selection can read every slice
    if (tid == 0) {
      int32_t* cnt = a.ws.seg_cnt + ((size_t)bh * d.collect_slices + slice) * 2;
      cnt[0] = 0;
      cnt[1] = 0;
    }
    return;
  }
  {
    int* list_a = reinterpret_cast<int*>(dyn);
    uint2* list_t = reinterpret_cast<uint2*>(dyn + kCollectEntries * sizeof(int));
    const int e1 = min(n_entries, e0 + kCollectEntries);
    const uint32_t* keys = a.ws.keys + (size_t)bh * d.cap;
    uint32_t kv[kCollectPerThread];
#pragma unroll
    for (int j = 0; j < kCollectPerThread; ++j) {
      const int e = e0 + j * kCollectThreads + tid;
      kv[j] = e < e1 ? keys[e] : 0u;
    }
    int beta, above, total;
    find_threshold(a.ws.hist + (size_t)bh * kHistStride, si.k, L.sh, &beta, &above, &total);
    // per-thread counts, block exclusive scan, then in-order placement
    int ca = 0, ct = 0;
#pragma unroll
    for (int j = 0; j < kCollectPerThread; ++j) {
      const int bucket = (int)(kv[j] >> (32 - kHistBits));
      const bool valid = kv[j] != 0u && beta >= 0;
      ca += (valid && bucket > beta);
      ct += (valid && bucket == beta);
    }
    const int lane = tid & 63, wave = tid >> 6, nwv = kCollectThreads / 64;
    int xa = ca, xt = ct;
    for (int o = 1; o < 64; o <<= 1) {
      const int ya = __shfl_up(xa, o), yt = __shfl_up(xt, o);
      if (lane >= o) { xa += ya; xt += yt; }
    }
    if (lane == 63) { scan_a[wave] = xa; scan_t[wave] = xt; }
    __syncthreads();
    if (tid == 0) {
      int ra = 0, rt = 0;
      for (int w = 0; w < nwv; ++w) {
        const int va = scan_a[w], vt = scan_t[w];
        scan_a[w] = ra; scan_t[w] = rt;
        ra += va; rt += vt;
      }
      scan_a[nwv] = ra;
      scan_t[nwv] = rt;
    }
    __syncthreads();
    int at_a = scan_a[wave] + xa - ca, at_t = scan_t[wave] + xt - ct;
#pragma unroll
    for (int j = 0; j < kCollectPerThread; ++j) {
      const int bucket = (int)(kv[j] >> (32 - kHistBits));
      const bool valid = kv[j] != 0u && beta >= 0;
      const int e = e0 + j * kCollectThreads + tid;
      if (valid && bucket > beta) list_a[at_a++] = e;
      if (valid && bucket == beta) list_t[at_t++] = make_uint2(kv[j], (uint32_t)e);
    }
    __syncthreads();
    const int na = scan_a[nwv], nt = scan_t[nwv];
    const int32_t* pos = a.ix.pos + (size_t)bh * d.cap;
    int2* seg_a = a.ws.seg_above + (size_t)bh * d.cap + e0;
    float* seg_aw = a.ws.seg_aw + ((size_t)bh * d.cap + e0) * G;
    uint4* seg_t = a.ws.seg_tie + (size_t)bh * d.cap + e0;
    float* seg_w = a.ws.seg_w + ((size_t)bh * d.cap + e0) * G;
    for (int i = tid; i < na; i += kCollectThreads) {
      const int e = list_a[i];
      const int c = entry_cluster(a, bh, e);
      float w[G];
      seg_a[i] = make_int2(pos[e], c);
      entry_weights<G>(a, bh, e, c, w);
#pragma unroll
      for (int g = 0; g < G; ++g) seg_aw[(size_t)i * G + g] = w[g];
    }
    for (int i = tid; i < nt; i += kCollectThreads) {
      const uint2 ke = list_t[i];
      const int e = (int)ke.y;
      const int c = entry_cluster(a, bh, e);
      float w[G];
      seg_t[i] = make_uint4(ke.x, (uint32_t)pos[e], (uint32_t)e, (uint32_t)c);
      entry_weights<G>(a, bh, e, c, w);
#pragma unroll
      for (int g = 0; g < G; ++g) seg_w[(size_t)i * G + g] = w[g];
    }
    if (tid == 0) {
      int32_t* cnt = a.ws.seg_cnt + ((size_t)bh * d.collect_slices + slice) * 2;
      cnt[0] = na;
      cnt[1] = nt;
    }
  }
}

// ---------------------------------------------------------------- launchers
#define PQHSA_G_DISPATCH(fn, ...)                   \
  switch (a.d.G) {                                  \
    case 1: return fn<1>(__VA_ARGS__);              \
    case 2: return fn<2>(__VA_ARGS__);              \
    case 4: return fn<4>(__VA_ARGS__);              \
    case 8: return fn<8>(__VA_ARGS__);              \
  }                                                 \
  return hipErrorInvalidValue;

template <int G>
static hipError_t tables_g(const StepArgs& a, const Launch& l) {
  const int BH = a.d.B * a.d.Hkv;
  return launch_kernel(k_tables<G>, dim3(BH, kM + (a.d.L + 15) / 16), dim3(256), 0, l, a);
}
hipError_t launch_tables(const StepArgs& a, const Launch& l) { PQHSA_G_DISPATCH(tables_g, a, l) }

template <int G>
static hipError_t scan_g(const StepArgs& a, const Launch& l) {
  const int BH = a.d.B * a.d.Hkv;
  const size_t lds = (size_t)kM * kKsub * G * sizeof(float) + kHistBins * sizeof(uint32_t);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_scan<G>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  return launch_kernel(k_scan<G>, dim3(BH * a.d.scan_blocks), dim3(kScanThreads), lds, l, a);
}
hipError_t launch_scan(const StepArgs& a, const Launch& l) { PQHSA_G_DISPATCH(scan_g, a, l) }

template <int G>
static hipError_t collect_g(const StepArgs& a, const Launch& l) {
  const int BH = a.d.B * a.d.Hkv;
  const size_t lds = (size_t)kCollectEntries * (sizeof(int) + sizeof(uint2));
  return launch_kernel(k_collect<G>, dim3(BH * a.d.collect_slices), dim3(kCollectThreads), lds,
                       l, a);
}
hipError_t launch_collect(const StepArgs& a, const Launch& l) {
  PQHSA_G_DISPATCH(collect_g, a, l)
}

template <int G>
static hipError_t select_g(const StepArgs& a, const Launch& l) {
  const int BH = a.d.B * a.d.Hkv;
  const size_t wsel = (size_t)a.d.L * G * sizeof(unsigned long long);
  const size_t lds = ((size_t)a.d.nwords * 4 + 15) / 16 * 16 + kWinCap * sizeof(uint2) +
                     (wsel <= kWselLdsBytes ? wsel : 0);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_select<G>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  return launch_kernel(k_select<G>, dim3(BH), dim3(kSelectThreads), lds, l, a);
}
hipError_t launch_select(const StepArgs& a, const Launch& l) { PQHSA_G_DISPATCH(select_g, a, l) }

}  // namespace pqhsa
