// The whole PQ-HSA decode step as one kernel.
//
// PQ-HSA page (rit.work blog), section "How approximate estimates return the
// discarded context": per KV head, every indexed token gets an approximate
// logit from the IVF-PQ index (third paragraph); the best of them within the
// budget are read from the paged cache and computed exactly, the others keep
// their approximate weight in the shared normalisation (fourth paragraph) and
// contribute through their cluster's mean value (fifth paragraph); the first
// tokens, the recent window and the not yet indexed tokens stay exact (sixth
// paragraph).  Partials are merged by the prefix/suffix law
// O = (N_P + N_S) / (D_P + D_S) of the quant_prune_distill post on query reuse.
//
// The staged kernels (tables, scan, collect, select, attend, merge) spend most
// of a 128K step at kernel boundaries: each boundary costs a launch gap and a
// cold start.  Here P blocks own the clusters of one (b, h) and meet at two
// per-head barriers:
//
//   phase 1  LUT of the G query heads into LDS; one wave per cluster computes
//            the approximate logits of its entries, their keys, the
//            cluster's (max, sum of exp2) bins and a 4096-bin histogram of
//            the keys' top 12 bits, added to the head's global histogram.
//   barrier  (histogram complete)
//   phase 2  threshold bucket from the histogram; the block's entries above
//            it are selected, those inside it are published as ties; the
//            selected entries' weights are added to per-cluster sums.
//   barrier  (counts and records complete)
//   phase 3  every block resolves the tie bucket with the same radix select
//            (52-bit composite: low key bits, then inverted position, so equal
//            keys prefer the lower position), takes an even share of the exact
//            rows (sink, selected, recent/tail) plus its own clusters'
//            background terms, and writes one partial (m, l, acc[128]) per
//            query head.  The last block of the head to finish merges the P
//            partials into O and the log-sum-exp, writes the ascending selected
//            positions if asked, and clears the head's counters and histogram
//            for the next step.
//
// Cross-block data moves only through device-scope stores, loads and atomics
// (coherent across XCDs without cache write-back or invalidation); a thread
// waits for its own stores before its block arrives at a barrier.
//
// Residency: the grid is at most as large as the device holds at once (blocks
// per CU by occupancy times CUs), so on a device that runs nothing else every
// block is resident at once and the barriers cannot deadlock; a block that
// arrives early only waits for blocks that are already running.  (A cooperative
// launch would guarantee the same but costs tens of µs per launch.)  If CUs
// are withheld, waits are bounded in time: a wait that runs out sets bit 0 of
// the workspace flags and the step goes on, so a call always finishes.
#include "pqhsa_internal.hpp"

namespace pqhsa {

namespace {

constexpr unsigned long long kBarrierTimeout = 200000000ull;   // 2 s of the 100 MHz clock

template <int G>
struct FusedCfg {
  static constexpr int NT = 512;   // 8 waves: up to 256 VGPRs each
  static constexpr int NW = NT / 64;
  static constexpr int NG = NT / 16;                // 16-lane row groups
  static constexpr int kItemsPerGroup = 4;
  static constexpr int kItems = NG * kItemsPerGroup;   // attention items staged per phase
  static constexpr size_t kUBytes = (size_t)kM * kKsub * G * sizeof(float);   // LUT, then reuse
  static constexpr size_t kHBytes = (size_t)kHistBins * sizeof(uint32_t);
  // clusters x G per block whose per-cluster values live in LDS (smaller at
  // G = 8, whose 128 KB LUT leaves less room)
  static constexpr int kCG = G == 8 ? kFusedWselMax / 2 : kFusedWselMax;
  static constexpr size_t kWBytes = (size_t)kCG * sizeof(unsigned long long);   // selected weights
  static constexpr size_t kQBytes = (size_t)kCG * sizeof(float);                // cluster logits
  static constexpr size_t kBBytes = (size_t)kCG * 2 * sizeof(float);            // cluster (max, sum)
  static constexpr size_t kDyn = kUBytes + kHBytes + kWBytes + kQBytes + kBBytes;
  static constexpr int kTieCap = (int)(kUBytes / sizeof(unsigned long long));
  static_assert((size_t)NW * G * (2 + kD) * sizeof(float) <= kUBytes, "merge arrays");
  static_assert((size_t)kItems * sizeof(long long) + 4096 <= kHBytes, "item staging");
};

struct FusedStatic {
  int nextc;        // the scan's next unclaimed cluster of the block
  int sh[40];
  uint32_t rh[256];
  int res[4];
  int apre[kMaxFusedP + 1];
  int tpre[kMaxFusedP + 1];
  int tbase[kMaxFusedP + 1];
  int last;
};

// ---------------------------------------------------------------- device-scope memory
__device__ __forceinline__ void st_dev(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_dev(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_dev(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
}

// Wait until every memory operation this thread issued has completed
// (s_waitcnt vmcnt(0)); no cache write-back or invalidation.
__device__ __forceinline__ void wait_mem() { __builtin_amdgcn_s_waitcnt(0xF70); }

// A barrier of the P blocks of a head, in two halves so that a block can
// issue loads of its own data while it waits.  Arrive: every thread's memory
// operations have completed, then one thread adds to the head's counter (true
// in thread 0 when this block arrived last).  Wait: thread 0 polls until all
// have arrived or the time bound has passed (then bit 0 of *flags is set).
__device__ bool barrier_arrive(uint32_t* ctr, uint32_t n) {
  wait_mem();
  __syncthreads();
  bool last = false;
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 >= n;
  return last;
}

__device__ void barrier_wait(uint32_t* ctr, uint32_t n, uint32_t* flags, bool last) {
  if (threadIdx.x == 0 && !last) {
    const unsigned long long t0 = wall_clock64();
    while (ld_dev(ctr) < n) {
      __builtin_amdgcn_s_sleep(8);
      if (wall_clock64() - t0 > kBarrierTimeout) {
        __hip_atomic_fetch_or(flags, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
}

// Exclusive block scan of two per-thread counts; the block totals go to *ta, *tb.
template <int NT>
__device__ void block_scan2(int a, int b, int* oa, int* ob, int* ta, int* tb, int* sh) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int xa = wave_incl_scan(a), xb = wave_incl_scan(b);
  if (lane == 63) { sh[wave] = xa; sh[NW + 1 + wave] = xb; }
  __syncthreads();
  if (threadIdx.x == 0) {
    int ra = 0, rb = 0;
    for (int w = 0; w < NW; ++w) {
      const int va = sh[w], vb = sh[NW + 1 + w];
      sh[w] = ra; sh[NW + 1 + w] = rb;
      ra += va; rb += vb;
    }
    sh[NW] = ra;
    sh[2 * NW + 1] = rb;
  }
  __syncthreads();
  *oa = sh[wave] + xa - a;
  *ob = sh[NW + 1 + wave] + xb - b;
  *ta = sh[NW];
  *tb = sh[2 * NW + 1];
  __syncthreads();
}

// The whole block, over bins [lo, 4096) of a histogram in LDS (bin = top 12
// bits of the key): the bucket beta holding the k-th largest key counted from
// the top, i.e. above(beta) < k <= above(beta) + hist[beta] with above(x) the
// count in bins (x, 4096); k is first capped at the range's total.  Thread t
// sums the 4096/NT bins below 4096 - t*4096/NT (thread 0 the highest); a
// block scan of the sums in that order finds the one thread whose range
// crosses k, which walks its bins.
// Writes beta (-1 if the capped k is 0), above(beta) and the total to
// out[0..2]; sh holds NT/64 ints.  Ends with a block barrier.
template <int NT>
__device__ void block_threshold(const uint32_t* hist, int lo, int k, int* out, int* sh) {
  constexpr int PER = kHistBins / NT;
  static_assert(PER * NT == kHistBins && PER % 4 == 0, "bins per thread");
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = kHistBins - PER * tid;   // this thread's bins are [hi - PER, hi)
  uint32_t v[PER];
#pragma unroll
  for (int i = 0; i < PER; i += 4) {
    const uint4 w = *reinterpret_cast<const uint4*>(hist + hi - PER + i);
    v[i] = w.x; v[i + 1] = w.y; v[i + 2] = w.z; v[i + 3] = w.w;
  }
  int s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) s += (hi - PER + i >= lo) ? (int)v[i] : 0;
  const int inc = wave_incl_scan(s);
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = sh[w];
    before += w < wave ? t : 0;
    tot += t;
  }
  const int kk = min(k, tot);
  const int x1 = before + inc, x0 = x1 - s;   // counts above and through this range
  if (kk > 0 && x0 < kk && kk <= x1) {
    int run = x0, beta = hi - PER;
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {
      const int c = (hi - PER + i >= lo) ? (int)v[i] : 0;
      if (run + c >= kk) { beta = hi - PER + i; break; }
      run += c;
    }
    out[0] = beta; out[1] = run; out[2] = tot;
  }
  if (kk == 0 && tid == 0) { out[0] = -1; out[1] = 0; out[2] = tot; }
  __syncthreads();
}

__device__ __forceinline__ unsigned long long tie_composite(unsigned long long rec) {
  // rec = key << 32 | position
  return composite52(make_uint4((uint32_t)(rec >> 32), (uint32_t)rec, 0u, 0u));
}

__device__ __forceinline__ unsigned long long to_fixed(float w) {
  return (unsigned long long)(w * kFixScale + 0.5f);
}

// One background item: the cluster's summed unselected weight as a logit
// s_g (base 2) and its mean value as the row's value (8 dims per lane).
template <int G>
__device__ __forceinline__ void attend_bg(AttnState<G>& st, const float* sg, uint4 m0, uint4 m1) {
  const float mu[8] = {__uint_as_float(m0.x), __uint_as_float(m0.y), __uint_as_float(m0.z),
                       __uint_as_float(m0.w), __uint_as_float(m1.x), __uint_as_float(m1.y),
                       __uint_as_float(m1.z), __uint_as_float(m1.w)};
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float s = sg[g];
    if (s == -INFINITY) continue;
    const float mn = fmaxf(st.m[g], s);
    const float al = __builtin_amdgcn_exp2f(st.m[g] - mn);
    const float p = __builtin_amdgcn_exp2f(s - mn);
    st.l[g] = fmaf(st.l[g], al, p);
#pragma unroll
    for (int i = 0; i < 8; ++i) st.acc[g][i] = fmaf(st.acc[g][i], al, p * mu[i]);
    st.m[g] = mn;
  }
}

// One exact row for the G query heads, with q kept as packed bf16 (the
// scale is applied to the row sum).
template <int G>
__device__ __forceinline__ void attend_row_pk(AttnState<G>& st, const uint4 (&qp)[G], float scl,
                                              uint4 kw, uint4 vw) {
  const float kf[8] = {bf16_lo(kw.x), bf16_hi(kw.x), bf16_lo(kw.y), bf16_hi(kw.y),
                       bf16_lo(kw.z), bf16_hi(kw.z), bf16_lo(kw.w), bf16_hi(kw.w)};
  const float vf[8] = {bf16_lo(vw.x), bf16_hi(vw.x), bf16_lo(vw.y), bf16_hi(vw.y),
                       bf16_lo(vw.z), bf16_hi(vw.z), bf16_lo(vw.w), bf16_hi(vw.w)};
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint4 q = qp[g];
    float s = bf16_lo(q.x) * kf[0];
    s = fmaf(bf16_hi(q.x), kf[1], s);
    s = fmaf(bf16_lo(q.y), kf[2], s);
    s = fmaf(bf16_hi(q.y), kf[3], s);
    s = fmaf(bf16_lo(q.z), kf[4], s);
    s = fmaf(bf16_hi(q.z), kf[5], s);
    s = fmaf(bf16_lo(q.w), kf[6], s);
    s = fmaf(bf16_hi(q.w), kf[7], s);
    s = row16_sum(s) * scl;
    const float mn = fmaxf(st.m[g], s);
    const float al = __builtin_amdgcn_exp2f(st.m[g] - mn);
    const float p = __builtin_amdgcn_exp2f(s - mn);
    st.l[g] = fmaf(st.l[g], al, p);
#pragma unroll
    for (int i = 0; i < 8; ++i) st.acc[g][i] = fmaf(st.acc[g][i], al, p * vf[i]);
    st.m[g] = mn;
  }
}

template <int G, int PT>
struct FRound {
  uint4 cw[PT];
  int pp[PT];
};

}  // namespace

template <int G>
__global__ __launch_bounds__(FusedCfg<G>::NT) void k_fused(StepArgs a) {
  using C = FusedCfg<G>;
  constexpr int NT = C::NT, NW = C::NW, NG = C::NG;
  constexpr int PT = 5;   // 64-entry tiles per scan round (most clusters in one)
  constexpr int kIB = G == 8 ? 2 : 4;  // attention items whose loads are in flight together
  extern __shared__ __align__(16) unsigned char dyn[];
  __shared__ FusedStatic S;
  float* lut = reinterpret_cast<float*>(dyn);
  uint32_t* hist = reinterpret_cast<uint32_t*>(dyn + C::kUBytes);
  unsigned long long* wsel = reinterpret_cast<unsigned long long*>(dyn + C::kUBytes + C::kHBytes);
  float* qcl = reinterpret_cast<float*>(dyn + C::kUBytes + C::kHBytes + C::kWBytes);   // [ncl][G]
  // (max, sum of exp2) of every cluster of the block and query head: [ncl][G][2]
  float* binl = reinterpret_cast<float*>(dyn + C::kUBytes + C::kHBytes + C::kWBytes + C::kQBytes);

  const Dims& d = a.d;
  const int P = d.fP;
  const int BH = d.B * d.Hkv;
  int bh, sub;
  xcd_map(blockIdx.x, BH, P, &bh, &sub);
  const int b = bh / d.Hkv, h = bh % d.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c0 = min(d.L, sub * d.fcpb), c1 = min(d.L, c0 + d.fcpb), ncl = c1 - c0;
  const int32_t* off = a.ix.list_off + (size_t)bh * (d.L + 1);
  auto entry_at = [&](int c) { return min(max(off[c], 0), d.cap); };
  const int E0 = entry_at(c0), E1 = max(E0, entry_at(c1));
  const SeqInfo si = seq_info(d, a.ctx, a.ix.n_indexed, b);
  // the head's three counters (barrier 1, barrier 2, finished blocks), each on
  // its own cache line: heads and counters do not contend for one line
  uint32_t* sync = a.ws.fsync + (size_t)bh * 3 * kSyncStride;
  uint32_t* ghist = a.ws.hist + (size_t)bh * kHistBins;
  // the top 16 bits of each entry's selection key (0: not a candidate),
  // enough for the 12-bit buckets; a tie's full key is recomputed from its
  // codes when it is recorded
  uint16_t* keys = reinterpret_cast<uint16_t*>(a.ws.keys) + (size_t)bh * d.cap;
  float* qcg = a.ws.qc + (size_t)bh * d.L * G;
  const uint4* codes = reinterpret_cast<const uint4*>(a.ix.codes + (size_t)bh * d.cap * kM);
  const int32_t* pos = a.ix.pos + (size_t)bh * d.cap;
  const int32_t* ent_list = a.ix.ent_list + (size_t)bh * d.cap;
  const float* cent = a.ix.centroids + (size_t)bh * d.L * kD;
  const uint16_t* qh = a.q + ((size_t)b * d.Hq + h * G) * kD;
  // per-head record arrays, indexed in entry space (block j writes from its
  // first entry on): selected positions, tie records, tie weights and clusters
  int32_t* fpos = reinterpret_cast<int32_t*>(a.ws.seg_above + (size_t)bh * d.cap);
  unsigned long long* ftie = reinterpret_cast<unsigned long long*>(a.ws.seg_tie + (size_t)bh * d.cap);
  float* ftw = a.ws.seg_w + (size_t)bh * d.cap * G;
  int32_t* ftc = reinterpret_cast<int32_t*>(a.ws.seg_aw + (size_t)bh * d.cap * G);
  int32_t* frows = a.ws.rows + (size_t)bh * d.cap;

  // ======================================================= phase 1: LUT and scan
  auto issue = [&](FRound<G, PT>& r, int base, int e1) {
#pragma unroll
    for (int t = 0; t < PT; ++t) {
      const int e = base + t * 64 + lane;
      r.pp[t] = -1;
      if (e < e1) {
        r.cw[t] = codes[e];
        r.pp[t] = pos[e];
      }
    }
  };
  // the wave's first round goes out before the tables are built, after the
  // tables' own loads (which need no index offsets)
  int c = c0 + wave;
  int e0 = 0, e1 = 0;
  FRound<G, PT> rb[2];
  {
    // LUT[m][j][g] = scale*log2e * q_g^(m) . B_m[j].  Every thread's codebook
    // rows are loaded at once (codeword j = tid % 256, subspaces tid / 256 +
    // step * i), while q is staged in LDS as scaled floats; then the dot
    // products run from registers and LDS.
    constexpr int kPairs = kM * kKsub / NT;
    constexpr int kMStep = NT / kKsub;
    static_assert(kPairs * NT == kM * kKsub && kMStep >= 1, "LUT pairs");
    const int j = tid & (kKsub - 1), m0 = tid / kKsub;
    float4 cb[kPairs][2];
#pragma unroll
    for (int i = 0; i < kPairs; ++i) {
      const float* cw = a.ix.codebooks + (((size_t)bh * kM + m0 + kMStep * i) * kKsub + j) * kDsub;
      cb[i][0] = *reinterpret_cast<const float4*>(cw);
      cb[i][1] = *reinterpret_cast<const float4*>(cw + 4);
    }
    // the first cluster of this thread's 16-lane row for the QC pass
    const int l16r = tid & 15;
    float4 cen0 = make_float4(0.f, 0.f, 0.f, 0.f), cen1 = cen0;
    if ((tid >> 4) < ncl) {
      const float* cp = cent + (size_t)(c0 + (tid >> 4)) * kD + l16r * 8;
      cen0 = *reinterpret_cast<const float4*>(cp);
      cen1 = *reinterpret_cast<const float4*>(cp + 4);
    }
    uint4 qw = make_uint4(0, 0, 0, 0);
    if (tid < G * kD / 8) qw = *reinterpret_cast<const uint4*>(qh + tid * 8);
    if (c < c1) {
      e0 = entry_at(c);
      e1 = max(e0, entry_at(c + 1));
      issue(rb[0], e0, e1);
    }
    float* qsl = reinterpret_cast<float*>(hist);   // scaled q [G][128] until the QC pass
    if (tid < G * kD / 8) {
      const uint4 w = qw;
      const float f[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                          bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
#pragma unroll
      for (int i = 0; i < 8; ++i) qsl[tid * 8 + i] = f[i] * d.scale_log2;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPairs; ++i) {
      const int m = m0 + kMStep * i;
      const float cv[8] = {cb[i][0].x, cb[i][0].y, cb[i][0].z, cb[i][0].w,
                           cb[i][1].x, cb[i][1].y, cb[i][1].z, cb[i][1].w};
      float outv[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float* qq = qsl + g * kD + m * kDsub;
        float sacc = qq[0] * cv[0];
#pragma unroll
        for (int t = 1; t < kDsub; ++t) sacc = fmaf(qq[t], cv[t], sacc);
        outv[g] = sacc;
      }
      float* dst = lut + (m * kKsub + j) * G;
      if constexpr (G == 8) {
        reinterpret_cast<float4*>(dst)[0] = make_float4(outv[0], outv[1], outv[2], outv[3]);
        reinterpret_cast<float4*>(dst)[1] = make_float4(outv[4], outv[5], outv[6], outv[7]);
      } else if constexpr (G == 4) {
        *reinterpret_cast<float4*>(dst) = make_float4(outv[0], outv[1], outv[2], outv[3]);
      } else if constexpr (G == 2) {
        *reinterpret_cast<float2*>(dst) = make_float2(outv[0], outv[1]);
      } else {
        dst[0] = outv[0];
      }
    }
    // QC of the block's clusters, one per 16-lane row: qc[c][g] =
    // scale*log2e * q_g . C_c (8 dims per lane, DPP row sum)
    for (int cl = tid >> 4; cl < ncl; cl += NT / 16) {
      float4 v0 = cen0, v1 = cen1;
      if (cl != (tid >> 4)) {
        const float* cp = cent + (size_t)(c0 + cl) * kD + l16r * 8;
        v0 = *reinterpret_cast<const float4*>(cp);
        v1 = *reinterpret_cast<const float4*>(cp + 4);
      }
      const float cv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      float qcv[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float* qq = qsl + g * kD + l16r * 8;
        float sacc = qq[0] * cv[0];
#pragma unroll
        for (int t = 1; t < 8; ++t) sacc = fmaf(qq[t], cv[t], sacc);
        qcv[g] = row16_sum(sacc);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (l16r == g) {
          qcl[cl * G + g] = qcv[g];
          qcg[(size_t)(c0 + cl) * G + g] = qcv[g];
        }
      }
    }
    __syncthreads();   // the staged q is read for the last time above
    for (int i = tid; i < kHistBins; i += NT) hist[i] = 0u;
    for (int i = tid; i < ncl * G; i += NT) wsel[i] = 0ull;
    if (tid == 0) S.nextc = c0 + NW;
  }
  __syncthreads();
  float qc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) qc[g] = c < c1 ? qcl[(c - c0) * G + g] : 0.0f;

  float mx[G], sm[G];
#pragma unroll
  for (int g = 0; g < G; ++g) { mx[g] = -INFINITY; sm[g] = 0.0f; }
  int base = e0;
  // one round of PT tiles; the next round (more of this cluster, or the first
  // of the wave's next one) is issued before this one is computed
  const bool claims = ncl > 4 * NW;
  auto round = [&](FRound<G, PT>& now, FRound<G, PT>& nxt) {
    int nc = c, nbase = base + 64 * PT, ne0 = e0, ne1 = e1;
    const bool last = nbase >= e1;
    if (last) {
      // the wave's next cluster: with many clusters per wave the block's next
      // unclaimed one, so that the waves finish together whatever the cluster
      // sizes; with few, the next in a fixed stride (no claim on the path)
      if (claims) {
        int claim = 0;
        if (lane == 0) claim = atomicAdd(&S.nextc, 1);
        nc = __builtin_amdgcn_readfirstlane(claim);
      } else {
        nc = c + NW;
      }
      if (nc < c1) {
        ne0 = entry_at(nc);
        ne1 = max(ne0, entry_at(nc + 1));
      }
      nbase = ne0;
    }
    if (nc < c1) issue(nxt, nbase, ne1);
    float s[PT][G];
#pragma unroll
    for (int t = 0; t < PT; ++t) {
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
        uint32_t key = 0;
        if (p >= si.cand_beg && p < si.cand_end) {
          key = order_key(kappa);
          atomicAdd(&hist[key >> (32 - kHistBits)], 1u);
#pragma unroll
          for (int g = 0; g < G; ++g) s[t][g] = v[g];
        }
        keys[e] = (uint16_t)(key >> 16);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float rm = s[0][g];
#pragma unroll
      for (int t = 1; t < PT; ++t) rm = fmaxf(rm, s[t][g]);
      const float Mn = fmaxf(mx[g], rm);
      if (Mn != -INFINITY) {
        float acc = sm[g] * __builtin_amdgcn_exp2f(mx[g] - Mn);
#pragma unroll
        for (int t = 0; t < PT; ++t) acc += __builtin_amdgcn_exp2f(s[t][g] - Mn);
        sm[g] = acc;
        mx[g] = Mn;
      }
    }
    if (last) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float M = wave_max_dpp(mx[g]);
        const float part = (mx[g] == -INFINITY) ? 0.0f : sm[g] * __builtin_amdgcn_exp2f(mx[g] - M);
        const float Ssum = wave_sum_dpp(part);
        if (lane == 0) {
          binl[((c - c0) * G + g) * 2] = M;
          binl[((c - c0) * G + g) * 2 + 1] = Ssum;
        }
        mx[g] = -INFINITY;
        sm[g] = 0.0f;
      }
      if (nc < c1) {
#pragma unroll
        for (int g = 0; g < G; ++g) qc[g] = qcl[(nc - c0) * G + g];
      }
    }
    c = nc;
    base = nbase;
    e0 = ne0;
    e1 = ne1;
  };
  while (c < c1) {
    round(rb[0], rb[1]);
    if (!(c < c1)) break;
    round(rb[1], rb[0]);
  }
  __syncthreads();
  // The block's own threshold bucket beta_b: at least k of its keys lie in
  // bins >= beta_b, so the head's threshold bucket is >= beta_b and the bins
  // below cannot matter.  Only bins >= beta_b go to the head's histogram
  // (fewer atomics on shared lines), and only those are read back.
  block_threshold<NT>(hist, 0, si.k, S.res, S.sh);
  const int beta_b = S.res[0];   // -1: no candidate in this block, or k = 0
  // with fewer than k candidates of its own the block flushes every bin, and
  // the head's threshold may lie below its bins: it then reads them all
  const int read_lo = S.res[2] >= si.k ? beta_b : 0;
  __syncthreads();
  if (beta_b >= 0) {
    for (int i = beta_b + tid; i < kHistBins; i += NT) {
      const uint32_t v = hist[i];
      if (v) __hip_atomic_fetch_add(&ghist[i], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  const bool last1 = barrier_arrive(&sync[0], (uint32_t)P);
  // while waiting: this block's first keys for the classification below
  constexpr int kPer = 16;
  uint32_t pk[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int e = E0 + u * NT + tid;
    pk[u] = e < E1 ? keys[e] : 0u;
  }
  barrier_wait(&sync[0], (uint32_t)P, a.ws.fflags, last1);

  // ======================================================= phase 2: threshold bucket
  // the head's histogram from read_lo up: exact there, because every block
  // with at least k candidates added all its bins >= its own beta_b <= beta,
  // and every other block added all of its bins
  int beta = -1;
  if (beta_b >= 0) {
    for (int i = read_lo + tid; i < kHistBins; i += NT) hist[i] = ld_dev(&ghist[i]);
    __syncthreads();
    block_threshold<NT>(hist, read_lo, si.k, S.res, S.sh);
    beta = S.res[0];
    __syncthreads();
  }
  const bool any = beta >= 0;
  auto entry_w = [&](int e, int cl, float* w, uint32_t* key) {
    const uint4 cw = codes[e];
    float q[G], sv[G];
#pragma unroll
    for (int g = 0; g < G; ++g) q[g] = qcl[(cl - c0) * G + g];
    entry_logits_lds<G>(lut, q, cw, sv);
    // the scan's key, bit for bit (same logits, same max order)
    float kappa = sv[0];
#pragma unroll
    for (int g = 1; g < G; ++g) kappa = fmaxf(kappa, sv[g]);
    *key = order_key(kappa);
#pragma unroll
    for (int g = 0; g < G; ++g)
      w[g] = __builtin_amdgcn_exp2f(sv[g] - binl[((cl - c0) * G + g) * 2]);
  };
  // The block's entries in chunks of NT*16 (entry cb + u*NT + tid to thread
  // tid): count, one block scan, list the chosen entries in LDS (above ones
  // from the front, ties from the back, each group in thread order).  The
  // list is recorded, one entry per thread, once it would overflow and after
  // the last chunk, so that the records' gathers of a many-chunk block wait
  // on memory once.  A chunk larger than the whole list records its entries
  // by their own threads.
  constexpr int kChunk = NT * kPer;
  constexpr int kListCap = (int)(C::kHBytes / sizeof(int));
  int* elist = reinterpret_cast<int*>(hist);
  int na = 0, nt = 0;   // records made or listed, above / tie
  int la = 0, lt = 0;   // of which listed and not yet recorded
  auto record = [&](int e, bool isA, int idx) {
    const int cl = min(max(ent_list[e], c0), c1 - 1);
    const int p = pos[e];
    float w[G];
    uint32_t key;
    entry_w(e, cl, w, &key);
    if (isA) {
      st_dev(&fpos[E0 + idx], p);
#pragma unroll
      for (int g = 0; g < G; ++g) atomicAdd(&wsel[(cl - c0) * G + g], to_fixed(w[g]));
    } else {
      const int slot = E0 + idx;
      st_dev(&ftie[slot], ((unsigned long long)key << 32) | (uint32_t)p);
#pragma unroll
      for (int g = 0; g < G; ++g) ftw[(size_t)slot * G + g] = w[g];
      ftc[slot] = cl;
    }
  };
  auto record_list = [&]() {
    __syncthreads();
    for (int li = tid; li < la + lt; li += NT) {
      const bool isA = li < la;
      if (isA) record(elist[li], true, na - la + li);
      else record(elist[kListCap - 1 - (li - la)], false, nt - lt + (li - la));
    }
    la = lt = 0;
    __syncthreads();
  };
  if (any && E1 - E0 <= kChunk) {
    // one chunk (the keys already in pk): list, then record
    int ca = 0, ct = 0;
    uint32_t chosenA = 0, chosenT = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint32_t kv = pk[u];
      const int bucket = (int)(kv >> (16 - kHistBits));
      if (kv != 0u && bucket > beta) { ++ca; chosenA |= 1u << u; }
      if (kv != 0u && bucket == beta) { ++ct; chosenT |= 1u << u; }
    }
    int oa, ot, ta, tt;
    block_scan2<NT>(ca, ct, &oa, &ot, &ta, &tt, S.sh);
    uint32_t chosen = chosenA | chosenT;
    while (chosen) {
      const int u = __ffs(chosen) - 1;
      chosen &= chosen - 1;
      const int e = E0 + u * NT + tid;
      const bool isA = (chosenA >> u) & 1u;
      const int li = isA ? oa++ : ta + ot++;
      if (li < kListCap) elist[li] = e;
      else record(e, isA, isA ? li : li - ta);
    }
    __syncthreads();
    for (int li = tid; li < min(ta + tt, kListCap); li += NT) {
      const bool isA = li < ta;
      record(elist[li], isA, isA ? li : li - ta);
    }
    na = ta;
    nt = tt;
  } else if (any) {
    for (int cb = E0; cb < E1; cb += kChunk) {
      // bit u: entry u of this thread is above (A) or in (T) the bucket
      uint32_t chosenA = 0, chosenT = 0;
      int ca = 0, ct = 0;
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const uint32_t kv = pk[u];
        const int bucket = (int)(kv >> (16 - kHistBits));
        if (kv != 0u && bucket > beta) { ++ca; chosenA |= 1u << u; }
        if (kv != 0u && bucket == beta) { ++ct; chosenT |= 1u << u; }
      }
      // the next chunk's keys load while this chunk is listed
      if (cb + kChunk < E1) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          const int e = cb + kChunk + u * NT + tid;
          pk[u] = e < E1 ? keys[e] : 0u;
        }
      }
      int oa, ot, ta, tt;
      block_scan2<NT>(ca, ct, &oa, &ot, &ta, &tt, S.sh);
      const bool fits = ta + tt <= kListCap;
      if (fits && la + lt + ta + tt > kListCap) record_list();
      uint32_t chosen = chosenA | chosenT;
      while (chosen) {
        const int u = __ffs(chosen) - 1;
        chosen &= chosen - 1;
        const int e = cb + u * NT + tid;
        const bool isA = (chosenA >> u) & 1u;
        if (!fits) record(e, isA, isA ? na + oa++ : nt + ot++);
        else if (isA) elist[la + oa++] = e;
        else elist[kListCap - 1 - (lt + ot++)] = e;
      }
      na += ta;
      nt += tt;
      if (fits) { la += ta; lt += tt; }
    }
    if (la + lt > 0) record_list();
  }
  if (tid == 0)
    st_dev(&a.ws.fcnt[(size_t)bh * kMaxFusedP + sub],
           ((unsigned long long)(uint32_t)nt << 32) | (uint32_t)na);
  const bool last2 = barrier_arrive(&sync[kSyncStride], (uint32_t)P);
  // while waiting: this block's own tie records' clusters and weights into LDS
  // (the histogram region is free until the background logits), so that
  // placing its winners needs no global load
  constexpr int kOwnCap = (int)(C::kHBytes / ((1 + G) * sizeof(float)));
  float* ownw = reinterpret_cast<float*>(hist);                  // [kOwnCap][G]
  int* ownc = reinterpret_cast<int*>(ownw + (size_t)kOwnCap * G);   // [kOwnCap]
  for (int i = tid; i < min(nt, kOwnCap); i += NT) {
    const int oc = ftc[E0 + i];
    float ow[G];
#pragma unroll
    for (int g = 0; g < G; ++g) ow[g] = ftw[(size_t)(E0 + i) * G + g];
    ownc[i] = oc;
#pragma unroll
    for (int g = 0; g < G; ++g) ownw[i * G + g] = ow[g];
  }
  barrier_wait(&sync[kSyncStride], (uint32_t)P, a.ws.fflags, last2);

  // ======================================================= phase 3: ties, rows, partials
  // the queries for the exact rows (packed bf16, 8 dims per lane of a 16-lane
  // row), loaded now so that their latency is hidden
  uint4 qp[G];
#pragma unroll
  for (int g = 0; g < G; ++g) qp[g] = *reinterpret_cast<const uint4*>(qh + g * kD + (tid & 15) * 8);
  if (tid < 64) {
    unsigned long long v = 0;
    if (tid < P) v = ld_dev(&a.ws.fcnt[(size_t)bh * kMaxFusedP + tid]);
    const int ca = (int)(uint32_t)v, ct = (int)(v >> 32);
    const int xa = wave_incl_scan(ca), xt = wave_incl_scan(ct);
    if (tid < P) {
      S.apre[tid] = xa - ca;
      S.tpre[tid] = xt - ct;
      S.tbase[tid] = entry_at(min(tid * d.fcpb, d.L));
    }
    if (tid == 63) { S.apre[P] = xa; S.tpre[P] = xt; }
  }
  __syncthreads();
  const int n_above = S.apre[P], n_tie = S.tpre[P];
  const int ksel = min(si.k, n_above + n_tie);
  const int r = max(ksel - n_above, 0);
  unsigned long long* tcache = reinterpret_cast<unsigned long long*>(dyn);
  const bool cached = n_tie <= C::kTieCap;
  auto tie_slot = [&](int i) {
    const int j = seg_of(S.tpre, P, i);
    return S.tbase[j] + (i - S.tpre[j]);
  };
  auto tie_rec = [&](int i) -> unsigned long long {
    return cached ? tcache[i] : ld_dev(&ftie[tie_slot(i)]);
  };
  const int own0 = S.tpre[sub];
  if (r > 0 && cached)
    for (int i = tid; i < n_tie; i += NT) tcache[i] = ld_dev(&ftie[tie_slot(i)]);
  // cluster and weights of the block's own tie i (a head-wide tie index)
  auto own_add = [&](int i) {
    const int t = i - own0;
    int cl;
    float w[G];
    if (t < kOwnCap) {
      cl = ownc[t];
#pragma unroll
      for (int g = 0; g < G; ++g) w[g] = ownw[t * G + g];
    } else {
      const int slot = S.tbase[sub] + t;
      cl = ftc[slot];
#pragma unroll
      for (int g = 0; g < G; ++g) w[g] = ftw[(size_t)slot * G + g];
    }
    cl = min(max(cl, c0), c1 - 1);
#pragma unroll
    for (int g = 0; g < G; ++g) atomicAdd(&wsel[(cl - c0) * G + g], to_fixed(w[g]));
  };
  // this block's rows of the head's exact list [sink | above | tie winners |
  // recent]: every row but the winners is known already
  const int n_rec = si.T - si.recent_beg;
  const int R = si.ns + ksel + n_rec;
  const int lo = (int)((long long)sub * R / P), hi = (int)((long long)(sub + 1) * R / P);
  for (int rr = lo + tid; rr < hi; rr += NT) {
    int p;
    if (rr < si.ns) {
      p = rr;
    } else if (rr < si.ns + n_above) {
      const int s = rr - si.ns;
      const int j = seg_of(S.apre, P, s);
      p = ld_dev(&fpos[S.tbase[j] + (s - S.apre[j])]);
    } else if (rr < si.ns + ksel) {
      continue;
    } else {
      p = si.recent_beg + (rr - si.ns - ksel);
    }
    frows[rr] = p;
  }
  __syncthreads();
  unsigned long long prefix = 0, mask = 0;
  const bool all = r >= n_tie;
  if (r > 0 && !all) {
    int need = r;
    for (int shift = 44;; shift -= 8) {
      const int s = shift > 0 ? shift : 0;
      const unsigned long long dm = shift >= 0 ? 0xffull : 0xfull;
      for (int i = tid; i < 256; i += NT) S.rh[i] = 0;
      __syncthreads();
      for (int i = tid; i < n_tie; i += NT) {
        const unsigned long long cp = tie_composite(tie_rec(i));
        if ((cp & mask) == prefix) atomicAdd(&S.rh[(cp >> s) & dm], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        int v4[4], sl = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int bin = 255 - (tid * 4 + i);
          v4[i] = bin <= (int)dm ? (int)S.rh[bin] : 0;
          sl += v4[i];
        }
        const int x = wave_incl_scan(sl);
        int run = x - sl;
        if (run < need && run + sl >= need) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (run < need && run + v4[i] >= need) {
              S.res[0] = 255 - (tid * 4 + i);
              S.res[1] = run;
              S.res[2] = v4[i];
            }
            run += v4[i];
          }
        }
      }
      __syncthreads();
      const int dig = S.res[0];
      need -= S.res[1];
      prefix |= (unsigned long long)dig << s;
      mask |= dm << s;
      const bool done = S.res[2] == need || s == 0;
      __syncthreads();
      if (done) break;
    }
  }
  auto is_winner = [&](unsigned long long rec) {
    return all || (tie_composite(rec) & mask) >= prefix;
  };
  // tie winners: the rows of this block's share, and the weights of this
  // block's own winners.  With the ties cached, each thread takes a
  // contiguous run of them and one block scan places their rows.
  if (r > 0 && cached) {
    const int per = (n_tie + NT - 1) / NT;
    const int i0 = min(n_tie, tid * per), i1 = min(n_tie, i0 + per);
    int cw = 0;
    for (int i = i0; i < i1; ++i) cw += is_winner(tcache[i]);
    int ow, dummy, tw, td;
    block_scan2<NT>(cw, 0, &ow, &dummy, &tw, &td, S.sh);
    int wi = ow;
    for (int i = i0; i < i1; ++i) {
      const unsigned long long rec = tcache[i];
      if (!is_winner(rec)) continue;
      const int row = si.ns + n_above + wi++;
      if (row >= lo && row < hi) frows[row] = (int32_t)(uint32_t)rec;
      if (i >= own0 && i < S.tpre[sub + 1]) own_add(i);
    }
  } else if (r > 0) {
    int run = 0;
    for (int base2 = 0; base2 < n_tie; base2 += NT) {
      const int i = base2 + tid;
      unsigned long long rec = 0;
      bool win = false;
      if (i < n_tie) {
        rec = tie_rec(i);
        win = is_winner(rec);
      }
      int ow, dummy, tw, td;
      block_scan2<NT>(win, 0, &ow, &dummy, &tw, &td, S.sh);
      if (win) {
        const int row = si.ns + n_above + run + ow;
        if (row >= lo && row < hi) frows[row] = (int32_t)(uint32_t)rec;
        if (i >= own0 && i < S.tpre[sub + 1]) own_add(i);
      }
      run += tw;
    }
  }
  __syncthreads();
  // background logits of the block's clusters: log2 of the unselected weight
  // (relative to the cluster max) plus the max
  float* sbg = reinterpret_cast<float*>(hist);
  long long* ioff = reinterpret_cast<long long*>(dyn + C::kUBytes + 4096);
  for (int i = tid; i < ncl * G; i += NT) {
    const int cl = c0 + i / G, g = i % G;
    const float M = binl[((cl - c0) * G + g) * 2];
    const float wb = binl[((cl - c0) * G + g) * 2 + 1] - (float)wsel[i] * kFixInv;
    sbg[i] = (wb > 0.0f && M != -INFINITY) ? M + log2f(wb) : -INFINITY;
  }
  // exact rows and background clusters as one item list through 16-lane groups
  const int l16 = tid & 15, rg = tid >> 4;
  AttnState<G> st;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.m[g] = -INFINITY;
    st.l[g] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) st.acc[g][i] = 0.0f;
  }
  const int nr = hi - lo;
  const int n_items = nr + (d.exact_only ? 0 : ncl);   // background items last
  const int32_t* tab = a.table + (size_t)b * d.max_pages;
  const uint16_t* kc = a.kc + l16 * 8;
  const uint16_t* vc = a.vc + l16 * 8;
  const float* means = a.ix.means + (size_t)bh * d.L * kD + l16 * 8;
  // Items are staged up to kStage at a time (their cache offsets in LDS); a
  // 16-lane group takes items rg, rg + NG, ... in that order, with the loads
  // of the next kIB of them in flight while it computes.
  constexpr int kStage = (int)((C::kHBytes - 4096) / sizeof(long long));
  for (int ph = 0; ph < n_items; ph += kStage) {
    const int n = min(kStage, n_items - ph);
    __syncthreads();
    {
      // a thread's rows, then their pages, each round of loads issued at once
      constexpr int kPerT = (kStage + NT - 1) / NT;
      int pr[kPerT], pg[kPerT];
#pragma unroll
      for (int i = 0; i < kPerT; ++i) {
        const int t = tid + i * NT, it = ph + t;
        pr[i] = (t < n && it < nr) ? min(max(frows[lo + it], 0), d.cap - 1) : -1;
      }
#pragma unroll
      for (int i = 0; i < kPerT; ++i) pg[i] = pr[i] >= 0 ? tab[pr[i] >> 4] : 0;
#pragma unroll
      for (int i = 0; i < kPerT; ++i) {
        const int t = tid + i * NT, it = ph + t;
        if (t < n) {
          if (it < nr) {
            const int page = min(max(pg[i], 0), d.num_pages - 1);
            ioff[t] = ((long long)(page * kPage + (pr[i] & (kPage - 1))) * d.Hkv + h) * kD;
          } else {
            ioff[t] = -1 - (long long)(it - nr);
          }
        }
      }
    }
    __syncthreads();
    auto load_item = [&](int j, uint4& kw, uint4& vw) {
      kw = vw = make_uint4(0, 0, 0, 0);
      if (j < n) {
        const long long o = ioff[j];
        if (o >= 0) {
          kw = *reinterpret_cast<const uint4*>(kc + o);
          vw = *reinterpret_cast<const uint4*>(vc + o);
        } else {
          const float* mu = means + (size_t)(c0 + (int)(-1 - o)) * kD;
          kw = *reinterpret_cast<const uint4*>(mu);
          vw = *reinterpret_cast<const uint4*>(mu + 4);
        }
      }
    };
    uint4 kw[kIB], vw[kIB];
#pragma unroll
    for (int u = 0; u < kIB; ++u) load_item(rg + u * NG, kw[u], vw[u]);
    for (int j0 = rg; j0 < n; j0 += kIB * NG) {
#pragma unroll
      for (int u = 0; u < kIB; ++u) {
        const int j = j0 + u * NG;
        if (j < n) {
          const long long o = ioff[j];
          if (o >= 0) attend_row_pk<G>(st, qp, d.scale_log2, kw[u], vw[u]);
          else attend_bg<G>(st, sbg + (int)(-1 - o) * G, kw[u], vw[u]);
        }
        load_item(j + kIB * NG, kw[u], vw[u]);
      }
    }
  }
  __syncthreads();
  // Block merge: every row group's state goes to LDS; the weight of each
  // (row group, head) against the head's max is computed once; then each
  // thread sums one output (head, dim) over the row groups.
  static_assert(NG == 32 && (size_t)NG * G * kD * sizeof(float) <= C::kUBytes, "row states");
  float* accr = reinterpret_cast<float*>(dyn);           // [NG][G][128]
  float* mlr = reinterpret_cast<float*>(hist);           // [NG][G][2]
  float* fr = mlr + NG * G * 2;                          // [G][NG]
  float* mlg = fr + G * NG;                              // [G][2] head max and sum
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (l16 == 0) {
      mlr[(rg * G + g) * 2] = st.m[g];
      mlr[(rg * G + g) * 2 + 1] = st.l[g];
    }
    float4* dst = reinterpret_cast<float4*>(accr + ((size_t)rg * G + g) * kD + l16 * 8);
    dst[0] = make_float4(st.acc[g][0], st.acc[g][1], st.acc[g][2], st.acc[g][3]);
    dst[1] = make_float4(st.acc[g][4], st.acc[g][5], st.acc[g][6], st.acc[g][7]);
  }
  __syncthreads();
  if (tid < G * NG) {
    // one 32-lane half wave per head
    const int g = tid / NG, r = tid % NG;
    const float m = mlr[(r * G + g) * 2];
    float M = m;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float f = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - M);
    fr[g * NG + r] = f;
    float L = f * mlr[(r * G + g) * 2 + 1];
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) L += __shfl_xor(L, o);
    if (r == 0) { mlg[g * 2] = M; mlg[g * 2 + 1] = L; }
  }
  __syncthreads();
  for (int idx = tid; idx < G * kD; idx += NT) {
    const int g = idx / kD, dim = idx % kD;
    float A = 0.0f;
#pragma unroll 8
    for (int r = 0; r < NG; ++r) A = fmaf(fr[g * NG + r], accr[((size_t)r * G + g) * kD + dim], A);
    float* out = a.ws.fpart + (((size_t)bh * G + g) * kMaxFusedP + sub) * kPart;
    st_dev(&out[4 + dim], A);
    if (dim == 0) {
      st_dev(&out[0], mlg[g * 2]);
      st_dev(&out[1], mlg[g * 2 + 1]);
    }
  }
  wait_mem();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old =
        __hip_atomic_fetch_add(&sync[2 * kSyncStride], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    S.last = old == (uint32_t)(P - 1);
  }
  __syncthreads();
  if (!S.last) return;

  // ======================================================= last block of the head
  // every (head, dim) thread loads its column of the P partials (a wave's
  // loads of one partial are contiguous) while one wave per head loads the
  // (m, l) pairs and forms the weights of the partials against the head's max
  {
    float* fp = reinterpret_cast<float*>(hist);     // [G][64] weights
    float* mlh = fp + G * kMaxFusedP;               // [G][2] head max and sum
    constexpr int kOut = (G * kD + NT - 1) / NT;    // outputs per thread
    const float* pbase = a.ws.fpart + (size_t)bh * G * kMaxFusedP * kPart;
    float x[kMaxFusedP];
    auto load_col = [&](int o) {
      // threads past the outputs load a valid column and discard it
      const int idx = min(tid + o * NT, G * kD - 1);
      const float* col = pbase + (size_t)(idx / kD) * kMaxFusedP * kPart + 4 + idx % kD;
#pragma unroll
      for (int j = 0; j < kMaxFusedP; ++j) x[j] = j < P ? ld_dev(&col[(size_t)j * kPart]) : 0.0f;
    };
    load_col(0);
    for (int g = wave; g < G; g += NW) {
      const float* pp = pbase + ((size_t)g * kMaxFusedP + lane) * kPart;
      const float m = lane < P ? ld_dev(&pp[0]) : -INFINITY;
      const float l = lane < P ? ld_dev(&pp[1]) : 0.0f;
      const float M = wave_max_dpp(m);
      const float f = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - M);
      fp[g * kMaxFusedP + lane] = f;
      const float L = wave_sum_dpp(f * l);
      if (lane == 0) { mlh[g * 2] = M; mlh[g * 2 + 1] = L; }
    }
    __syncthreads();
#pragma unroll
    for (int o = 0; o < kOut; ++o) {
      if (o > 0) load_col(o);
      const int idx = tid + o * NT;
      if (idx < G * kD) {
        const int g = idx / kD, dim = idx % kD;
        const float* fg = fp + g * kMaxFusedP;
        float A = 0.0f;
        // weights and loads are 0 for j >= P
#pragma unroll
        for (int j = 0; j < kMaxFusedP; ++j) A = fmaf(fg[j], x[j], A);
        const float M = mlh[g * 2], L = mlh[g * 2 + 1];
        const size_t bq = (size_t)b * d.Hq + h * G + g;
        a.out[bq * kD + dim] = L > 0.0f ? A / L : 0.0f;
        if (dim == 0 && a.lse)
          a.lse[bq] = L > 0.0f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
      }
    }
  }
  if (a.selected) {
    // ascending selected positions through a bitmap over positions
    uint32_t* bits = reinterpret_cast<uint32_t*>(dyn);
    const int nw = d.nwords;
    __syncthreads();
    for (int i = tid; i < nw; i += NT) bits[i] = 0u;
    __syncthreads();
    for (int s = tid; s < n_above; s += NT) {
      const int j = seg_of(S.apre, P, s);
      const int p = ld_dev(&fpos[S.tbase[j] + (s - S.apre[j])]);
      if (p >= 0 && p < d.cap) atomicOr(&bits[p >> 5], 1u << (p & 31));
    }
    if (r > 0) {
      for (int i = tid; i < n_tie; i += NT) {
        const unsigned long long rec = ld_dev(&ftie[tie_slot(i)]);
        const int p = (int)(uint32_t)rec;
        if (is_winner(rec) && p >= 0 && p < d.cap) atomicOr(&bits[p >> 5], 1u << (p & 31));
      }
    }
    __syncthreads();
    const int per = (nw + NT - 1) / NT;
    const int w0 = min(nw, tid * per), w1 = min(nw, w0 + per);
    int cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(bits[w]);
    int oc, dummy, tc, td;
    block_scan2<NT>(cnt, 0, &oc, &dummy, &tc, &td, S.sh);
    int32_t* selout = a.selected + (size_t)bh * a.max_sel;
    int at = oc;
    for (int w = w0; w < w1; ++w) {
      uint32_t bw = bits[w];
      while (bw) {
        const int bit = __ffs(bw) - 1;
        bw &= bw - 1;
        if (at < a.max_sel) selout[at] = w * 32 + bit;
        ++at;
      }
    }
    for (int i = tc + tid; i < a.max_sel; i += NT) selout[i] = -1;
  }
  if (tid == 0) a.ws.n_rows[bh] = R;
  // every block of the head is past both barriers and has read the histogram
  for (int i = tid; i < kHistBins; i += NT) st_dev(&ghist[i], 0u);
  if (tid == 0) {
    st_dev(&sync[0], 0u);
    st_dev(&sync[kSyncStride], 0u);
    st_dev(&sync[2 * kSyncStride], 0u);
  }
}

// ---------------------------------------------------------------- host side
namespace {

struct FusedDeviceInfo {
  int ready;        // 0 unknown, 1 known
  int cus;
  int occ[4];       // blocks per CU for G = 1, 2, 4, 8
};

constexpr int kMaxDevices = 64;
FusedDeviceInfo g_info[kMaxDevices];

int g_index(int G) { return G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3; }

template <int G>
hipError_t prepare_g(int* occ) {
  using C = FusedCfg<G>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_fused<G>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::kDyn);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, k_fused<G>, C::NT, C::kDyn);
}

const FusedDeviceInfo* device_info() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  FusedDeviceInfo& fi = g_info[dev];
  if (__atomic_load_n(&fi.ready, __ATOMIC_ACQUIRE)) return &fi;
  FusedDeviceInfo t{};
  if (hipDeviceGetAttribute(&t.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return nullptr;
  if (prepare_g<1>(&t.occ[0]) != hipSuccess || prepare_g<2>(&t.occ[1]) != hipSuccess ||
      prepare_g<4>(&t.occ[2]) != hipSuccess || prepare_g<8>(&t.occ[3]) != hipSuccess)
    return nullptr;
  t.ready = 1;
  fi.cus = t.cus;
  for (int i = 0; i < 4; ++i) fi.occ[i] = t.occ[i];
  __atomic_store_n(&fi.ready, 1, __ATOMIC_RELEASE);
  return &fi;
}

}  // namespace

size_t fused_lds_bytes(int G) {
  switch (G) {
    case 1: return FusedCfg<1>::kDyn;
    case 2: return FusedCfg<2>::kDyn;
    case 4: return FusedCfg<4>::kDyn;
    case 8: return FusedCfg<8>::kDyn;
  }
  return 0;
}

int fused_cluster_cap(int G) {
  switch (G) {
    case 1: return FusedCfg<1>::kCG;
    case 2: return FusedCfg<2>::kCG;
    case 4: return FusedCfg<4>::kCG;
    case 8: return FusedCfg<8>::kCG;
  }
  return 0;
}

int fused_blocks_per_head(const Dims& d) {
  const FusedDeviceInfo* fi = device_info();
  if (!fi || fi->occ[g_index(d.G)] < 1) return 0;
  const int BH = d.B * d.Hkv;
  const long long total = (long long)fi->occ[g_index(d.G)] * fi->cus;
  long long p0 = total / BH;
  if (p0 > kMaxFusedP) p0 = kMaxFusedP;
  if (p0 > d.L) p0 = d.L;
  // no more blocks than about 1024 index entries each: below that the scan is
  // short and every extra block only adds a partial to merge
  const long long by_work = ((long long)d.cap + 1023) / 1024;
  if (p0 > by_work) p0 = by_work;
  if (p0 < 1) return 0;
  const int cpb = (int)((d.L + p0 - 1) / p0);
  if ((long long)cpb * d.G > fused_cluster_cap(d.G)) return 0;
  // the selected-position bitmap of the last block lives in LDS
  const size_t lut_hist = (size_t)kM * kKsub * d.G * sizeof(float) + kHistBins * sizeof(uint32_t);
  if ((size_t)d.nwords * 4 > lut_hist) return 0;
  return (d.L + cpb - 1) / cpb;
}

template <int G>
static hipError_t fused_g(const StepArgs& a, const Launch& l) {
  using C = FusedCfg<G>;
  return launch_kernel(k_fused<G>, dim3(a.d.B * a.d.Hkv * a.d.fP), dim3(C::NT), C::kDyn, l, a);
}

hipError_t launch_fused(const StepArgs& a, const Launch& l) {
  switch (a.d.G) {
    case 1: return fused_g<1>(a, l);
    case 2: return fused_g<2>(a, l);
    case 4: return fused_g<4>(a, l);
    case 8: return fused_g<8>(a, l);
  }
  return hipErrorInvalidValue;
}

}  // namespace pqhsa
