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
//   phase 3  every block resolves the tie bucket alike (64-bit composite:
//            the full key, then the inverted position, so equal keys prefer
//            the lower position; rank counting for up to 512 ties, 128 at
//            G = 8, else a radix select), takes an even share of the exact
//            rows (sink, selected, recent/tail) plus its own clusters'
//            background terms, attends them in the 16-row MFMA tiles of the
//            dense step, and writes one partial (m, l, acc[128]) per query
//            head.  The P partials are merged into O and the log-sum-exp by
//            the head's last block to finish (found by a counter), or at
//            G = 8 by one merger block per query head that polls tagged
//            partials; the last block (block 0 at G = 8) writes the
//            ascending selected positions if asked and clears the head's
//            counters and histogram for the next step.
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
// the workspace flags and the head's own flag, and the step goes on, so a call
// always finishes; the head's outputs are then NaN instead of a result (the
// last block reads the head's flag; at G = 8 the mergers see the timeout in
// the partials' tags, and a merger whose own wait for the partials runs out
// sets the flag too).  Counts read across blocks are clamped to each block's
// own entry range, so that whatever a late block left behind, every access
// stays inside its array.
#include "pqhsa_internal.hpp"

namespace pqhsa {

namespace {

template <int G>
struct FusedCfg {
  static constexpr int NT = 512;   // 8 waves: up to 256 VGPRs each
  static constexpr int NW = NT / 64;
  static constexpr size_t kUBytes = (size_t)kM * kKsub * G * sizeof(float);   // LUT, then reuse
  static constexpr size_t kHBytes = (size_t)kHistBins * sizeof(uint32_t);
  // clusters x G per block whose per-cluster values live in LDS (smaller at
  // G = 8, whose 128 KB LUT leaves less room)
  static constexpr int kCG = G == 8 ? kFusedWselMax / 2 : kFusedWselMax;
  static constexpr size_t kWBytes = (size_t)kCG * sizeof(unsigned long long);   // selected weights
  static constexpr size_t kQBytes = (size_t)kCG * sizeof(float);                // cluster logits
  static constexpr size_t kBBytes = (size_t)kCG * 2 * sizeof(float);            // cluster (max, sum)
  // 16-bit keys of the block's entries, from the scan to phase 2, when the
  // block has at most kKeyCap entries (none at G = 8: no LDS left)
  static constexpr int kKeyCap = G == 8 ? 0 : 8192;
  static constexpr size_t kKBytes = (size_t)kKeyCap * sizeof(uint16_t);
  static constexpr size_t kDyn = kUBytes + kHBytes + kWBytes + kQBytes + kBBytes + kKBytes;
  static constexpr int kTieCap = (int)(kUBytes / sizeof(unsigned long long));
};

// Threshold-bucket ties resolved by counting ranks, at most: a tie bucket at
// the 512K shape (G = 8) holds ~200 ties, for which the radix select is faster.
template <int G>
constexpr int kRankMax = G == 8 ? 128 : 512;

struct FusedStatic {
  unsigned long long thr;   // the r-th largest tie composite
  uint32_t dif[2];  // bits at which cached tie composites differ (low, high word)
  int nextc;        // the scan's next unclaimed cluster of the block
  int sh[40];
  uint32_t rh[256];
  int res[4];
  int tout;         // 1: a barrier wait of this block ran out
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
// have arrived or `ticks` of the 100 MHz clock have passed; then bit 0 of
// *flags (the workspace's word), of *hflag (the head's) and of *tout (the
// block's, in LDS) are set.
__device__ bool barrier_arrive(uint32_t* ctr, uint32_t n) {
  wait_mem();
  __syncthreads();
  bool last = false;
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 >= n;
  return last;
}

__device__ void barrier_wait(uint32_t* ctr, uint32_t n, uint32_t* flags, uint32_t* hflag,
                             int* tout, unsigned int ticks, bool last) {
  if (threadIdx.x == 0 && !last) {
    const unsigned long long t0 = wall_clock64();
    while (ld_dev(ctr) < n) {
      __builtin_amdgcn_s_sleep(8);
      if (wall_clock64() - t0 > ticks) {
        __hip_atomic_fetch_or(flags, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_or(hflag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *tout = 1;
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
  lds_sync();
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
  lds_sync();
  *oa = sh[wave] + xa - a;
  *ob = sh[NW + 1 + wave] + xb - b;
  *ta = sh[NW];
  *tb = sh[2 * NW + 1];
  lds_sync();
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
  lds_sync();
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
  lds_sync();
}

// 16-bit code of an order key, monotone (a larger key never gets a smaller
// code): the sign, the binary exponent clamped to a window of 16 binades
// (|x| in [2^-7, 2^9), where base-2 logits of interest lie), then 11 mantissa
// bits.  Its top 12 bits are the histogram bin: 128 bins per binade, 16 times
// finer than the key's own top 12 bits, so that far fewer keys share the
// threshold bin.  Keys outside the window share the window's edge bins, and
// ties are resolved on the full key, so selection stays exact for any input.
// 0 stays reserved for "not a candidate".
constexpr int kWinLo = 127 - 7;   // lowest biased exponent of the window
__device__ __forceinline__ uint32_t key_code16(uint32_t u) {
  const uint32_t s = u >> 31;
  // the exponent field of the order key: e for x >= 0, 255 - e below 0; the
  // window is the same field range [kWinLo, kWinLo + 15] in both halves
  const int f = (int)((u >> 23) & 0xffu);
  uint32_t v;
  if (f < kWinLo) v = 0;
  else if (f > kWinLo + 15) v = 0x7fffu;
  else v = ((uint32_t)(f - kWinLo) << 11) | ((u >> 12) & 0x7ffu);
  return max((s << 15) | v, 1u);
}

// Selection order of a tie record (rec = key << 32 | position): the key,
// then the lower position.
__device__ __forceinline__ unsigned long long tie_composite(unsigned long long rec) {
  return rec ^ 0xffffffffull;
}

__device__ __forceinline__ unsigned long long to_fixed(float w) {
  return (unsigned long long)(w * kFixScale + 0.5f);
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
  constexpr int NT = C::NT, NW = C::NW;
  constexpr int PT = 5;   // 64-entry tiles per scan round (most clusters in one)
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
  // the scan's keys reach phase 2 through LDS when they fit, else through
  // the workspace (which also gets them when asked to)
  uint16_t* klds = reinterpret_cast<uint16_t*>(dyn + C::kDyn - C::kKBytes);
  const bool lkeys = E1 - E0 <= C::kKeyCap;
  const bool gkeys = !lkeys || d.fkeys_out != 0;
  const SeqInfo si = seq_info(d, a.ctx, a.ix.n_indexed, b);
  // the head's three counters (barrier 1, barrier 2, finished blocks), each on
  // its own cache line: heads and counters do not contend for one line
  uint32_t* sync = a.ws.fsync + (size_t)bh * 3 * kSyncStride;
  // the head's timeout flag shares the finished-blocks line
  uint32_t* hflag = sync + 2 * kSyncStride + 1;
  // The head's partials, [G][kMaxFusedP][kPart].  At G = 8 (tagged) each word
  // is 64-bit, a float (low half) and a tag (high half: 0 not written in this
  // step, 1 written, 2 written by a block one of whose barrier waits ran
  // out), and mergers poll the tags; elsewhere plain floats that the head's
  // last block reads after the finished-blocks counter.
  constexpr bool kTagged = G == 8;
  unsigned long long* hpart = a.ws.fpart + (size_t)bh * G * kMaxFusedP * kPart;
  float* hpartf = reinterpret_cast<float*>(a.ws.fpart) + (size_t)bh * G * kMaxFusedP * kPart;
  const uint32_t nbar = (uint32_t)(P + d.fbar_extra);   // arrivals a barrier waits for
  uint32_t* ghist = a.ws.hist + (size_t)bh * kHistStride;
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
  // one round's codes and positions (-1: past the cluster)
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
  // the same for the first round, where lanes past the cluster load its
  // first entry (or entry 0) instead, so that every thread issues the same
  // loads in phase 1 and the waits on them are exact
  auto issue_all = [&](FRound<G, PT>& r, int base, int e1) {
#pragma unroll
    for (int t = 0; t < PT; ++t) {
      const int e = base + t * 64 + lane;
      const int el = e < e1 ? e : min(base, max(d.cap - 1, 0));
      r.cw[t] = codes[el];
      r.pp[t] = pos[el];
      if (e >= e1) r.pp[t] = -1;
    }
  };
  // the wave's first round goes out before the tables are built
  int c = c0 + wave;
  int e0 = 0, e1 = 0;
  FRound<G, PT> rb[2];
  {
    // LUT[m][j][g] = scale*log2e * q_g^(m) . B_m[j].  Thread t computes the
    // entries of subspace m = t / 32 for codewords j = t % 32 + 32 i: its
    // q^(m) of the G heads stays in registers, and the lanes of a half wave
    // read consecutive codebook rows.  Loads go out in the order they are
    // needed (they complete in issue order, and every thread issues the same
    // ones): q, then the codebook rows and the first centroids, then the
    // scan's first round (the cluster offsets are scalar loads).
    constexpr int kTPM = NT / kM;           // threads per subspace
    constexpr int kPer = kKsub / kTPM;      // codewords per thread
    static_assert(kTPM * kM == NT && kPer * kTPM == kKsub, "LUT split");
    const int lm = tid / kTPM, lj = tid % kTPM;
    const int l16r = tid & 15;
    // q of the G heads, packed bf16: subspace lm (LUT) and dims l16r*8.. (QC)
    uint4 qlw[G], qcw[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      qlw[g] = *reinterpret_cast<const uint4*>(qh + g * kD + lm * kDsub);
      qcw[g] = *reinterpret_cast<const uint4*>(qh + g * kD + l16r * 8);
    }
    if (c < c1) {
      e0 = entry_at(c);
      e1 = max(e0, entry_at(c + 1));
    }
    float4 cb[kPer][2];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const float* cw =
          a.ix.codebooks + (((size_t)bh * kM + lm) * kKsub + lj + kTPM * i) * kDsub;
      cb[i][0] = *reinterpret_cast<const float4*>(cw);
      cb[i][1] = *reinterpret_cast<const float4*>(cw + 4);
    }
    // the first cluster of this thread's 16-lane row for the QC pass
    float4 cen0, cen1;
    {
      const int cl0 = min(c0 + min(tid >> 4, max(ncl - 1, 0)), d.L - 1);
      const float* cp = cent + (size_t)cl0 * kD + l16r * 8;
      cen0 = *reinterpret_cast<const float4*>(cp);
      cen1 = *reinterpret_cast<const float4*>(cp + 4);
    }
    issue_all(rb[0], e0, e1);
    // keep every load above in flight before any of them is used (the
    // scheduler would otherwise sink the codebook loads into the loop below,
    // one memory round trip per piece)
    __builtin_amdgcn_sched_barrier(0);
    // the scaled q values, as the staged table kernel forms them
    auto scaled = [&](const uint4& w, float* f) {
      const float v[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                          bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = v[i] * d.scale_log2;
    };
    float qr[G][kDsub];
#pragma unroll
    for (int g = 0; g < G; ++g) scaled(qlw[g], qr[g]);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int j = lj + kTPM * i;
      const float cv[8] = {cb[i][0].x, cb[i][0].y, cb[i][0].z, cb[i][0].w,
                           cb[i][1].x, cb[i][1].y, cb[i][1].z, cb[i][1].w};
      float outv[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float sacc = qr[g][0] * cv[0];
#pragma unroll
        for (int t = 1; t < kDsub; ++t) sacc = fmaf(qr[g][t], cv[t], sacc);
        outv[g] = sacc;
      }
      float* dst = lut + (lm * kKsub + j) * G;
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
        float qq[8];
        scaled(qcw[g], qq);
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
    for (int i = tid; i < kHistBins; i += NT) hist[i] = 0u;
    for (int i = tid; i < ncl * G; i += NT) wsel[i] = 0ull;
    if (tid == 0) {
      S.nextc = c0 + NW;
      S.tout = 0;
    }
  }
  // LDS only: the scan's first round stays in flight
  lds_sync();
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
        uint32_t code = 0;
        if (p >= si.cand_beg && p < si.cand_end) {
          code = key_code16(order_key(kappa));
          atomicAdd(&hist[code >> (16 - kHistBits)], 1u);
#pragma unroll
          for (int g = 0; g < G; ++g) s[t][g] = v[g];
        }
        if (lkeys) klds[e - E0] = (uint16_t)code;
        if (gkeys) keys[e] = (uint16_t)code;
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
  lds_sync();
  // The block's own threshold bucket beta_b: at least k of its keys lie in
  // bins >= beta_b, so the head's threshold bucket is >= beta_b and the bins
  // below cannot matter.  Only bins >= beta_b go to the head's histogram
  // (fewer atomics on shared lines), and only those are read back.
  block_threshold<NT>(hist, 0, si.k, S.res, S.sh);
  const int beta_b = S.res[0];   // -1: no candidate in this block, or k = 0
  // with fewer than k candidates of its own the block flushes every bin, and
  // the head's threshold may lie below its bins: it then reads them all
  const int read_lo = S.res[2] >= si.k ? beta_b : 0;
  lds_sync();
  if (beta_b >= 0) {
    for (int i = beta_b + tid; i < kHistBins; i += NT) {
      const uint32_t v = hist[i];
      if (v) __hip_atomic_fetch_add(&ghist[i], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  const bool last1 = barrier_arrive(&sync[0], nbar);
  if constexpr (kTagged) {
    // while waiting: this block's partial slots are marked unwritten; the
    // stores complete before the block arrives at barrier 2, so no merger
    // (which reads after barrier 2) can take a slot left from an earlier step
    for (int i = tid; i < G * kPart; i += NT)
      st_dev(&hpart[((size_t)(i / kPart) * kMaxFusedP + sub) * kPart + i % kPart], 0ull);
  }
  // while waiting: this block's first keys for the classification below
  // (kPer per thread, so that phase 2 takes a block's entries in one chunk
  // when it holds up to NT * kPer of them: 18 at G = 8, whose blocks at the
  // 512K shape hold 7.9K-8.4K entries; 16 elsewhere, where 18 measured
  // slower at the 16-sequence batch)
  constexpr int kPer = G == 8 ? 18 : 16;
  uint32_t pk[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int e = E0 + u * NT + tid;
    pk[u] = e < E1 ? (lkeys ? klds[e - E0] : keys[e]) : 0u;
  }
  barrier_wait(&sync[0], nbar, a.ws.fflags, hflag, &S.tout, d.fbar_ticks, last1);

  // ======================================================= phase 2: threshold bucket
  // the head's histogram from read_lo up: exact there, because every block
  // with at least k candidates added all its bins >= its own beta_b <= beta,
  // and every other block added all of its bins
  int beta = -1;
  if (beta_b >= 0) {
    for (int i = read_lo + tid; i < kHistBins; i += NT) hist[i] = ld_dev(&ghist[i]);
    lds_sync();
    block_threshold<NT>(hist, read_lo, si.k, S.res, S.sh);
    beta = S.res[0];
    lds_sync();
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
    lds_sync();
    for (int li = tid; li < la + lt; li += NT) {
      const bool isA = li < la;
      if (isA) record(elist[li], true, na - la + li);
      else record(elist[kListCap - 1 - (li - la)], false, nt - lt + (li - la));
    }
    la = lt = 0;
    lds_sync();
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
    lds_sync();
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
          pk[u] = e < E1 ? (lkeys ? klds[e - E0] : keys[e]) : 0u;
        }
      }
      int oa, ot, ta, tt;
      block_scan2<NT>(ca, ct, &oa, &ot, &ta, &tt, S.sh);
      const bool fits = ta + tt <= kListCap;
      // the listed entries are recorded at the last slots counted so far: a
      // chunk that is recorded directly (or would overflow the list) goes
      // after them, so they are recorded first
      if (la + lt > 0 && (!fits || la + lt + ta + tt > kListCap)) record_list();
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
  const bool last2 = barrier_arrive(&sync[kSyncStride], nbar);
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
  barrier_wait(&sync[kSyncStride], nbar, a.ws.fflags, hflag, &S.tout, d.fbar_ticks, last2);

  // ======================================================= phase 3: ties, rows, partials
  // the queries as the row tiles' B operand, loaded now so that their latency
  // is hidden
  const int tcol = lane & 15, tj = lane >> 4;
  bf16x8 qb[4];
  tile_query<G>(qh, tcol, tj, qb);
  if (tid < 64) {
    unsigned long long v = 0;
    int jb = 0, je = 0;   // block tid's entries [jb, je)
    if (tid < P) {
      v = ld_dev(&a.ws.fcnt[(size_t)bh * kMaxFusedP + tid]);
      jb = entry_at(min(tid * d.fcpb, d.L));
      je = max(jb, entry_at(min((tid + 1) * d.fcpb, d.L)));
    }
    // a block lists at most its own entries; clamping keeps every record
    // index inside the block's range even after a barrier wait ran out
    const int ca = min((int)min((uint32_t)v, 0x7fffffffu), je - jb);
    const int ct = min((int)min((uint32_t)(v >> 32), 0x7fffffffu), je - jb - ca);
    const int xa = wave_incl_scan(ca), xt = wave_incl_scan(ct);
    if (tid < P) {
      S.apre[tid] = xa - ca;
      S.tpre[tid] = xt - ct;
      S.tbase[tid] = jb;
    }
    if (tid == 63) { S.apre[P] = xa; S.tpre[P] = xt; }
  }
  lds_sync();
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
  // This block's rows of the head's exact list [sink | above | tie winners |
  // recent]: every row but the winners is known already.  When the block's
  // share fits one staging (and the cached ties leave room at the top of the
  // LUT region), the rows go straight to LDS: the known rows' positions are
  // loaded now, so that their latency overlaps the tie loads and the tie
  // selection, and the winners are placed there by the selection; otherwise
  // they go through the head's row list in the workspace.
  const int n_rec = si.T - si.recent_beg;
  const int R = si.ns + ksel + n_rec;
  const int lo = (int)((long long)sub * R / P), hi = (int)((long long)(sub + 1) * R / P);
  const int nr = hi - lo;
  constexpr int kStage = (int)((C::kHBytes - 4096) / sizeof(long long));   // rows per staging
  constexpr int kPerT = (kStage + NT - 1) / NT;
  const size_t tie_bytes = (r > 0 && cached) ? (size_t)n_tie * sizeof(unsigned long long) : 0;
  const bool direct =
      nr <= kStage && tie_bytes + (size_t)kStage * (sizeof(long long) + sizeof(int32_t)) <= C::kUBytes;
  long long* ioffd = reinterpret_cast<long long*>(dyn + C::kUBytes - (size_t)kStage * sizeof(long long));
  int32_t* posd = reinterpret_cast<int32_t*>(ioffd) - kStage;   // winners' positions
  auto known_pos = [&](int rr) -> int {   // -1 for a tie winner's row
    if (rr < si.ns) return rr;
    if (rr < si.ns + n_above) {
      const int s = rr - si.ns;
      const int j = seg_of(S.apre, P, s);
      return ld_dev(&fpos[S.tbase[j] + (s - S.apre[j])]);
    }
    if (rr < si.ns + ksel) return -1;
    return si.recent_beg + (rr - si.ns - ksel);
  };
  int kp[kPerT];
#pragma unroll
  for (int u = 0; u < kPerT; ++u) kp[u] = -1;
  if (direct) {
#pragma unroll
    for (int u = 0; u < kPerT; ++u) {
      const int rr = lo + tid + u * NT;
      if (rr < hi) kp[u] = known_pos(rr);
    }
  } else {
    for (int rr = lo + tid; rr < hi; rr += NT) {
      const int p = known_pos(rr);
      if (p >= 0) frows[rr] = p;
    }
  }
  if (r > 0 && cached)
    for (int i = tid; i < n_tie; i += NT) tcache[i] = ld_dev(&ftie[tie_slot(i)]);
  if (G == 8 && tid == 0) { S.dif[0] = 0u; S.dif[1] = 0u; }
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
  lds_sync();
  // the r winners of the bucket: the composites >= the r-th largest
  // (prefix under mask)
  unsigned long long prefix = 0, mask = 0;
  const bool all = r >= n_tie;
  if (r > 0 && !all && cached && n_tie <= kRankMax<G>) {
    // few ties: each one counts the ties above it; the one with r - 1 above
    // is the r-th largest (composites are distinct: positions are)
    for (int i = tid; i < n_tie; i += NT) {
      const unsigned long long ci = tie_composite(tcache[i]);
      int above = 0;
      for (int j = 0; j < n_tie; ++j) above += tie_composite(tcache[j]) > ci;
      if (above == r - 1) S.thr = ci;
    }
    lds_sync();
    prefix = S.thr;
    mask = ~0ull;
  } else if (r > 0 && !all) {
    // many ties: radix select over the composites, 8 bits at a time; at
    // G = 8 from the highest bit at which the cached ties differ (they share
    // every bit above it: the bucket's and more), where one round usually
    // isolates the r-th largest; else from the top
    int s0 = 56;
    if (G == 8 && cached) {
      const unsigned long long c0v = tie_composite(tcache[0]);
      unsigned long long dv = 0;
      for (int i = tid; i < n_tie; i += NT) dv |= tie_composite(tcache[i]) ^ c0v;
      uint32_t lo32 = (uint32_t)dv, hi32 = (uint32_t)(dv >> 32);
      for (int o = 32; o >= 1; o >>= 1) {
        lo32 |= __shfl_xor(lo32, o);
        hi32 |= __shfl_xor(hi32, o);
      }
      if (lane == 0 && (lo32 | hi32)) {
        atomicOr(&S.dif[0], lo32);
        atomicOr(&S.dif[1], hi32);
      }
      lds_sync();
      const unsigned long long dif = ((unsigned long long)S.dif[1] << 32) | S.dif[0];
      // dif != 0 when the composites are distinct (positions are)
      s0 = dif ? max(63 - __clzll((long long)dif) - 7, 0) : 0;
    }
    int need = r;
    for (int s = s0;; s = max(s - 8, 0)) {
      constexpr unsigned long long dm = 0xffull;
      for (int i = tid; i < 256; i += NT) S.rh[i] = 0;
      lds_sync();
      for (int i = tid; i < n_tie; i += NT) {
        const unsigned long long cp = tie_composite(tie_rec(i));
        if ((cp & mask) == prefix) atomicAdd(&S.rh[(cp >> s) & dm], 1u);
      }
      lds_sync();
      if (tid < 64) {
        int v4[4], sl = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int bin = 255 - (tid * 4 + i);
          v4[i] = (int)S.rh[bin];
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
      lds_sync();
      const int dig = S.res[0];
      need -= S.res[1];
      prefix |= (unsigned long long)dig << s;
      mask |= dm << s;
      const bool done = S.res[2] == need || s == 0;
      lds_sync();
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
      if (row >= lo && row < hi) {
        if (direct) posd[row - lo] = (int32_t)(uint32_t)rec;
        else frows[row] = (int32_t)(uint32_t)rec;
      }
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
        if (row >= lo && row < hi) {
          if (direct) posd[row - lo] = (int32_t)(uint32_t)rec;
          else frows[row] = (int32_t)(uint32_t)rec;
        }
        if (i >= own0 && i < S.tpre[sub + 1]) own_add(i);
      }
      run += tw;
    }
  }
  lds_sync();
  // background logits of the block's clusters: log2 of the unselected weight
  // (relative to the cluster max) plus the max
  float* sbg = reinterpret_cast<float*>(hist);
  for (int i = tid; i < ncl * G; i += NT) {
    const int cl = c0 + i / G, g = i % G;
    const float M = binl[((cl - c0) * G + g) * 2];
    const float wb = binl[((cl - c0) * G + g) * 2 + 1] - (float)wsel[i] * kFixInv;
    sbg[i] = (wb > 0.0f && M != -INFINITY) ? M + log2f(wb) : -INFINITY;
  }
  // Exact rows and background clusters in 16-row tiles (the row-tile MFMAs of
  // the dense and staged steps): the exact rows of a phase are staged as
  // cache offsets in LDS, up to kStage at a time; the phase's tiles are its
  // exact-row tiles followed, in the last phase, by the background tiles,
  // whose rows are clusters with a given logit per query head and the
  // cluster mean as value.  Wave w takes tiles w, w + NW, ... with the next
  // tile's loads in flight.  Every tile issues the same 8 loads per lane
  // (rows past the end load a valid row with weight zero), so that the waits
  // on them are exact.
  RowTileState st;
  tile_init(st);
  const int nbg = d.exact_only ? 0 : ncl;
  const int nbt = (nbg + 15) / 16;
  const int32_t* tab = a.table + (size_t)b * d.max_pages;
  const float* means = a.ix.means + ((size_t)bh * d.L + c0) * kD;
  // staged offsets: at the top of the LUT region on the direct path, else
  // after the background logits in the histogram region
  long long* ioff = direct ? ioffd : reinterpret_cast<long long*>(dyn + C::kUBytes + 4096);
  const int n_ph = max(1, (nr + kStage - 1) / kStage);
  for (int phi = 0; phi < n_ph; ++phi) {
    const int ph = phi * kStage;
    const int n = max(0, min(kStage, nr - ph));
    __syncthreads();
    {
      // a thread's rows, then their pages, each round of loads issued at once
      int pr[kPerT], pg[kPerT];
#pragma unroll
      for (int i = 0; i < kPerT; ++i) {
        const int t = tid + i * NT;
        int p = -1;
        if (t < n) p = direct ? (kp[i] >= 0 ? kp[i] : posd[t]) : frows[lo + ph + t];
        pr[i] = t < n ? min(max(p, 0), d.cap - 1) : -1;
      }
#pragma unroll
      for (int i = 0; i < kPerT; ++i) pg[i] = pr[i] >= 0 ? tab[pr[i] >> 4] : 0;
#pragma unroll
      for (int i = 0; i < kPerT; ++i) {
        const int t = tid + i * NT;
        if (t < n) {
          const int page = min(max(pg[i], 0), d.num_pages - 1);
          ioff[t] = ((long long)(page * kPage + (pr[i] & (kPage - 1))) * d.Hkv + h) * kD;
        }
      }
    }
    lds_sync();
    const int net = (n + 15) / 16;
    const int ntl = net + (phi == n_ph - 1 ? nbt : 0);
    // exact tile: K[row col] 64 B at 32j in bf[0..3], V[row 4j + i] 16 B at
    // 8 col in bf[4 + i]; background tile: the means of clusters 4j + i, 32 B
    // at 8 col, in bf[2i], bf[2i + 1]
    auto load_tile = [&](int t, uint4 (&bf)[8]) {
      if (t < net) {
        const uint16_t* kr = a.kc + ioff[min(16 * t + tcol, n - 1)] + 32 * tj;
#pragma unroll
        for (int c = 0; c < 4; ++c) bf[c] = *reinterpret_cast<const uint4*>(kr + 8 * c);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          bf[4 + i] = *reinterpret_cast<const uint4*>(
              a.vc + ioff[min(16 * t + 4 * tj + i, n - 1)] + 8 * tcol);
      } else {
        const int cb = 16 * (t - net) + 4 * tj;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float* mu = means + (size_t)min(cb + i, nbg - 1) * kD + 8 * tcol;
          bf[2 * i] = *reinterpret_cast<const uint4*>(mu);
          bf[2 * i + 1] = *reinterpret_cast<const uint4*>(mu + 4);
        }
      }
    };
    uint4 bf[2][8];
    int t = wave;
    if (t < ntl) load_tile(t, bf[0]);
    auto step = [&](uint4 (&cur)[8], uint4 (&nxt)[8]) {
      if (t + NW < ntl) load_tile(t + NW, nxt);
      float sv[4];
      if (t < net) {
        const f32x4 lg = tile_logits(qb, *reinterpret_cast<const uint4(*)[4]>(&cur[0]),
                                     d.scale_log2);
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[i] = 16 * t + 4 * tj + i < n ? lg[i] : -INFINITY;
        tile_accumulate(st, sv, *reinterpret_cast<const uint4(*)[4]>(&cur[4]));
      } else {
        const int cb = 16 * (t - net) + 4 * tj;
        float v[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sv[i] = (cb + i < nbg && tcol < G) ? sbg[(cb + i) * G + min(tcol, G - 1)] : -INFINITY;
          const uint4 m0 = cur[2 * i], m1 = cur[2 * i + 1];
          v[i][0] = __uint_as_float(m0.x); v[i][1] = __uint_as_float(m0.y);
          v[i][2] = __uint_as_float(m0.z); v[i][3] = __uint_as_float(m0.w);
          v[i][4] = __uint_as_float(m1.x); v[i][5] = __uint_as_float(m1.y);
          v[i][6] = __uint_as_float(m1.z); v[i][7] = __uint_as_float(m1.w);
        }
        tile_accumulate_f32(st, sv, v);
      }
      t += NW;
    };
    while (t < ntl) {
      step(bf[0], bf[1]);
      if (t >= ntl) break;
      step(bf[1], bf[0]);
    }
  }
  tile_finish(st);
  __syncthreads();
  // Block merge: the waves' states go to LDS; each thread then forms one
  // output (head, dim) over the NW waves.
  constexpr int kAS = kD + 4;   // padded row of a wave's accumulator
  static_assert((size_t)NW * G * (kAS + 2) * sizeof(float) <= C::kUBytes, "wave states");
  float* accw = reinterpret_cast<float*>(dyn);   // [NW][G][kAS]
  float* mlw = accw + NW * G * kAS;              // [NW][G][2]
  if (tcol < G) {
    float* row = accw + (wave * G + tcol) * kAS + 32 * tj;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<float4*>(row + 8 * i) =
          make_float4(st.acc[0][i], st.acc[1][i], st.acc[2][i], st.acc[3][i]);
      *reinterpret_cast<float4*>(row + 8 * i + 4) =
          make_float4(st.acc[4][i], st.acc[5][i], st.acc[6][i], st.acc[7][i]);
    }
    if (tj == 0) {
      mlw[(wave * G + tcol) * 2] = st.m;
      mlw[(wave * G + tcol) * 2 + 1] = st.l;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * kD; idx += NT) {
    const int g = idx / kD, dim = idx % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, mlw[(w * G + g) * 2]);
    float L = 0.0f, A = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float m = mlw[(w * G + g) * 2];
      const float f = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - M);
      L = fmaf(f, mlw[(w * G + g) * 2 + 1], L);
      A = fmaf(f, accw[(w * G + g) * kAS + dim], A);
    }
    if constexpr (kTagged) {
      unsigned long long* out = hpart + ((size_t)g * kMaxFusedP + sub) * kPart;
      const unsigned long long tag = (unsigned long long)(S.tout ? 2u : 1u) << 32;
      st_dev(&out[4 + dim], tag | __float_as_uint(A));
      if (dim == 0) {
        st_dev(&out[0], tag | __float_as_uint(M));
        st_dev(&out[1], tag | __float_as_uint(L));
      }
    } else {
      float* out = hpartf + ((size_t)g * kMaxFusedP + sub) * kPart;
      st_dev(&out[4 + dim], A);
      if (dim == 0) {
        st_dev(&out[0], M);
        st_dev(&out[1], L);
      }
    }
  }

  if constexpr (kTagged) {
    // ======================================================= mergers
    // Query head g of the head is merged by block g mod P once all P partials
    // of g carry this step's tag; a block merges all of its query heads in one
    // round.  The lanes of wave 0 poll the (m, l) words of one partial each
    // (lane gi * P + j: partial j of the block's query head gi) and form the
    // partials' weights against each head's max; then every thread loads one
    // output dim of every kq-th partial of one head (loading again any word
    // still unwritten) and the kq sums meet in LDS.  A merger waits at most
    // as long as a barrier wait may; if that runs out it sets the flags.  A
    // timeout there or a partial tagged 2 makes the head's outputs NaN (its
    // partials may rest on an incomplete histogram or incomplete records).
    // No block waits for the mergers, and no counter orders them.
    const int ng = sub < G ? (G - 1 - sub) / P + 1 : 0;   // query heads sub, sub + P, ...
    if (sub == 0) {
      // every block is past both barriers' arrivals and has read the
      // histogram and the first counter; the second is cleared at the end
      // (a block may still be polling it)
      for (int i = tid; i < kHistBins; i += NT) st_dev(&ghist[i], 0u);
      if (tid == 0) st_dev(&sync[0], 0u);
    }
    if (ng > 0) {
      // ng * P <= 64: one head when P >= G, else P < G <= 8 and ng * P < 2G
      constexpr int kPerQ = kMaxFusedP / (NT / kD);    // words per thread and head
      static_assert(kMaxFusedP <= 64 && NT % kD == 0, "merger layout");
      const int kq = max(1, NT / (ng * kD));            // threads per output
      float* fpw = reinterpret_cast<float*>(hist);      // [ng * P] partial weights
      float* hml = fpw + 64;                            // [8][2] heads' max and sum
      float* red = hml + 16;                            // [ng][kq][kD] partial sums
      auto part_of = [&](int gi, int j) {
        return hpart + ((size_t)(sub + gi * P) * kMaxFusedP + j) * kPart;
      };
      __syncthreads();
      if (tid < 64) {
        const int gi = tid / P, j = tid % P;
        const bool mine = gi < ng;
        float m = -INFINITY, l = 0.0f;
        int bad = 0;
        if (mine) {
          const unsigned long long* pp = part_of(gi, j);
          const unsigned long long t0 = wall_clock64();
          unsigned long long wm, wl;
          for (;;) {
            wm = ld_dev(&pp[0]);
            wl = ld_dev(&pp[1]);
            if ((wm >> 32) != 0ull && (wl >> 32) != 0ull) break;
            if (wall_clock64() - t0 > d.fbar_ticks) { bad = 1; break; }
            __builtin_amdgcn_s_sleep(2);
          }
          if (!bad) {
            m = __uint_as_float((uint32_t)wm);
            l = __uint_as_float((uint32_t)wl);
            bad = ((wm >> 32) | (wl >> 32)) == 2ull ? 2 : 0;
          }
        }
        float myM = -INFINITY;
        for (int q = 0; q < ng; ++q) {
          const float Mq = wave_max_dpp(gi == q ? m : -INFINITY);
          if (gi == q) myM = Mq;
          if (tid == 0) hml[2 * q] = Mq;
        }
        const float f = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - myM);
        for (int q = 0; q < ng; ++q) {
          const float Lq = wave_sum_dpp(gi == q ? f * l : 0.0f);
          if (tid == 0) hml[2 * q + 1] = Lq;
        }
        if (mine) fpw[tid] = f;
        const uint64_t any_late = __ballot(bad == 1), any_tag2 = __ballot(bad == 2);
        if (tid == 0) S.res[2] = (any_late ? 1 : 0) | (any_tag2 ? 2 : 0);
        if (tid == 0) S.res[3] = 0;
      }
      __syncthreads();
      int bad = 0;
      for (int it = tid; it < ng * kq * kD; it += NT) {
        const int dim = it % kD, q = (it / kD) % kq, gi = it / (kD * kq);
        const unsigned long long* pp = part_of(gi, 0) + 4 + dim;
        unsigned long long w[kPerQ];
#pragma unroll
        for (int u = 0; u < kPerQ; ++u) {
          const int j = q + u * kq;
          w[u] = j < P ? ld_dev(&pp[(size_t)j * kPart]) : (1ull << 32);
        }
        const unsigned long long t0 = wall_clock64();
        float A = 0.0f;
#pragma unroll
        for (int u = 0; u < kPerQ; ++u) {
          const int j = q + u * kq;
          while ((w[u] >> 32) == 0ull && !(bad & 1)) {
            if (wall_clock64() - t0 > d.fbar_ticks) bad |= 1;
            __builtin_amdgcn_s_sleep(2);
            w[u] = ld_dev(&pp[(size_t)j * kPart]);
          }
          if ((w[u] >> 32) == 2ull) bad |= 2;
          if (j < P) A = fmaf(fpw[gi * P + j], __uint_as_float((uint32_t)w[u]), A);
        }
        red[it] = A;
      }
      if (bad) atomicOr(&S.res[3], bad);
      __syncthreads();
      const int flags = S.res[2] | S.res[3];
      if ((flags & 1) && tid == 0)
        __hip_atomic_fetch_or(a.ws.fflags, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int o = tid; o < ng * kD; o += NT) {
        const int gi = o / kD, dim = o % kD;
        float Asum = 0.0f;
        for (int q = 0; q < kq; ++q) Asum += red[(gi * kq + q) * kD + dim];
        const float M = hml[2 * gi], L = hml[2 * gi + 1];
        const size_t bq = (size_t)b * d.Hq + h * G + sub + gi * P;
        // no rows at all: O = 0, lse = -inf; a NaN sum stays NaN
        float ov = L != 0.0f ? Asum / L : 0.0f;
        float ls = L != 0.0f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
        if (flags) ov = ls = __builtin_nanf("");
        a.out[bq * kD + dim] = ov;
        if (dim == 0 && a.lse) a.lse[bq] = ls;
      }
    }
    if (sub != 0) return;
    // Block 0 has seen every block's partial of query head 0, so every
    // block is past both barriers and has read the head's histogram
    // and counts.
  } else {
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
    // (m, l) pairs and forms the weights of the partials against the head's max.
    // A head one of whose barrier waits ran out gets NaN instead: its partials
    // may be built on an incomplete histogram or incomplete records.
    const bool timed_out = ld_dev(hflag) != 0u;
    {
      float* fp = reinterpret_cast<float*>(hist);     // [G][64] weights
      float* mlh = fp + G * kMaxFusedP;               // [G][2] head max and sum
      constexpr int kOut = (G * kD + NT - 1) / NT;    // outputs per thread
      const float* pbase = hpartf;
      float x[kMaxFusedP];
      auto load_col = [&](int o) {
        // threads past the outputs load a valid column and discard it
        const int idx = min(tid + o * NT, G * kD - 1);
        const float* col = pbase + (size_t)(idx / kD) * kMaxFusedP * kPart + 4 + idx % kD;
#pragma unroll
        for (int j = 0; j < kMaxFusedP; ++j) x[j] = j < P ? ld_dev(&col[(size_t)j * kPart]) : 0.0f;
      };
      // wave g loads the (m, l) pairs of query head g, then every thread its
      // column, and then the head's histogram and counters are cleared (every
      // block is past both barriers and done with them): the clears are
      // issued after the loads, so waiting for the loads never waits for them
      static_assert(G <= NW && kOut == 1, "one wave per head, one output per thread");
      float m = -INFINITY, l = 0.0f;
      if (wave < G && lane < P) {
        const float* pp = pbase + ((size_t)wave * kMaxFusedP + lane) * kPart;
        m = ld_dev(&pp[0]);
        l = ld_dev(&pp[1]);
      }
      load_col(0);
      for (int i = tid; i < kHistBins; i += NT) st_dev(&ghist[i], 0u);
      if (tid == 0) {
        st_dev(&sync[0], 0u);
        st_dev(&sync[kSyncStride], 0u);
        st_dev(&sync[2 * kSyncStride], 0u);
      }
      if (wave < G) {
        const float M = wave_max_dpp(m);
        const float f = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - M);
        fp[wave * kMaxFusedP + lane] = f;
        const float L = wave_sum_dpp(f * l);
        if (lane == 0) { mlh[wave * 2] = M; mlh[wave * 2 + 1] = L; }
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
          // no rows at all: O = 0, lse = -inf; a NaN sum stays NaN
          float o = L != 0.0f ? A / L : 0.0f;
          float ls = L != 0.0f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
          if (timed_out) o = ls = __builtin_nanf("");
          a.out[bq * kD + dim] = o;
          if (dim == 0 && a.lse) a.lse[bq] = ls;
        }
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
  if (tid == 0) {
    a.ws.n_rows[bh] = R;
    // the histogram and the other counters were cleared above
    st_dev(&sync[kSyncStride], 0u);
    st_dev(&sync[2 * kSyncStride], 0u);
    st_dev(hflag, 0u);
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
