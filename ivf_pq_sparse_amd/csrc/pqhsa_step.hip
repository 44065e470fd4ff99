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
#include "pqhsa_internal.hpp"

namespace pqhsa {

// ---------------------------------------------------------------- tables
// grid (B*Hkv, 16 + ceil(L/64)), 256 threads.
//   y < 16 : lut[m = y][j = thread][g] = scale*log2e * q_g^(m) . B_m[j]
//   y >= 16: qc[c][g] = scale*log2e * q_g . C_c for 64 clusters, one wave per 16
// Every block also clears its share of the step's counters and bitmaps.
template <int G>
__global__ __launch_bounds__(256) void k_tables(StepArgs a) {
  const Dims& d = a.d;
  const int bh = blockIdx.x;
  const int b = bh / d.Hkv, h = bh % d.Hkv;
  const uint16_t* q = a.q + ((size_t)b * d.Hq + h * G) * kD;
  {
    // clear hist, candidate counter and both bitmaps of this (b, h)
    const int nb = gridDim.y;
    const int words = kHistBins + 1 + 2 * d.nwords;
    for (int i = blockIdx.y * blockDim.x + threadIdx.x; i < words; i += nb * blockDim.x) {
      if (i < kHistBins) a.ws.hist[(size_t)bh * kHistBins + i] = 0;
      else if (i == kHistBins) a.ws.cand_count[bh] = 0;
      else if (i < kHistBins + 1 + d.nwords) a.ws.sel_p[(size_t)bh * d.nwords + (i - kHistBins - 1)] = 0;
      else a.ws.sel_e[(size_t)bh * d.nwords + (i - kHistBins - 1 - d.nwords)] = 0;
    }
  }
  if (blockIdx.y < kM) {
    const int m = blockIdx.y;
    const int j = threadIdx.x;
    float qs[G][kDsub];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < kDsub; ++i) qs[g][i] = bf16_to_f32(q[g * kD + m * kDsub + i]) * d.scale_log2;
    const float* cw = a.ix.codebooks + (((size_t)bh * kM + m) * kKsub + j) * kDsub;
    const float4 c0 = *reinterpret_cast<const float4*>(cw);
    const float4 c1 = *reinterpret_cast<const float4*>(cw + 4);
    const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    float* out = a.ws.lut + (((size_t)bh * kM + m) * kKsub + j) * G;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s = qs[g][0] * cv[0];
#pragma unroll
      for (int i = 1; i < kDsub; ++i) s = fmaf(qs[g][i], cv[i], s);
      out[g] = s;
    }
  } else {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    float qv[G][2];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      qv[g][0] = bf16_to_f32(q[g * kD + 2 * lane]) * d.scale_log2;
      qv[g][1] = bf16_to_f32(q[g * kD + 2 * lane + 1]) * d.scale_log2;
    }
    const int cbase = (blockIdx.y - kM) * 64 + wave * 16;
    for (int i = 0; i < 16; ++i) {
      const int c = cbase + i;
      if (c >= d.L) continue;
      const float2 cv = *reinterpret_cast<const float2*>(a.ix.centroids + ((size_t)bh * d.L + c) * kD + 2 * lane);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float s = wave_sum(fmaf(qv[g][1], cv.y, qv[g][0] * cv.x));
        if (lane == 0) a.ws.qc[((size_t)bh * d.L + c) * G + g] = s;
      }
    }
  }
}

// ---------------------------------------------------------------- scan
// grid (B*Hkv*scan_blocks), 1024 threads, LDS = LUT (16*256*G floats) + 4096
// histogram bins.  Each block owns 16 consecutive clusters of one (b, h); a
// wave takes a whole cluster at a time (so the cluster's qc is wave-uniform
// and its bin needs no atomics).  For every entry: approximate base-2 logits
// of the G query heads, key = max over heads written in order-preserving bits
// (0 for non-candidates), one histogram count on the key's top 12 bits, and
// an online (max, sum of exp2) per lane and head over candidates, reduced per
// cluster into bins[c][g] = (max, sum).
template <int G>
__global__ __launch_bounds__(kScanThreads) void k_scan(StepArgs a) {
  extern __shared__ float4 smem4[];
  float* lut = reinterpret_cast<float*>(smem4);
  uint32_t* hist = reinterpret_cast<uint32_t*>(lut + kM * kKsub * G);
  const Dims& d = a.d;
  const int bh = blockIdx.x / d.scan_blocks;
  const int blk = blockIdx.x % d.scan_blocks;
  const int b = bh / d.Hkv;
  {
    const float4* src = reinterpret_cast<const float4*>(a.ws.lut + (size_t)bh * kM * kKsub * G);
    for (int i = threadIdx.x; i < kM * kKsub * G / 4; i += blockDim.x) smem4[i] = src[i];
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) hist[i] = 0;
  }
  __syncthreads();
  const SeqInfo si = seq_info(d, a.ctx, a.ix.n_indexed, b);
  const int lane = threadIdx.x & 63;
  // wave id as a scalar: the cluster loop below is uniform across the wave,
  // so its cross-lane reductions always see every lane
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = kScanThreads / 64;
  const int c0 = blk * kScanListsPerBlock;
  const int nl = min(kScanListsPerBlock, d.L - c0);
  const int32_t* off = a.ix.list_off + (size_t)bh * (d.L + 1);
  const uint4* codes = reinterpret_cast<const uint4*>(a.ix.codes + (size_t)bh * d.cap * kM);
  const int32_t* pos = a.ix.pos + (size_t)bh * d.cap;
  uint32_t* keys = a.ws.keys + (size_t)bh * d.cap;
  for (int li = wave; li < nl; li += nwaves) {
    const int c = c0 + li;
    float qc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) qc[g] = a.ws.qc[((size_t)bh * d.L + c) * G + g];
    const int e1 = min(off[c + 1], d.cap), e0 = min(max(off[c], 0), e1);
    float mx[G], sm[G];
#pragma unroll
    for (int g = 0; g < G; ++g) { mx[g] = -INFINITY; sm[g] = 0.0f; }
    for (int eb = e0; eb < e1; eb += 64) {
      const int e = eb + lane;
      if (e < e1) {
        const uint4 cw = codes[e];
        const int p = pos[e];
        float s[G];
        entry_logits<G>(lut, qc, cw, s);
        float kappa = s[0];
#pragma unroll
        for (int g = 1; g < G; ++g) kappa = fmaxf(kappa, s[g]);
        const bool cand = p >= si.cand_beg && p < si.cand_end;
        uint32_t key = 0;
        if (cand) {
          key = order_key(kappa);
          atomicAdd(&hist[key >> (32 - kHistBits)], 1u);
#pragma unroll
          for (int g = 0; g < G; ++g) {
            // online max/sum of exp2 with one exp2 per value
            const float x = s[g];
            const float dlt = x - mx[g];
            const float ex = exp2f(-fabsf(dlt));
            const bool up = dlt > 0.0f;
            sm[g] = up ? fmaf(sm[g], ex, 1.0f) : sm[g] + ex;
            mx[g] = up ? x : mx[g];
          }
        }
        keys[e] = key;
      }
    }
    // reduce the cluster's (max, sum) over the wave
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float M = wave_max(mx[g]);
      const float part = (mx[g] == -INFINITY) ? 0.0f : sm[g] * exp2f(mx[g] - M);
      const float S = wave_sum(part);
      if (lane == 0) {
        float* bin = a.ws.bins + (((size_t)bh * d.L + c) * G + g) * 2;
        bin[0] = M;
        bin[1] = S;
      }
    }
  }
  __syncthreads();
  uint32_t* gh = a.ws.hist + (size_t)bh * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) {
    const uint32_t v = hist[i];
    if (v) atomicAdd(&gh[i], v);
  }
}

// ---------------------------------------------------------------- threshold bucket
// From the 4096-bin histogram of candidate keys (top 12 bits), find the bucket
// holding the k-th largest key: beta with above(beta) < k <= above(beta) +
// hist[beta], where above(x) counts keys in buckets > x.  Also returns the
// total count.  Uses the whole block; blockDim divides 4096 and is a multiple
// of 64.  sh must hold blockDim/64 + 3 ints.
__device__ void find_threshold(const uint32_t* __restrict__ gh, int k, int* sh, int* beta,
                               int* above, int* total) {
  const int nt = blockDim.x;
  const int per = kHistBins / nt;
  const int t = threadIdx.x;
  // thread t owns bins [hi - per, hi), hi = 4096 - t*per (thread 0 has the top)
  const int hi = kHistBins - t * per;
  int s = 0;
  for (int i = 1; i <= per; ++i) s += (int)gh[hi - i];
  // inclusive scan over threads in order t = 0, 1, ... (top bins first)
  const int lane = t & 63, wave = t >> 6, nw = nt >> 6;
  int x = s;
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  if (t == 0) { sh[nw] = -1; sh[nw + 1] = 0; }
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int w = 0; w < nw; ++w) { int v = sh[w]; sh[w] = run; run += v; }
    sh[nw + 2] = run;
  }
  __syncthreads();
  const int tot = sh[nw + 2];
  const int kk = min(k, tot);
  const int before = sh[wave] + x - s;   // keys in bins above this thread's range
  if (kk > 0 && before < kk && before + s >= kk) {
    int run = before;
    for (int i = 1; i <= per; ++i) {
      const int bin = hi - i;
      const int v = (int)gh[bin];
      if (run + v >= kk) { sh[nw] = bin; sh[nw + 1] = run; break; }
      run += v;
    }
  }
  __syncthreads();
  *beta = sh[nw];
  *above = sh[nw + 1];
  *total = tot;
  __syncthreads();
}

// ---------------------------------------------------------------- collect
// grid (B*Hkv*collect_slices), 256 threads.  Entries whose key bucket is above
// the threshold bucket are selected (bits set in both bitmaps); entries in
// the threshold bucket are appended to the candidate list for the exact pass.
__global__ __launch_bounds__(256) void k_collect(StepArgs a) {
  __shared__ int sh[8];
  const Dims& d = a.d;
  const int bh = blockIdx.x / d.collect_slices;
  const int slice = blockIdx.x % d.collect_slices;
  const int b = bh / d.Hkv;
  const SeqInfo si = seq_info(d, a.ctx, a.ix.n_indexed, b);
  const int n_entries = min(a.ix.list_off[(size_t)bh * (d.L + 1) + d.L], d.cap);
  const int e0 = slice * kCollectEntries;
  if (si.k <= 0 || e0 >= n_entries) return;
  int beta, above, total;
  find_threshold(a.ws.hist + (size_t)bh * kHistBins, si.k, sh, &beta, &above, &total);
  if (beta < 0) return;
  const int e1 = min(n_entries, e0 + kCollectEntries);
  const uint32_t* keys = a.ws.keys + (size_t)bh * d.cap;
  const int32_t* pos = a.ix.pos + (size_t)bh * d.cap;
  uint32_t* sel_p = a.ws.sel_p + (size_t)bh * d.nwords;
  uint32_t* sel_e = a.ws.sel_e + (size_t)bh * d.nwords;
  uint4* cand = a.ws.cand + (size_t)bh * d.cap;
  uint32_t* ccount = a.ws.cand_count + bh;
  for (int eb = e0; eb < e1; eb += blockDim.x) {
    const int e = eb + threadIdx.x;
    uint32_t key = 0;
    if (e < e1) key = keys[e];
    const int bucket = (int)(key >> (32 - kHistBits));
    const bool take = key != 0 && bucket > beta;
    const bool tie = key != 0 && bucket == beta;
    if (take) {
      const int p = pos[e];
      atomicOr(&sel_p[p >> 5], 1u << (p & 31));
      atomicOr(&sel_e[e >> 5], 1u << (e & 31));
    }
    if (tie) {
      const uint32_t idx = atomicAdd(ccount, 1u);
      cand[idx] = make_uint4(key, (uint32_t)pos[e], (uint32_t)e, 0u);
    }
  }
}

// ---------------------------------------------------------------- select
// grid (B*Hkv), 1024 threads.  Resolves the threshold bucket exactly with an
// 8-bit radix select over 52-bit composites (20 low key bits, then the
// bit-inverted position so that equal keys prefer the lower position), marks
// the winners, then compacts the position bitmap into the ascending list of
// exact rows: sink rows, selected rows, recent/tail rows.
__device__ __forceinline__ unsigned long long composite(uint4 c) {
  return ((unsigned long long)c.x << 32) | (unsigned long long)(0xffffffffu - c.y);
}

__device__ __forceinline__ uint32_t load_coherent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(1024) void k_select(StepArgs a) {
  __shared__ int sh[24];
  __shared__ uint32_t rh[256];
  __shared__ int res[3];
  const Dims& d = a.d;
  const int bh = blockIdx.x;
  const int b = bh / d.Hkv, h = bh % d.Hkv;
  const SeqInfo si = seq_info(d, a.ctx, a.ix.n_indexed, b);
  uint32_t* sel_p = a.ws.sel_p + (size_t)bh * d.nwords;
  uint32_t* sel_e = a.ws.sel_e + (size_t)bh * d.nwords;
  int ksel = 0;
  if (si.k > 0) {
    int beta, above, total;
    find_threshold(a.ws.hist + (size_t)bh * kHistBins, si.k, sh, &beta, &above, &total);
    ksel = min(si.k, total);
    const int n_cand = (int)a.ws.cand_count[bh];
    const int r = ksel - above;
    const uint4* cand = a.ws.cand + (size_t)bh * d.cap;
    unsigned long long prefix = 0, mask = 0;
    bool all = r >= n_cand;
    if (!all && r > 0) {
      int need = r;
      for (int shift = 44; ; shift -= 8) {
        const int s = shift > 0 ? shift : 0;
        const unsigned long long dm = shift >= 0 ? 0xffull : 0xfull;
        for (int i = threadIdx.x; i < 256; i += blockDim.x) rh[i] = 0;
        __syncthreads();
        for (int i = threadIdx.x; i < n_cand; i += blockDim.x) {
          const unsigned long long c = composite(cand[i]) & 0x000fffffffffffffull;
          if ((c & mask) == prefix) atomicAdd(&rh[(c >> s) & dm], 1u);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
          int run = 0, dig = 0;
          for (int v = (int)dm; v >= 0; --v) {
            const int n = (int)rh[v];
            if (run + n >= need) { dig = v; res[1] = run; res[2] = n; break; }
            run += n;
          }
          res[0] = dig;
        }
        __syncthreads();
        const int dig = res[0];
        need -= res[1];
        prefix |= (unsigned long long)dig << s;
        mask |= dm << s;
        const bool done = res[2] == need || s == 0;
        __syncthreads();
        if (done) break;
      }
    }
    if (r > 0) {
      for (int i = threadIdx.x; i < n_cand; i += blockDim.x) {
        const uint4 cv = cand[i];
        const unsigned long long c = composite(cv) & 0x000fffffffffffffull;
        if (all || (c & mask) >= prefix) {
          atomicOr(&sel_p[cv.y >> 5], 1u << (cv.y & 31));
          atomicOr(&sel_e[cv.z >> 5], 1u << (cv.z & 31));
        }
      }
    }
    __syncthreads();
  }
  // compaction of the position bitmap into ascending rows
  int32_t* rows = a.ws.rows + (size_t)bh * d.cap;
  for (int i = threadIdx.x; i < si.ns; i += blockDim.x) rows[i] = i;
  const int nw = d.nwords;
  const int per = (nw + blockDim.x - 1) / blockDim.x;
  const int w0 = min(nw, (int)threadIdx.x * per), w1 = min(nw, w0 + per);
  int cnt = 0;
  if (ksel > 0)
    for (int w = w0; w < w1; ++w) cnt += __popc(load_coherent(&sel_p[w]));
  // block exclusive scan of cnt
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwv = blockDim.x >> 6;
  int x = cnt;
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < nwv; ++w) { int v = sh[w]; sh[w] = run; run += v; }
    sh[nwv] = run;
  }
  __syncthreads();
  int at = si.ns + sh[wave] + x - cnt;
  const int nsel = sh[nwv];
  int32_t* selout = a.selected ? a.selected + (size_t)bh * a.max_sel : nullptr;
  if (ksel > 0) {
    for (int w = w0; w < w1; ++w) {
      uint32_t bits = load_coherent(&sel_p[w]);
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
  for (int i = threadIdx.x; i < si.T - rb; i += blockDim.x) rows[base_r + i] = rb + i;
  if (selout)
    for (int i = nsel + threadIdx.x; i < a.max_sel; i += blockDim.x) selout[i] = -1;
  if (threadIdx.x == 0) a.ws.n_rows[bh] = base_r + (si.T - rb);
  (void)h;
}

// ---------------------------------------------------------------- launchers
template <int G>
static hipError_t tables_g(const StepArgs& a, hipStream_t st) {
  const int BH = a.d.B * a.d.Hkv;
  hipLaunchKernelGGL(k_tables<G>, dim3(BH, kM + (a.d.L + 63) / 64), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_tables(const StepArgs& a, hipStream_t st) {
  switch (a.d.G) {
    case 1: return tables_g<1>(a, st);
    case 2: return tables_g<2>(a, st);
    case 4: return tables_g<4>(a, st);
    case 8: return tables_g<8>(a, st);
  }
  return hipErrorInvalidValue;
}

template <int G>
static hipError_t scan_g(const StepArgs& a, hipStream_t st) {
  const int BH = a.d.B * a.d.Hkv;
  const size_t lds = (size_t)kM * kKsub * G * sizeof(float) + kHistBins * sizeof(uint32_t);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_scan<G>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_scan<G>, dim3(BH * a.d.scan_blocks), dim3(kScanThreads), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_scan(const StepArgs& a, hipStream_t st) {
  switch (a.d.G) {
    case 1: return scan_g<1>(a, st);
    case 2: return scan_g<2>(a, st);
    case 4: return scan_g<4>(a, st);
    case 8: return scan_g<8>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_collect(const StepArgs& a, hipStream_t st) {
  const int BH = a.d.B * a.d.Hkv;
  hipLaunchKernelGGL(k_collect, dim3(BH * a.d.collect_slices), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_select(const StepArgs& a, hipStream_t st) {
  const int BH = a.d.B * a.d.Hkv;
  hipLaunchKernelGGL(k_select, dim3(BH), dim3(1024), 0, st, a);
  return hipGetLastError();
}

}  // namespace pqhsa
