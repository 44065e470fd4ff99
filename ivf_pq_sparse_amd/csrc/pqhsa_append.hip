// Appending new tokens to an uploaded index.
//
// PQ-HSA page (rit.work blog), section "How approximate estimates return the
// discarded context", sixth paragraph: the index is built after the prompt,
// newer tokens stay outside it and are added in batches; section "Too early
// to change the architecture, a prototype can be built" lists the cost of
// updating the index among the things to measure.  The encoder is the IVF-PQ
// residual encoder matching the decode step's key model
// k_hat = C[list] + concat_m B_m[code_m]:
//   list = argmin_c ||K_t - C_c||^2, code_m = argmin_j ||r^(m) - B_m[j]||^2,
//   r = K_t - C[list], lowest index on equal distances, fp32 arithmetic.
//
//   k_append_encode  one block per (b, h, 16 new tokens): keys from the paged
//                    cache into LDS; every thread scans its share of the
//                    centroids for all 16 keys, a block reduction picks each
//                    key's list; then thread (key, subspace) scans the 256
//                    codewords of its subspace from an LDS copy of the
//                    codebook.  Writes the token-order list ids and codes.
//   regroup          new cluster offsets from the new tokens' counts; old
//                    entries move (from a snapshot) by the number of new
//                    entries in clusters before theirs; new tokens are placed
//                    after their cluster's old entries, in token order.
//   k_append_means   one wave per cluster: the cluster's new entries are the
//                    last ones of its range (the sort keeps token order), so
//                    mu' = (n_old mu + sum of their V) / n_new.
#include "pqhsa_internal.hpp"

namespace pqhsa {

namespace {

constexpr int kEncTokens = 16;     // new tokens per encode block
constexpr int kEncThreads = 256;   // = kEncTokens * kM
// codebook rows padded by 4 floats per subspace so that the 16 subspaces read
// by one wave fall on different LDS banks
constexpr int kCbStride = kKsub * kDsub + 4;

struct EncodeLds {
  float key[kEncTokens][kD];          // keys, then residuals
  float best_d[4][kEncTokens];        // per-wave best distance and centroid
  int best_c[4][kEncTokens];
  int list[kEncTokens];
};

__device__ __forceinline__ void better(float& d, int& c, float d2, int c2) {
  if (d2 < d || (d2 == d && c2 < c)) { d = d2; c = c2; }
}

}  // namespace

__global__ __launch_bounds__(kEncThreads) void k_append_encode(AppendArgs a) {
  extern __shared__ float cb[];        // [16][kCbStride]
  __shared__ EncodeLds sh;
  const Dims& d = a.d;
  const int bh = blockIdx.x;
  const int b = bh / d.Hkv, h = bh % d.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int old_n = min(max(a.ix.n_indexed[b], 0), d.cap);
  const int new_n = min(max(a.new_n_indexed[b], 0), d.cap);
  const int t0 = old_n + blockIdx.y * kEncTokens;
  const int nt = min(kEncTokens, new_n - t0);
  if (nt <= 0) return;
  // keys of the block's tokens (bf16 -> fp32), 8 dims per thread
  const int32_t* tab = a.table + (size_t)b * d.max_pages;
  for (int i = tid; i < kEncTokens * (kD / 8); i += kEncThreads) {
    const int tk = i / (kD / 8), part = i % (kD / 8);
    float f[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (tk < nt) {
      const int t = t0 + tk;
      int page = tab[t >> 4];
      page = min(max(page, 0), d.num_pages - 1);
      const uint4 w = *reinterpret_cast<const uint4*>(
          a.kc + ((size_t)(page * kPage + (t & (kPage - 1))) * d.Hkv + h) * kD + part * 8);
      f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
      f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) sh.key[tk][part * 8 + u] = f[u];
  }
  // the codebook of this (b, h) into LDS (used after the assignment)
  const float* cbg = a.ix.codebooks + (size_t)bh * kM * kKsub * kDsub;
  for (int i = tid; i < kM * kKsub * kDsub / 4; i += kEncThreads) {
    const int m = i / (kKsub * kDsub / 4), r = i % (kKsub * kDsub / 4);
    *reinterpret_cast<float4*>(cb + m * kCbStride + r * 4) =
        reinterpret_cast<const float4*>(cbg)[i];
  }
  __syncthreads();
  // assignment: thread scans centroids tid, tid + 256, ... in ascending order
  float bd[kEncTokens];
  int bc[kEncTokens];
#pragma unroll
  for (int k = 0; k < kEncTokens; ++k) { bd[k] = INFINITY; bc[k] = 0x7fffffff; }
  const float* cen = a.ix.centroids + (size_t)bh * d.L * kD;
  for (int c = tid; c < d.L; c += kEncThreads) {
    float acc[kEncTokens];
#pragma unroll
    for (int k = 0; k < kEncTokens; ++k) acc[k] = 0.0f;
    const float4* cp = reinterpret_cast<const float4*>(cen + (size_t)c * kD);
    for (int q4 = 0; q4 < kD / 4; ++q4) {
      const float4 cv = cp[q4];
#pragma unroll
      for (int k = 0; k < kEncTokens; ++k) {
        const float4 kv = *reinterpret_cast<const float4*>(&sh.key[k][q4 * 4]);
        const float d0 = kv.x - cv.x, d1 = kv.y - cv.y, d2 = kv.z - cv.z, d3 = kv.w - cv.w;
        acc[k] = fmaf(d0, d0, acc[k]);
        acc[k] = fmaf(d1, d1, acc[k]);
        acc[k] = fmaf(d2, d2, acc[k]);
        acc[k] = fmaf(d3, d3, acc[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < kEncTokens; ++k) better(bd[k], bc[k], acc[k], c);
  }
  // block argmin per token: wave butterfly, then the 4 waves
#pragma unroll
  for (int k = 0; k < kEncTokens; ++k) {
    float dv = bd[k];
    int cv = bc[k];
    for (int o = 32; o >= 1; o >>= 1) {
      const float d2 = __shfl_xor(dv, o);
      const int c2 = __shfl_xor(cv, o);
      better(dv, cv, d2, c2);
    }
    if (lane == 0) { sh.best_d[wave][k] = dv; sh.best_c[wave][k] = cv; }
  }
  __syncthreads();
  if (tid < kEncTokens) {
    float dv = sh.best_d[0][tid];
    int cv = sh.best_c[0][tid];
    for (int w = 1; w < 4; ++w) better(dv, cv, sh.best_d[w][tid], sh.best_c[w][tid]);
    sh.list[tid] = min(max(cv, 0), d.L - 1);
  }
  __syncthreads();
  // residuals in place
  for (int i = tid; i < kEncTokens * kD; i += kEncThreads) {
    const int tk = i / kD, dim = i % kD;
    sh.key[tk][dim] -= cen[(size_t)sh.list[tk] * kD + dim];
  }
  __syncthreads();
  // PQ codes: thread (token, subspace) scans the 256 codewords in order
  const int tk = tid / kM, m = tid % kM;
  const float4 r0 = *reinterpret_cast<const float4*>(&sh.key[tk][m * kDsub]);
  const float4 r1 = *reinterpret_cast<const float4*>(&sh.key[tk][m * kDsub + 4]);
  float best = INFINITY;
  int code = 0;
  const float* cbm = cb + m * kCbStride;
  for (int j = 0; j < kKsub; ++j) {
    const float4 w0 = *reinterpret_cast<const float4*>(cbm + j * kDsub);
    const float4 w1 = *reinterpret_cast<const float4*>(cbm + j * kDsub + 4);
    float e = r0.x - w0.x, acc = e * e;
    e = r0.y - w0.y; acc = fmaf(e, e, acc);
    e = r0.z - w0.z; acc = fmaf(e, e, acc);
    e = r0.w - w0.w; acc = fmaf(e, e, acc);
    e = r1.x - w1.x; acc = fmaf(e, e, acc);
    e = r1.y - w1.y; acc = fmaf(e, e, acc);
    e = r1.z - w1.z; acc = fmaf(e, e, acc);
    e = r1.w - w1.w; acc = fmaf(e, e, acc);
    if (acc < best) { best = acc; code = j; }
  }
  if (tk < nt) {
    const int t = t0 + tk;
    a.codes[((size_t)bh * d.cap + t) * kM + m] = (uint8_t)code;
    if (m == 0) a.list_ids[(size_t)bh * d.cap + t] = sh.list[tk];
  }
}

// One wave per cluster: fold the cluster's new entries (the last
// n_new - n_old of its range) into its mean.
__global__ __launch_bounds__(256) void k_append_means(AppendArgs a) {
  __shared__ float red[4][4][kD];
  const Dims& d = a.d;
  const int bh = blockIdx.x;
  const int b = bh / d.Hkv, h = bh % d.Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = lane >> 4, l16 = lane & 15;
  const int c = blockIdx.y * 4 + wave;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int n_old = 0, n_new = 0;
  if (c < d.L) {
    const int32_t* off = a.ix.list_off + (size_t)bh * (d.L + 1);
    const int32_t* oo = a.old_off + (size_t)bh * (d.L + 1);
    const int e1 = off[c + 1];
    n_new = e1 - off[c];
    n_old = oo[c + 1] - oo[c];
    const int32_t* pos = a.ix.pos + (size_t)bh * d.cap;
    const int32_t* tab = a.table + (size_t)b * d.max_pages;
    for (int e = e1 - (n_new - n_old) + row; e < e1; e += 4) {
      const int p = pos[e];
      int page = tab[p / kPage];
      page = min(max(page, 0), d.num_pages - 1);
      const uint4 w = *reinterpret_cast<const uint4*>(
          a.vc + ((size_t)(page * kPage + p % kPage) * d.Hkv + h) * kD + l16 * 8);
      acc[0] += bf16_lo(w.x); acc[1] += bf16_hi(w.x);
      acc[2] += bf16_lo(w.y); acc[3] += bf16_hi(w.y);
      acc[4] += bf16_lo(w.z); acc[5] += bf16_hi(w.z);
      acc[6] += bf16_lo(w.w); acc[7] += bf16_hi(w.w);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[wave][row][l16 * 8 + i] = acc[i];
  __syncthreads();
  if (c < d.L && n_new > n_old) {
    float* mu = a.ix.means + ((size_t)bh * d.L + c) * kD;
    const float inv = 1.0f / (float)n_new;
    for (int i = lane; i < kD; i += 64) {
      const float s = ((red[wave][0][i] + red[wave][1][i]) + red[wave][2][i]) + red[wave][3][i];
      mu[i] = fmaf((float)n_old, mu[i], s) * inv;
    }
  }
}

// Incremental regroup.  Per (b, h): count the new tokens per cluster, new
// offsets off'[c] = off[c] + (new tokens in clusters < c); old entries move
// from a snapshot of the index arrays to off'[c] + (their index within c);
// new tokens go after them in token order.
__global__ __launch_bounds__(1024) void k_append_offsets(AppendArgs a) {
  extern __shared__ int32_t cnt[];     // [L] new tokens per cluster
  __shared__ int wsum[16];
  const Dims& d = a.d;
  const int bh = blockIdx.x;
  const int b = bh / d.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  for (int c = tid; c < d.L; c += blockDim.x) cnt[c] = 0;
  __syncthreads();
  const int old_n = min(max(a.ix.n_indexed[b], 0), d.cap);
  const int new_n = min(max(a.new_n_indexed[b], 0), d.cap);
  const int32_t* lists = a.list_ids + (size_t)bh * d.cap;
  for (int t = old_n + tid; t < new_n; t += blockDim.x) {
    const int c = lists[t];
    if (c >= 0 && c < d.L) atomicAdd(&cnt[c], 1);
  }
  __syncthreads();
  // exclusive prefix over clusters: each thread owns a run of them
  const int per = (d.L + blockDim.x - 1) / blockDim.x;
  const int c0 = min(d.L, tid * per), c1 = min(d.L, c0 + per);
  int mine = 0;
  for (int c = c0; c < c1; ++c) mine += cnt[c];
  const int incl = wave_incl_scan(mine);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = incl - mine;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  int32_t* off = a.ix.list_off + (size_t)bh * (d.L + 1);
  const int32_t* oo = a.old_off + (size_t)bh * (d.L + 1);
  int32_t* shift = a.shift + (size_t)bh * (d.L + 1);
  for (int c = c0; c < c1; ++c) {
    shift[c] = before;
    off[c] = oo[c] + before;
    before += cnt[c];
  }
  if (tid == blockDim.x - 1) {
    int tot = 0;
    for (int w = 0; w < nw; ++w) tot += wsum[w];
    off[d.L] = oo[d.L] + tot;
    shift[d.L] = tot;
  }
}

// One thread per old entry: move codes, position and cluster to the new slot.
__global__ __launch_bounds__(256) void k_append_move(AppendArgs a) {
  const Dims& d = a.d;
  const int bh = blockIdx.y;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  const int32_t* oo = a.old_off + (size_t)bh * (d.L + 1);
  if (e >= min(oo[d.L], d.cap)) return;
  const size_t base = (size_t)bh * d.cap;
  const int c = min(max(a.snap_list[base + e], 0), d.L - 1);
  const int dst = e + a.shift[(size_t)bh * (d.L + 1) + c];
  if (dst < 0 || dst >= d.cap) return;
  reinterpret_cast<uint4*>(a.ix.codes)[base + dst] = reinterpret_cast<const uint4*>(a.snap_codes)[base + e];
  a.ix.pos[base + dst] = a.snap_pos[base + e];
  a.ix.ent_list[base + dst] = c;
}

// One wave per (b, h): the new tokens in token order, each after the old
// entries of its cluster and the earlier new ones (rank inside a 64-token
// tile by comparing list ids, running counts per cluster in LDS).
__global__ __launch_bounds__(64) void k_append_place(AppendArgs a) {
  extern __shared__ int32_t run[];     // [L] new tokens placed so far per cluster
  __shared__ int32_t tile[64];
  const Dims& d = a.d;
  const int bh = blockIdx.x;
  const int b = bh / d.Hkv;
  const int lane = threadIdx.x;
  for (int c = lane; c < d.L; c += 64) run[c] = 0;
  const int old_n = min(max(a.ix.n_indexed[b], 0), d.cap);
  const int new_n = min(max(a.new_n_indexed[b], 0), d.cap);
  const size_t base = (size_t)bh * d.cap;
  const int32_t* off = a.ix.list_off + (size_t)bh * (d.L + 1);
  const int32_t* oo = a.old_off + (size_t)bh * (d.L + 1);
  __syncthreads();
  for (int s = old_n; s < new_n; s += 64) {
    const int t = s + lane;
    int c = -1;
    if (t < new_n) {
      c = a.list_ids[base + t];
      if (c < 0 || c >= d.L) c = -1;
    }
    tile[lane] = c;
    __syncthreads();
    int rank = 0, same = 0;
    for (int j = 0; j < 64; ++j) {
      const int cj = tile[j];
      same += (cj == c);
      rank += (cj == c) & (j < lane);
    }
    if (c >= 0) {
      const int dst = off[c] + (oo[c + 1] - oo[c]) + run[c] + rank;
      if (dst >= 0 && dst < d.cap) {
        reinterpret_cast<uint4*>(a.ix.codes)[base + dst] =
            reinterpret_cast<const uint4*>(a.codes)[base + t];
        a.ix.pos[base + dst] = t;
        a.ix.ent_list[base + dst] = c;
      }
    }
    __syncthreads();
    if (c >= 0 && rank == same - 1) run[c] += same;
    __syncthreads();
  }
}

hipError_t launch_append_regroup(const AppendArgs& a, hipStream_t st) {
  const Dims& d = a.d;
  const int BH = d.B * d.Hkv;
  hipLaunchKernelGGL(k_append_offsets, dim3(BH), dim3(1024), d.L * sizeof(int32_t), st, a);
  hipLaunchKernelGGL(k_append_move, dim3((d.cap + 255) / 256, BH), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_append_place, dim3(BH), dim3(64), d.L * sizeof(int32_t), st, a);
  return hipGetLastError();
}

hipError_t launch_append_encode(const AppendArgs& a, int max_new, hipStream_t st) {
  const int BH = a.d.B * a.d.Hkv;
  const int tiles = (max_new + kEncTokens - 1) / kEncTokens;
  if (tiles == 0) return hipSuccess;
  const size_t lds = (size_t)kM * kCbStride * sizeof(float);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_append_encode),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_append_encode, dim3(BH, tiles), dim3(kEncThreads), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_append_means(const AppendArgs& a, hipStream_t st) {
  const int BH = a.d.B * a.d.Hkv;
  hipLaunchKernelGGL(k_append_means, dim3(BH, (a.d.L + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace pqhsa
