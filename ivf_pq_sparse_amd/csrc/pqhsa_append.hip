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
//   k_append_assign  one block per (b, h, 64 new tokens, run of centroid
//                    chunks): keys from the paged cache and 64-centroid chunks
//                    (the next chunk's loads in flight) in padded LDS rows;
//                    each thread owns a 4 token x 4 centroid tile of
//                    distances, a 16-lane reduction picks each key's nearest
//                    centroid of the run.  Small batches split the centroids
//                    over several blocks, whose results meet in a 64-bit
//                    minimum of (distance bits, list) per token.
//   k_append_pq      one wave per (b, h, 64 new tokens, subspace, quarter of
//                    the codewords): the wave stages its 64 codewords in LDS
//                    (one per lane) and each lane scans them, by broadcast
//                    reads, for its token's residual slice; the block's four
//                    quarters are merged in LDS.  Writes the codes and the
//                    list ids.
//   k_append_snapshot the cluster offsets and the held entries' codes,
//                    positions and clusters copied to the workspace first.
//   regroup          new cluster offsets from the new tokens' counts, and the
//                    new tokens placed after their cluster's old entries, in
//                    token order (k_append_place); then the old entries move
//                    (from the snapshot) by the number of new entries in
//                    clusters before theirs (k_append_move).
//   k_append_means   one wave per cluster: the cluster's new entries are the
//                    last ones of its range (the sort keeps token order), so
//                    mu' = (n_old mu + sum of their V) / n_new.
#include <algorithm>

#include "pqhsa_internal.hpp"

namespace pqhsa {

namespace {

constexpr int kEncTokens = 64;     // new tokens per assignment / code block
constexpr int kEncThreads = 256;
constexpr int kAsgCents = 64;      // centroids per LDS chunk of the assignment
// LDS rows of keys and centroids, padded so that 16 consecutive rows read by
// one 16-lane group start 4 banks apart
constexpr int kRowPad = kD + 4;
constexpr int kPqQuarter = kKsub / 4;   // codewords per wave of the code pass

__device__ __forceinline__ void better(float& d, int& c, float d2, int c2) {
  if (d2 < d || (d2 == d && c2 < c)) { d = d2; c = c2; }
}

}  // namespace

__global__ __launch_bounds__(kEncThreads) void k_append_assign(AppendArgs a) {
  extern __shared__ __align__(16) float alds[];
  float* keyl = alds;                          // [64][kRowPad]
  float* cenl = alds + kEncTokens * kRowPad;   // [64][kRowPad]
  const Dims& d = a.d;
  const int bh = blockIdx.x;
  const int b = bh / d.Hkv, h = bh % d.Hkv;
  const int tid = threadIdx.x;
  int old_n, new_n;
  append_span(a, b, &old_n, &new_n);
  const int t0 = old_n + blockIdx.y * kEncTokens;
  const int nt = min(kEncTokens, new_n - t0);
  if (nt <= 0) return;
  // keys of the block's tokens (bf16 -> fp32), 8 dims per thread and pass
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
    float4* dst = reinterpret_cast<float4*>(keyl + tk * kRowPad + part * 8);
    dst[0] = make_float4(f[0], f[1], f[2], f[3]);
    dst[1] = make_float4(f[4], f[5], f[6], f[7]);
  }
  // thread tile: tokens tq*4 + i, centroids c0 + cq + 16 j of each chunk
  const int tq = tid / 16, cq = tid % 16;
  float bd[4];
  int bc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { bd[i] = INFINITY; bc[i] = 0x7fffffff; }
  const float4* cen4 = reinterpret_cast<const float4*>(a.ix.centroids + (size_t)bh * d.L * kD);
  constexpr int kPer = kAsgCents * (kD / 4) / kEncThreads;   // float4 of a chunk per thread
  // this block's centroids [cb0, cb1)
  const int cb0 = blockIdx.z * a.asg_chunks * kAsgCents;
  const int cb1 = min(d.L, cb0 + a.asg_chunks * kAsgCents);
  float4 pre[kPer];
  auto load_chunk = [&](int c0) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int idx = tid + u * kEncThreads, row = idx / (kD / 4), q = idx % (kD / 4);
      pre[u] = c0 + row < cb1 ? cen4[(size_t)(c0 + row) * (kD / 4) + q]
                              : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  load_chunk(cb0);
  const float4* keyl4 = reinterpret_cast<const float4*>(keyl);
  const float4* cenl4 = reinterpret_cast<const float4*>(cenl);
  for (int c0 = cb0; c0 < cb1; c0 += kAsgCents) {
    __syncthreads();   // the previous chunk is no longer read
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int idx = tid + u * kEncThreads, row = idx / (kD / 4), q = idx % (kD / 4);
      reinterpret_cast<float4*>(cenl + row * kRowPad)[q] = pre[u];
    }
    __syncthreads();
    if (c0 + kAsgCents < cb1) load_chunk(c0 + kAsgCents);
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
#pragma unroll 2
    for (int q4 = 0; q4 < kD / 4; ++q4) {
      float4 kv[4], cv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) kv[i] = keyl4[(tq * 4 + i) * (kRowPad / 4) + q4];
#pragma unroll
      for (int j = 0; j < 4; ++j) cv[j] = cenl4[(cq + 16 * j) * (kRowPad / 4) + q4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float e0 = kv[i].x - cv[j].x, e1 = kv[i].y - cv[j].y, e2 = kv[i].z - cv[j].z,
                      e3 = kv[i].w - cv[j].w;
          float x = acc[i][j];
          x = fmaf(e0, e0, x);
          x = fmaf(e1, e1, x);
          x = fmaf(e2, e2, x);
          x = fmaf(e3, e3, x);
          acc[i][j] = x;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = c0 + cq + 16 * j;
        if (c < cb1) better(bd[i], bc[i], acc[i][j], c);
      }
  }
  // each token's best over the 16 lanes of its row
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) {
      const float d2 = __shfl_xor(bd[i], o);
      const int c2 = __shfl_xor(bc[i], o);
      better(bd[i], bc[i], d2, c2);
    }
  }
  if (cq == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tk = tq * 4 + i;
      if (tk < nt) {
        // distances are >= 0, so their bits order like the floats; on equal
        // distances the lower list wins
        const unsigned long long v = ((unsigned long long)__float_as_uint(bd[i]) << 32) |
                                     (uint32_t)min(max(bc[i], 0), d.L - 1);
        unsigned long long* dst = a.best + (size_t)bh * d.cap + t0 + tk;
        if (gridDim.z > 1) atomicMin(dst, v);
        else *dst = v;
      }
    }
  }
}

// Before anything moves: the cluster offsets and, for the entries the index
// holds, their codes, positions and clusters go to the workspace; the new
// tokens' 64-bit minima start above every candidate.  grid (cap/256, BH).
__global__ __launch_bounds__(256) void k_append_snapshot(AppendArgs a) {
  const Dims& d = a.d;
  const int bh = blockIdx.y;
  const int b = bh / d.Hkv;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  const int32_t* off = a.ix.list_off + (size_t)bh * (d.L + 1);
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= d.L; i += blockDim.x) a.old_off[(size_t)bh * (d.L + 1) + i] = off[i];
  const size_t base = (size_t)bh * d.cap;
  if (e < min(max(off[d.L], 0), d.cap)) {
    reinterpret_cast<uint4*>(a.snap_codes)[base + e] =
        reinterpret_cast<const uint4*>(a.ix.codes)[base + e];
    a.snap_pos[base + e] = a.ix.pos[base + e];
    a.snap_list[base + e] = a.ix.ent_list[base + e];
  }
  int old_n, new_n;
  append_span(a, b, &old_n, &new_n);
  if (e >= old_n && e < new_n) a.best[base + e] = ~0ull;
}

__global__ __launch_bounds__(256) void k_append_pq(AppendArgs a) {
  __shared__ float4 cbq[4][kPqQuarter][2];   // each wave's codewords
  __shared__ float qbest[4][64];
  __shared__ int qcode[4][64];
  const Dims& d = a.d;
  const int bh = blockIdx.x;
  const int b = bh / d.Hkv, h = bh % d.Hkv;
  const int lane = threadIdx.x & 63;
  const int quarter = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = blockIdx.z;
  int old_n, new_n;
  append_span(a, b, &old_n, &new_n);
  const int t0 = old_n + blockIdx.y * kEncTokens;
  const int nt = min(kEncTokens, new_n - t0);
  if (nt <= 0) return;
  const int t = t0 + lane;
  const bool ok = lane < nt;
  // this wave's quarter of subspace m's codewords, one per lane, into LDS
  const int j0 = quarter * kPqQuarter;
  {
    const float4* cbg = reinterpret_cast<const float4*>(
        a.ix.codebooks + (((size_t)bh * kM + m) * kKsub + j0 + lane) * kDsub);
    cbq[quarter][lane][0] = cbg[0];
    cbq[quarter][lane][1] = cbg[1];
  }
  // residual slice r^(m) = K_t[m] - C[list_t][m] of this lane's token
  float r[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int list = 0;
  if (ok) {
    list = min(max((int)(uint32_t)a.best[(size_t)bh * d.cap + t], 0), d.L - 1);
    const int32_t* tab = a.table + (size_t)b * d.max_pages;
    int page = tab[t >> 4];
    page = min(max(page, 0), d.num_pages - 1);
    const uint4 w = *reinterpret_cast<const uint4*>(
        a.kc + ((size_t)(page * kPage + (t & (kPage - 1))) * d.Hkv + h) * kD + m * kDsub);
    const float* cen = a.ix.centroids + ((size_t)bh * d.L + list) * kD + m * kDsub;
    const float4 c0v = *reinterpret_cast<const float4*>(cen);
    const float4 c1v = *reinterpret_cast<const float4*>(cen + 4);
    r[0] = bf16_lo(w.x) - c0v.x; r[1] = bf16_hi(w.x) - c0v.y;
    r[2] = bf16_lo(w.y) - c0v.z; r[3] = bf16_hi(w.y) - c0v.w;
    r[4] = bf16_lo(w.z) - c1v.x; r[5] = bf16_hi(w.z) - c1v.y;
    r[6] = bf16_lo(w.w) - c1v.z; r[7] = bf16_hi(w.w) - c1v.w;
  }
  __syncthreads();
  // every lane scans the same codewords (LDS broadcast reads)
  float best = INFINITY;
  int code = j0;
#pragma unroll 2
  for (int j = 0; j < kPqQuarter; j += 4) {
    float4 wv[4][2];   // four codewords read ahead of their use
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      wv[k][0] = cbq[quarter][j + k][0];
      wv[k][1] = cbq[quarter][j + k][1];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float w[8] = {wv[k][0].x, wv[k][0].y, wv[k][0].z, wv[k][0].w,
                          wv[k][1].x, wv[k][1].y, wv[k][1].z, wv[k][1].w};
      float e = r[0] - w[0], acc = e * e;
#pragma unroll
      for (int u = 1; u < kDsub; ++u) {
        e = r[u] - w[u];
        acc = fmaf(e, e, acc);
      }
      if (acc < best) { best = acc; code = j0 + j + k; }
    }
  }
  qbest[quarter][lane] = best;
  qcode[quarter][lane] = code;
  __syncthreads();
  if (quarter == 0 && ok) {
    // quarters in codeword order: a strictly smaller distance wins, so the
    // lowest codeword stays on ties
#pragma unroll
    for (int q = 1; q < 4; ++q)
      if (qbest[q][lane] < best) { best = qbest[q][lane]; code = qcode[q][lane]; }
    a.codes[((size_t)bh * d.cap + t) * kM + m] = (uint8_t)code;
    if (m == 0) a.list_ids[(size_t)bh * d.cap + t] = list;
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
  // the index now covers the new tokens (nothing in this kernel reads it)
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    for (int i = threadIdx.x; i < d.B; i += blockDim.x) {
      int o, n;
      append_span(a, i, &o, &n);
      a.ix.n_indexed[i] = n;
    }
  }
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

// Incremental regroup, one block per (b, h).  First the new cluster offsets:
// the new tokens are counted per cluster, off'[c] = off[c] + (new tokens in
// clusters before c), and that shift is kept for the move of the old entries
// (a later kernel, from the snapshot).  Then the new tokens are placed after
// their clusters' old entries, in token order, kPlaceTile tokens at a time
// (slots that the old entries never take).  The tile's list ids go to LDS;
// W waves each take a contiguous chunk of it and count its tokens per cluster;
// a prefix over the chunks gives every chunk its first slot in each cluster
// (the cluster's next free slot plus the earlier chunks' tokens); then each
// wave gives its tokens their slots, 64 at a time, the earlier tokens of the
// same cluster among the 64 read lane by lane from registers; finally all
// threads copy the entries to their slots.
constexpr int kPlaceTile = 4096;

// chunks of a tile: as many as up to 16 waves, within 128 KB of counters
__host__ __device__ inline int place_chunks(int L) { return min(16, max(1, 32768 / L - 1)); }

__global__ __launch_bounds__(1024) void k_append_place(AppendArgs a) {
  extern __shared__ int32_t slot[];    // [W][L] chunk counts, then chunk slots; [L] next free
  __shared__ int32_t lid[kPlaceTile];  // a tile's clusters, then their slots (-1: none)
  __shared__ int wsum[16];
  const Dims& d = a.d;
  const int L = d.L;
  const int W = place_chunks(L);
  int32_t* nextf = slot + (size_t)W * L;
  const int bh = blockIdx.x;
  const int b = bh / d.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  int old_n, new_n;
  append_span(a, b, &old_n, &new_n);
  const size_t base = (size_t)bh * d.cap;
  int32_t* off = a.ix.list_off + (size_t)bh * (L + 1);
  const int32_t* oo = a.old_off + (size_t)bh * (L + 1);
  int32_t* shift = a.shift + (size_t)bh * (L + 1);
  // new tokens per cluster
  for (int c = tid; c < L; c += blockDim.x) nextf[c] = 0;
  __syncthreads();
  for (int t = old_n + tid; t < new_n; t += blockDim.x) {
    const int c = a.list_ids[base + t];
    if (c >= 0 && c < L) atomicAdd(&nextf[c], 1);
  }
  __syncthreads();
  {
    // exclusive prefix over clusters, each thread a run of them; a cluster's
    // new entries start after its old ones, at its new offset
    const int per = (L + blockDim.x - 1) / blockDim.x;
    const int c0 = min(L, tid * per), c1 = min(L, c0 + per);
    int mine = 0;
    for (int c = c0; c < c1; ++c) mine += nextf[c];
    const int incl = wave_incl_scan(mine);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int before = incl - mine;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    for (int c = c0; c < c1; ++c) {
      const int n_new_c = nextf[c];
      shift[c] = before;
      off[c] = oo[c] + before;
      nextf[c] = oo[c] + before + (oo[c + 1] - oo[c]);
      before += n_new_c;
    }
    if (tid == blockDim.x - 1) {
      int tot = 0;
      for (int w = 0; w < nw; ++w) tot += wsum[w];
      off[L] = oo[L] + tot;
      shift[L] = tot;
    }
  }
  for (int s0 = old_n; s0 < new_n; s0 += kPlaceTile) {
    const int n = min(kPlaceTile, new_n - s0);
    const int chunk = (n + W - 1) / W;
    for (int i = tid; i < n; i += blockDim.x) {
      const int c = a.list_ids[base + s0 + i];
      lid[i] = (c < 0 || c >= L) ? -1 : c;
    }
    for (int i = tid; i < W * L; i += blockDim.x) slot[i] = 0;
    __syncthreads();
    if (wave < W) {
      const int e = min(n, (wave + 1) * chunk);
      for (int i = wave * chunk + lane; i < e; i += 64) {
        const int c = lid[i];
        if (c >= 0) atomicAdd(&slot[wave * L + c], 1);
      }
    }
    __syncthreads();
    for (int c = tid; c < L; c += blockDim.x) {
      int run = nextf[c];
      for (int w = 0; w < W; ++w) {
        const int t = slot[w * L + c];
        slot[w * L + c] = run;
        run += t;
      }
      nextf[c] = run;
    }
    __syncthreads();
    if (wave < W) {
      int32_t* sw = slot + wave * L;
      const int e = min(n, (wave + 1) * chunk);
      for (int g = wave * chunk; g < e; g += 64) {
        const int i = g + lane;
        const int c = i < e ? lid[i] : -1;
        int rank = 0, same = 0;
#pragma unroll
        for (int j = 0; j < 64; ++j) {
          const int cj = __builtin_amdgcn_readlane(c, j);
          same += (cj == c);
          rank += (cj == c) & (j < lane);
        }
        int dst = -1;
        if (c >= 0) {
          dst = sw[c] + rank;
          if (dst < 0 || dst >= d.cap) dst = -1;
        }
        // every lane has read its cluster's slot before any lane moves it
        __builtin_amdgcn_wave_barrier();
        if (i < e) lid[i] = dst;
        if (c >= 0 && rank == same - 1) sw[c] += same;
        __builtin_amdgcn_wave_barrier();
      }
    }
    __syncthreads();
    for (int i = tid; i < n; i += blockDim.x) {
      const int dst = lid[i];
      if (dst >= 0) {
        const int t = s0 + i;
        reinterpret_cast<uint4*>(a.ix.codes)[base + dst] =
            reinterpret_cast<const uint4*>(a.codes)[base + t];
        a.ix.pos[base + dst] = t;
        a.ix.ent_list[base + dst] = a.list_ids[base + t];
      }
    }
    __syncthreads();
  }
}

hipError_t launch_append_regroup(const AppendArgs& a, hipStream_t st) {
  const Dims& d = a.d;
  const int BH = d.B * d.Hkv;
  // the new offsets and the new tokens' slots first; the old entries then
  // move by the shift that kernel leaves (disjoint slots)
  const size_t plds = (size_t)(place_chunks(d.L) + 1) * d.L * sizeof(int32_t);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_append_place),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)plds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_append_place, dim3(BH), dim3(1024), plds, st, a);
  hipLaunchKernelGGL(k_append_move, dim3((d.cap + 255) / 256, BH), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_append_snapshot(const AppendArgs& a, hipStream_t st) {
  const int BH = a.d.B * a.d.Hkv;
  hipLaunchKernelGGL(k_append_snapshot, dim3((a.d.cap + 255) / 256, BH), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_append_encode(const AppendArgs& a, int max_new, hipStream_t st) {
  const int BH = a.d.B * a.d.Hkv;
  const int tiles = (max_new + kEncTokens - 1) / kEncTokens;
  if (tiles == 0) return hipSuccess;
  const size_t alds = (size_t)2 * kEncTokens * kRowPad * sizeof(float);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_append_assign),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)alds);
  if (e != hipSuccess) return e;
  // small batches split the centroid chunks over blocks until about 512
  // blocks run (two per CU fit in LDS)
  AppendArgs x = a;
  const int nch = (a.d.L + kAsgCents - 1) / kAsgCents;
  const int want = std::max(1, std::min(nch, (512 + BH * tiles - 1) / (BH * tiles)));
  x.asg_chunks = (nch + want - 1) / want;
  const int splits = (nch + x.asg_chunks - 1) / x.asg_chunks;
  hipLaunchKernelGGL(k_append_assign, dim3(BH, tiles, splits), dim3(kEncThreads), alds, st, x);
  hipLaunchKernelGGL(k_append_pq, dim3(BH, tiles, kM), dim3(256), 0, st, x);
  return hipGetLastError();
}

hipError_t launch_append_means(const AppendArgs& a, hipStream_t st) {
  const int BH = a.d.B * a.d.Hkv;
  hipLaunchKernelGGL(k_append_means, dim3(BH, (a.d.L + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace pqhsa
