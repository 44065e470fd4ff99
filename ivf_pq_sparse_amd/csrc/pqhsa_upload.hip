// Index upload: regroup the IVF-PQ codes by cluster and compute the cluster
// means (PQ-HSA page, section "How approximate estimates return the discarded
// context": the index groups keys into clusters and keeps compressed codes;
// unread tokens are represented by their cluster's mean value).
//
// The regrouping is a stable counting sort per (sequence, KV head):
//   1. per 4096-token chunk, a histogram of list ids (LDS atomics);
//   2. per (b, h), cluster sizes, cluster offsets and each chunk's base offset
//      inside every cluster;
//   3. per chunk, one wave walks its tokens in order in tiles of 64, ranks each
//      token among equal list ids earlier in the tile, and scatters codes and
//      positions.  Token order inside a cluster is kept, so the layout (and
//      every later floating-point sum over a cluster) is deterministic.
// Means: one wave per cluster sums its tokens' bf16 values in fp32, 4 tokens
// at a time (one per 16-lane row), reading them from the paged cache.
#include "pqhsa_internal.hpp"

namespace pqhsa {

__global__ __launch_bounds__(256) void k_upload_count(UploadArgs a) {
  extern __shared__ uint32_t lh[];
  const Dims& d = a.d;
  const int bh = blockIdx.x;
  const int chunk = blockIdx.y;
  const int b = bh / d.Hkv;
  for (int c = threadIdx.x; c < d.L; c += blockDim.x) lh[c] = 0;
  __syncthreads();
  const int Ti = min(max(a.n_indexed[b], 0), d.cap);
  const int t0 = chunk * kUploadChunk;
  const int t1 = min(Ti, t0 + kUploadChunk);
  const int32_t* lists = a.list_ids + (size_t)bh * d.cap;
  unsigned int bad = 0;
  for (int t = t0 + threadIdx.x; t < t1; t += blockDim.x) {
    const int c = lists[t];
    if (c >= 0 && c < d.L) atomicAdd(&lh[c], 1u);
    else ++bad;
  }
  if (bad) atomicAdd(a.ix.dropped, (unsigned long long)bad);
  __syncthreads();
  int32_t* out = a.chunk_counts + ((size_t)bh * d.upload_chunks + chunk) * d.L;
  for (int c = threadIdx.x; c < d.L; c += blockDim.x) out[c] = (int32_t)lh[c];
}

// Block-wide exclusive scan of one value per thread (blockDim multiple of 64).
__device__ int block_exclusive_scan(int v, int* sh_waves, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh_waves[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = lane < nw ? sh_waves[lane] : 0;
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(w, o);
      if (lane >= o) w += y;
    }
    if (lane < nw) sh_waves[lane] = w;   // inclusive wave totals
  }
  __syncthreads();
  const int before = wave ? sh_waves[wave - 1] : 0;
  *total = sh_waves[nw - 1];
  __syncthreads();
  return before + x - v;
}

__global__ __launch_bounds__(1024) void k_upload_offsets(UploadArgs a) {
  __shared__ int sh[16];
  const Dims& d = a.d;
  const int bh = blockIdx.x;
  int32_t* cnt = a.chunk_counts + (size_t)bh * d.upload_chunks * d.L;
  int32_t* off = a.ix.list_off + (size_t)bh * (d.L + 1);
  // each thread owns a contiguous run of clusters
  const int per = (d.L + blockDim.x - 1) / blockDim.x;
  const int c0 = min(d.L, (int)threadIdx.x * per), c1 = min(d.L, c0 + per);
  int mine = 0;
  for (int c = c0; c < c1; ++c)
    for (int ch = 0; ch < d.upload_chunks; ++ch) mine += cnt[(size_t)ch * d.L + c];
  int total;
  int run = block_exclusive_scan(mine, sh, &total);
  for (int c = c0; c < c1; ++c) {
    off[c] = run;
    for (int ch = 0; ch < d.upload_chunks; ++ch) {
      const int n = cnt[(size_t)ch * d.L + c];
      cnt[(size_t)ch * d.L + c] = run;   // becomes the chunk's base offset in cluster c
      run += n;
    }
  }
  if (threadIdx.x == 0) off[d.L] = total;
}

__global__ __launch_bounds__(64) void k_upload_scatter(UploadArgs a) {
  extern __shared__ int32_t base[];     // [L] next free slot of each cluster for this chunk
  __shared__ int32_t tile[64];
  const Dims& d = a.d;
  const int bh = blockIdx.x;
  const int chunk = blockIdx.y;
  const int b = bh / d.Hkv;
  const int lane = threadIdx.x;
  const int32_t* cb = a.chunk_counts + ((size_t)bh * d.upload_chunks + chunk) * d.L;
  for (int c = lane; c < d.L; c += 64) base[c] = cb[c];
  const int Ti = min(max(a.n_indexed[b], 0), d.cap);
  const int t0 = chunk * kUploadChunk;
  const int t1 = min(Ti, t0 + kUploadChunk);
  const int32_t* lists = a.list_ids + (size_t)bh * d.cap;
  const uint4* codes_in = reinterpret_cast<const uint4*>(a.codes + (size_t)bh * d.cap * kM);
  uint4* codes_out = reinterpret_cast<uint4*>(a.ix.codes + (size_t)bh * d.cap * kM);
  int32_t* pos_out = a.ix.pos + (size_t)bh * d.cap;
  int32_t* list_out = a.ix.ent_list + (size_t)bh * d.cap;
  __syncthreads();
  for (int s = t0; s < t1; s += 64) {
    const int t = s + lane;
    int c = -1;
    if (t < t1) {
      c = lists[t];
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
      const int dest = base[c] + rank;
      codes_out[dest] = codes_in[t];
      pos_out[dest] = t;
      list_out[dest] = c;
    }
    __syncthreads();
    if (c >= 0 && rank == same - 1) base[c] += same;
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void k_upload_means(UploadArgs a) {
  __shared__ float red[4][4][kD];
  const Dims& d = a.d;
  const int bh = blockIdx.x;
  const int b = bh / d.Hkv, h = bh % d.Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = lane >> 4, l16 = lane & 15;
  const int c = blockIdx.y * 4 + wave;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int n = 0;
  if (c < d.L) {
    const int32_t* off = a.ix.list_off + (size_t)bh * (d.L + 1);
    const int e0 = off[c], e1 = off[c + 1];
    n = e1 - e0;
    const int32_t* pos = a.ix.pos + (size_t)bh * d.cap;
    const int32_t* tab = a.table + (size_t)b * d.max_pages;
    for (int e = e0 + row; e < e1; e += 4) {
      const int p = pos[e];
      int page = tab[p / kPage];
      page = min(max(page, 0), d.num_pages - 1);
      const size_t off_row = ((size_t)(page * kPage + p % kPage) * d.Hkv + h) * kD + l16 * 8;
      const uint4 w = *reinterpret_cast<const uint4*>(a.vc + off_row);
      acc[0] += bf16_lo(w.x); acc[1] += bf16_hi(w.x);
      acc[2] += bf16_lo(w.y); acc[3] += bf16_hi(w.y);
      acc[4] += bf16_lo(w.z); acc[5] += bf16_hi(w.z);
      acc[6] += bf16_lo(w.w); acc[7] += bf16_hi(w.w);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[wave][row][l16 * 8 + i] = acc[i];
  __syncthreads();
  if (c < d.L) {
    float* mu = a.ix.means + ((size_t)bh * d.L + c) * kD;
    const float inv = n > 0 ? 1.0f / (float)n : 0.0f;
    for (int i = lane; i < kD; i += 64) {
      const float s = ((red[wave][0][i] + red[wave][1][i]) + red[wave][2][i]) + red[wave][3][i];
      mu[i] = n > 0 ? s * inv : 0.0f;
    }
  }
}

// Counting sort of the token-order list ids and codes into the cluster-major
// index (no means).
hipError_t launch_upload_regroup(const UploadArgs& a, hipStream_t st) {
  const Dims& d = a.d;
  const int BH = d.B * d.Hkv;
  hipLaunchKernelGGL(k_upload_count, dim3(BH, d.upload_chunks), dim3(256),
                     d.L * sizeof(uint32_t), st, a);
  hipLaunchKernelGGL(k_upload_offsets, dim3(BH), dim3(1024), 0, st, a);
  hipLaunchKernelGGL(k_upload_scatter, dim3(BH, d.upload_chunks), dim3(64),
                     d.L * sizeof(int32_t), st, a);
  return hipGetLastError();
}

hipError_t launch_upload(const UploadArgs& a, hipStream_t st) {
  const Dims& d = a.d;
  const int BH = d.B * d.Hkv;
  hipError_t e = launch_upload_regroup(a, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_upload_means, dim3(BH, (d.L + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace pqhsa
