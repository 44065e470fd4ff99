// Query reuse: search of each query head's ring of earlier queries, and ring
// clearing.
//
// The quant_prune_distill post on query reuse (opening paragraph and section
// "Important practical considerations"): when an earlier query is close to
// the current one, that query's attention numerator and denominator over its
// prefix are reused and only the later tokens are computed; closeness is the
// L2 distance of pre-RoPE vectors, searched over a small sliding buffer of
// recent queries (section "Experiments": the last 1024 tokens).
//
// Search block: 256 threads = 16 row groups of 16 lanes; block (bq, s) scores
// the 128 slots [128 s, 128 s + 128) of head bq's ring.  Each group takes 8
// slots, issues all 8 loads (16 B per lane of each 256 B bf16 vector) before
// using any, forms the squared distance with a 16-lane DPP reduction, and
// keeps the best eligible slot; the block's best goes to one candidate
// record.  The split-K attention blocks reduce the candidates of their heads.
#include <algorithm>

#include "pqhsa_internal.hpp"

namespace pqhsa {

__global__ __launch_bounds__(256) void k_reuse_search(StepArgs a) {
  __shared__ int stj[kReuseSlab];
  __shared__ unsigned long long gkey[16];
  __shared__ int gslot[16];
  const ReusePtrs& r = a.ru;
  const int bq = blockIdx.x / r.S, s = blockIdx.x % r.S;
  const int b = bq / a.d.Hq;
  const int T = min(max(a.ctx[b], 0), a.d.cap);
  const int tid = threadIdx.x, l16 = tid & 15, rg = tid >> 4;
  const int w0 = s * kReuseSlab;
  if (tid < kReuseSlab) stj[tid] = w0 + tid < r.W ? r.tj[(size_t)bq * r.W + w0 + tid] : 0;
  float x[8];
  {
    const uint4 v = *reinterpret_cast<const uint4*>(r.q_search + (size_t)bq * kD + l16 * 8);
    const float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                        bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = f[i];
  }
  constexpr int kPer = kReuseSlab / 16;
  uint4 y[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int w = w0 + rg + 16 * u;
    y[u] = make_uint4(0, 0, 0, 0);
    if (w < r.W) y[u] = *reinterpret_cast<const uint4*>(r.qs + ((size_t)bq * r.W + w) * kD + l16 * 8);
  }
  __syncthreads();
  unsigned long long best = ~0ull;
  int bslot = -1;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const uint4 v = y[u];
    const float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                        bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
    float d2 = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e = x[i] - f[i];
      d2 = fmaf(e, e, d2);
    }
    d2 = row16_sum(d2);
    const int w = w0 + rg + 16 * u;
    const int t = stj[rg + 16 * u];
    // eligible: a filled slot, inserted at or before T, within the window
    if (w < r.W && t >= 1 && t <= T && T - t < r.W) {
      // distance ascending, then T_j descending; slots rise with u
      const unsigned long long key =
          ((unsigned long long)__float_as_uint(d2) << 32) | (uint32_t)~(uint32_t)t;
      if (key < best) { best = key; bslot = w; }
    }
  }
  if (l16 == 0) { gkey[rg] = best; gslot[rg] = bslot; }
  __syncthreads();
  if (tid == 0) {
    for (int g = 1; g < 16; ++g) {
      if (gkey[g] < best || (gkey[g] == best && (uint32_t)gslot[g] < (uint32_t)bslot)) {
        best = gkey[g];
        bslot = gslot[g];
      }
    }
    int4 c;
    if (bslot >= 0) c = make_int4((int)(uint32_t)(best >> 32), (int)~(uint32_t)best, bslot, 0);
    else c = make_int4((int)0x7f800000u, 0, -1, 0);
    r.cand[(size_t)bq * r.S + s] = c;
  }
}

// Empty the rings of sequences [b0, b1): every slot's T_j and the count to 0.
__global__ __launch_bounds__(256) void k_reuse_clear(StepArgs a, int b0, int b1) {
  const ReusePtrs& r = a.ru;
  const size_t q0 = (size_t)b0 * a.d.Hq, q1 = (size_t)b1 * a.d.Hq;
  const size_t n = (q1 - q0) * r.W;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    r.tj[q0 * r.W + i] = 0;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < q1 - q0;
       i += (size_t)gridDim.x * blockDim.x)
    r.cnt[q0 + i] = 0;
}

hipError_t launch_reuse_search(const StepArgs& a, const Launch& l) {
  return launch_kernel(k_reuse_search, dim3(a.d.B * a.d.Hq * a.ru.S), dim3(256), 0, l, a);
}

hipError_t launch_reuse_clear(const StepArgs& a, int seq_begin, int seq_end, hipStream_t st) {
  if (seq_end <= seq_begin) return hipSuccess;
  const size_t n = (size_t)(seq_end - seq_begin) * a.d.Hq * a.ru.W;
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(k_reuse_clear, dim3(blocks), dim3(256), 0, st, a, seq_begin, seq_end);
  return hipGetLastError();
}

}  // namespace pqhsa
