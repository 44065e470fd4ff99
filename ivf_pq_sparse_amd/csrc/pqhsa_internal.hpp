// Internal declarations of libpqhsa: argument blocks, device helpers and the
// kernel launchers shared by the translation units.  Not part of the ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pqhsa.h"
#include "pqhsa_config.hpp"

namespace pqhsa {

struct IndexPtrs {
  float* centroids;    // [BH][L][128]
  float* codebooks;    // [BH][16][256][8]
  int32_t* list_off;   // [BH][L+1]
  uint8_t* codes;      // [BH][cap][16] cluster order
  int32_t* pos;        // [BH][cap]     token position of each entry
  int32_t* ent_list;   // [BH][cap]     cluster of each entry
  float* means;        // [BH][L][128]
  int32_t* n_indexed;  // [B]
  unsigned long long* dropped;  // [1]
};

struct WsPtrs {
  float* lut;          // [BH][16][256][G]
  float* qc;           // [BH][L][G]
  uint32_t* keys;      // [BH][cap]
  float* bins;         // [BH][L][G][2]
  uint32_t* hist;      // [BH][4096]
  int2* seg_above;     // [BH][cap]  (pos, cluster) of keys above the threshold bucket,
                       //            one 4096-slot segment per collect block
  float* seg_aw;       // [BH][cap][G] their approximate weights relative to the cluster max
  uint4* seg_tie;      // [BH][cap]  (key, pos, entry, cluster) of keys in the threshold bucket
  float* seg_w;        // [BH][cap][G] their approximate weights relative to the cluster max
  int32_t* seg_cnt;    // [BH][slices][2] counts (above, tie) of each segment
  unsigned long long* wsel;  // [BH][L][G] selected entries' weights per cluster, fixed point 2^-40
                             // (written by the selection with plain stores)
  int32_t* rows;       // [BH][cap] exact rows as physical cache rows (page * 16 + slot)
  int32_t* n_rows;     // [BH] exact rows (query reuse: partials to merge)
  float* partials;     // [B][Hq][n_parts][132]
  // fused step only
  uint32_t* fsync;     // [BH][3][kSyncStride] arrivals at the two per-head barriers,
                       //   finished blocks: each counter on a cache line of its own
  uint32_t* fflags;    // [1] bit 0: a barrier wait timed out
  unsigned long long* fcnt;  // [BH][kMaxFusedP] (above count | tie count << 32) per block
  unsigned long long* fpart;  // [BH][G][kMaxFusedP][132] one partial per block and query
                              //   head: at G = 8 64-bit words (float | tag << 32),
                              //   else floats
};

// Query reuse: the per-(sequence, query head) rings of earlier queries and
// the step's inputs and outputs that belong to reuse only.
struct ReusePtrs {
  uint16_t* qs;               // [B*Hq][W][128] bf16 search vectors
  float* st;                  // [B*Hq][W][132] states: m (base 2), l, pad, pad, acc[128]
  int32_t* tj;                // [B*Hq][W] context length at insertion, 0 = empty slot
  int32_t* cnt;               // [B*Hq] entries inserted so far
  int4* cand;                 // [B*Hq][S] best entry of each slab: (d2 bits, T_j, slot, 0)
  const uint16_t* q_search;   // [B][Hq][128] bf16
  int32_t* slot_out;          // [B][Hq] reused slot or -1 (optional)
  float* d2_out;              // [B][Hq] smallest eligible squared distance (optional)
  int W;                      // slots per ring (the search window in tokens)
  int S;                      // search slabs per ring, ceil(W / kReuseSlab)
  float max_d2;               // reuse when the smallest distance is <= this
};

struct StepArgs {
  Dims d;
  IndexPtrs ix;
  WsPtrs ws;
  ReusePtrs ru;
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* table;
  const int32_t* ctx;
  float* out;
  int32_t* selected;
  int32_t max_sel;
  float* lse;
};

struct UploadArgs {
  Dims d;
  IndexPtrs ix;
  const int32_t* list_ids;   // [BH][cap]
  const uint8_t* codes;      // [BH][cap][16]
  const int32_t* n_indexed;  // [B]
  const uint16_t* vc;
  const int32_t* table;
  int32_t* chunk_counts;     // [BH][chunks][L]
};

struct AppendArgs {
  Dims d;
  IndexPtrs ix;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* table;
  const int32_t* new_n_indexed;  // [B]
  int32_t* list_ids;             // [BH][cap] token order (written for the new tokens)
  uint8_t* codes;                // [BH][cap][16] token order (written for the new tokens)
  int32_t* old_off;              // [BH][L+1] cluster offsets before the append
  int32_t* shift;                // [BH][L+1] new tokens in clusters before c
  uint8_t* snap_codes;           // [BH][cap][16] index arrays before the append
  int32_t* snap_pos;             // [BH][cap]
  int32_t* snap_list;            // [BH][cap]
  // [BH][cap] token order: (fp32 bits of the distance << 32) | list of the
  // nearest centroid found so far; the minimum over centroid splits
  unsigned long long* best;
  int asg_chunks;                // 64-centroid chunks per assignment block
  int max_new;                   // at most this many new tokens per sequence are added
};

// Tokens [*old_n, *new_n) of sequence b that an append adds: the requested
// span, clamped to the capacity and to max_new tokens (the rest stay in the
// exact tail).
__device__ __forceinline__ void append_span(const AppendArgs& a, int b, int* old_n, int* new_n) {
  const int o = min(max(a.ix.n_indexed[b], 0), a.d.cap);
  const int n = min(max(a.new_n_indexed[b], 0), a.d.cap);
  *old_n = o;
  *new_n = min(n, o + a.max_new);
}

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Order-preserving map float -> uint32 (larger float, larger integer).  Every
// non-NaN float maps above 0, which is reserved for "not a candidate".
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Block barrier that orders LDS only.  __syncthreads also makes earlier
// global stores visible, and its wait for them (vmcnt) waits for every global
// load still in flight as well; this barrier leaves those loads in flight.
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
// quad_perm(1,0,3,2), quad_perm(2,3,0,1), row_half_mirror, row_mirror.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x141>(x);
  x += dpp_f<0x140>(x);
  return x;
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xF, false);
}

__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));
  x = fmaxf(x, dpp_f<0x4E>(x));
  x = fmaxf(x, dpp_f<0x141>(x));
  x = fmaxf(x, dpp_f<0x140>(x));
  return x;
}

// Sum and max over the 64 lanes without LDS traffic: DPP within each 16-lane
// row, then the four row results through scalar reads (wave-uniform result).
__device__ __forceinline__ float wave_sum_dpp(float x) {
  x = row16_sum(x);
  const int b = __float_as_int(x);
  return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) +
          __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(b, 32)) +
          __int_as_float(__builtin_amdgcn_readlane(b, 48)));
}
__device__ __forceinline__ float wave_max_dpp(float x) {
  x = row16_max(x);
  const int b = __float_as_int(x);
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)),
                     __int_as_float(__builtin_amdgcn_readlane(b, 16))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)),
                     __int_as_float(__builtin_amdgcn_readlane(b, 48))));
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts within each
// 16-lane row (row_shr 1, 2, 4, 8; lanes shifted in from outside the row add
// 0), then row_bcast:15 and row_bcast:31 carry the row totals upwards.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_i<0x111, 0xF>(x);
  x += dpp_i<0x112, 0xF>(x);
  x += dpp_i<0x114, 0xF>(x);
  x += dpp_i<0x118, 0xF>(x);
  x += dpp_i<0x142, 0xA>(x);
  x += dpp_i<0x143, 0xC>(x);
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// Block index -> (b*Hkv + h, sub-block) so that every kernel runs all blocks
// of one (b, h) on the same XCD: workgroups go to the 8 XCDs round-robin by
// linear index, and each XCD has its own L2, so a consumer kernel then finds
// its producer's data in the same L2.  `per` blocks per (b, h), BH heads.
constexpr int kXcds = 8;
__device__ __forceinline__ void xcd_map(int x, int BH, int per, int* bh, int* sub) {
  const int total = BH * per;
  if (total % kXcds == 0) {
    const int xcd = x % kXcds, j = x / kXcds;
    if (BH % kXcds == 0) {
      *bh = xcd + kXcds * (j / per);
      *sub = j % per;
      return;
    }
    if (kXcds % BH == 0) {
      *bh = xcd % BH;
      *sub = xcd / BH + (kXcds / BH) * j;
      return;
    }
  }
  *bh = x / per;
  *sub = x % per;
}

// Per-sequence quantities of the forced/candidate split.
struct SeqInfo {
  int T;          // context length (clamped to [0, cap])
  int ns;         // sink rows actually present, min(n_sink, T)
  int cand_beg;   // candidates are positions [cand_beg, cand_end)
  int cand_end;
  int n_cand;
  int k;          // budget, min(ceil(T*bp/10000), n_cand)
  int recent_beg; // exact rows [recent_beg, T) after the selected ones
};

__device__ __forceinline__ SeqInfo seq_info(const Dims& d, const int32_t* ctx,
                                            const int32_t* n_indexed, int b) {
  SeqInfo s;
  int T = min(max(ctx[b], 0), d.cap);
  int Ti = min(max(n_indexed[b], 0), T);
  int R = max(d.n_recent, T - Ti);
  s.T = T;
  s.ns = min(d.n_sink, T);
  s.cand_beg = d.n_sink;
  s.cand_end = T - R;
  s.n_cand = max(s.cand_end - s.cand_beg, 0);
  long long kk = ((long long)T * d.budget_bp + 9999) / 10000;
  s.k = (int)min((long long)s.n_cand, kk);
  s.recent_beg = max(T - R, s.ns);
  return s;
}

// Approximate base-2 logits of one index entry for the G query heads of its
// KV head: qc_g + sum_m lut[m][code_m][g], summed in subspace order.  The scan
// and the background kernel both call this, so an entry's value is
// bit-identical in both.
template <int G>
__device__ __forceinline__ void entry_logits(const float* __restrict__ lut, const float* qc,
                                             uint4 cw, float* s) {
#pragma unroll
  for (int g = 0; g < G; ++g) s[g] = qc[g];
  const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    const uint32_t code = (w[m >> 2] >> ((m & 3) * 8)) & 0xffu;
    const float* e = lut + (m * kKsub + code) * G;
    if constexpr (G == 8) {
      float4 a = *reinterpret_cast<const float4*>(e);
      float4 c = *reinterpret_cast<const float4*>(e + 4);
      s[0] += a.x; s[1] += a.y; s[2] += a.z; s[3] += a.w;
      s[4] += c.x; s[5] += c.y; s[6] += c.z; s[7] += c.w;
    } else if constexpr (G == 4) {
      float4 a = *reinterpret_cast<const float4*>(e);
      s[0] += a.x; s[1] += a.y; s[2] += a.z; s[3] += a.w;
    } else if constexpr (G == 2) {
      float2 a = *reinterpret_cast<const float2*>(e);
      s[0] += a.x; s[1] += a.y;
    } else {
      s[0] += e[0];
    }
  }
}

// ---------------------------------------------------------------- scan helpers
// LUT entry (m, code) of a G-interleaved table in LDS: byte offset code*4G
// plus the subspace base m*256*4G, which the compiler folds into the LDS
// instruction's immediate offset.
template <int G, int M>
__device__ __forceinline__ void lut_add(const float* lut, uint32_t code, float* s) {
  const float* e = lut + M * kKsub * G + code * G;
  if constexpr (G == 8) {
    const float4 a = *reinterpret_cast<const float4*>(e);
    const float4 c = *reinterpret_cast<const float4*>(e + 4);
    s[0] += a.x; s[1] += a.y; s[2] += a.z; s[3] += a.w;
    s[4] += c.x; s[5] += c.y; s[6] += c.z; s[7] += c.w;
  } else if constexpr (G == 4) {
    const float4 a = *reinterpret_cast<const float4*>(e);
    s[0] += a.x; s[1] += a.y; s[2] += a.z; s[3] += a.w;
  } else if constexpr (G == 2) {
    const float2 a = *reinterpret_cast<const float2*>(e);
    s[0] += a.x; s[1] += a.y;
  } else {
    s[0] += e[0];
  }
}

// Same sum as entry_logits (same order: qc, then subspaces 0..15).  For
// G <= 4 all 16 table reads are issued before the first add, so that a wave
// keeps 16 LDS reads in flight instead of a few.
template <int G>
__device__ __forceinline__ void entry_logits_lds(const float* lut, const float* qc, uint4 cw,
                                                 float* s) {
#pragma unroll
  for (int g = 0; g < G; ++g) s[g] = qc[g];
  if constexpr (G == 4) {
    const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
    float4 v[kM];
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      const uint32_t code = (w[m >> 2] >> ((m & 3) * 8)) & 0xffu;
      v[m] = *reinterpret_cast<const float4*>(lut + m * kKsub * 4 + code * 4);
    }
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      s[0] += v[m].x; s[1] += v[m].y; s[2] += v[m].z; s[3] += v[m].w;
    }
    return;
  }
  lut_add<G, 0>(lut, cw.x & 0xffu, s);
  lut_add<G, 1>(lut, (cw.x >> 8) & 0xffu, s);
  lut_add<G, 2>(lut, (cw.x >> 16) & 0xffu, s);
  lut_add<G, 3>(lut, cw.x >> 24, s);
  lut_add<G, 4>(lut, cw.y & 0xffu, s);
  lut_add<G, 5>(lut, (cw.y >> 8) & 0xffu, s);
  lut_add<G, 6>(lut, (cw.y >> 16) & 0xffu, s);
  lut_add<G, 7>(lut, cw.y >> 24, s);
  lut_add<G, 8>(lut, cw.z & 0xffu, s);
  lut_add<G, 9>(lut, (cw.z >> 8) & 0xffu, s);
  lut_add<G, 10>(lut, (cw.z >> 16) & 0xffu, s);
  lut_add<G, 11>(lut, cw.z >> 24, s);
  lut_add<G, 12>(lut, cw.w & 0xffu, s);
  lut_add<G, 13>(lut, (cw.w >> 8) & 0xffu, s);
  lut_add<G, 14>(lut, (cw.w >> 16) & 0xffu, s);
  lut_add<G, 15>(lut, cw.w >> 24, s);
}

// ---------------------------------------------------------------- threshold bucket
// From the 4096-bin histogram of candidate keys (top 12 bits), find the bucket
// holding the k-th largest key: beta with above(beta) < k <= above(beta) +
// hist[beta], where above(x) counts keys in buckets > x.  Also returns the
// total count.  Uses the whole block; blockDim is 256 or 1024.  sh must hold
// blockDim/64 + 3 ints.
__device__ inline void find_threshold(const uint32_t* __restrict__ gh, int k, int* sh, int* beta,
                               int* above, int* total) {
  const int nt = blockDim.x;
  const int per = kHistBins / nt;
  const int t = threadIdx.x;
  // thread t owns bins [hi - per, hi), hi = 4096 - t*per (thread 0 has the top)
  const int hi = kHistBins - t * per;
  int v[16];
  int s = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[i] = i < per ? (int)gh[hi - 1 - i] : 0;
    s += v[i];
  }
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
    for (int w = 0; w < nw; ++w) { int u = sh[w]; sh[w] = run; run += u; }
    sh[nw + 2] = run;
  }
  __syncthreads();
  const int tot = sh[nw + 2];
  const int kk = min(k, tot);
  const int before = sh[wave] + x - s;   // keys in bins above this thread's range
  if (kk > 0 && before < kk && before + s >= kk) {
    int run = before;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < per && run < kk) {
        if (run + v[i] >= kk) { sh[nw] = hi - 1 - i; sh[nw + 1] = run; }
        run += v[i];
      }
    }
  }
  __syncthreads();
  *beta = sh[nw];
  *above = sh[nw + 1];
  *total = tot;
  __syncthreads();
}

// ---------------------------------------------------------------- selection helpers
// Radix-select composite of a threshold-bucket entry: the key's low 20 bits,
// then the bit-inverted position, so that equal keys prefer the lower position.
__device__ __forceinline__ unsigned long long composite52(uint4 c) {
  return (((unsigned long long)c.x << 32) | (unsigned long long)(0xffffffffu - c.y)) &
         0x000fffffffffffffull;
}

// Flat index i over the concatenated segments -> segment, given the exclusive
// prefix pre[0..n] of segment sizes (pre[n] = total, i < total).
__device__ __forceinline__ int seg_of(const int* pre, int n, int i) {
  int lo = 0, hi = n;   // pre[lo] <= i < pre[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= i) lo = mid; else hi = mid;
  }
  return lo;
}

// ---------------------------------------------------------------- row tiles on MFMA
// Every exact-attention path (the dense step, the exact rows and background
// terms of the sparse steps, query reuse) accumulates through these.  A wave
// takes tiles of 16 rows (cache rows, or background terms with a given logit
// and value) for the 16 columns of its query heads (G of them used):
//   logits:  S^T[16 rows][16 cols] = K[16 rows][128] . Q^T[128][16 cols],
//            four 16x16x32 bf16 MFMAs; lane l holds S[row 4(l/16) + i][col
//            l%16], i = 0..3, and supplies K[row l%16][32(l/16) + 8c .. + 8]
//            to MFMA c (with q[col][32(l/16) + 8c .. + 8] as its B operand)
//   softmax: per column a running base-2 maximum, raised only when a tile's
//            maximum exceeds it by more than 8 (weights stay below 2^8); the
//            lane's four weights are exactly the B operand of
//   values:  O^T[128][16 cols] += V^T[128][16 rows] . P^T[16 rows][16 cols]
//            as eight 16x16x32 bf16 MFMAs, one per dim offset c (the MFMA's
//            row m stands for dim 8m + c): lane l supplies the bf16 values of
//            rows 4(l/16) + i at dim 8(l%16) + c, each twice, against the
//            weights split into a bf16 part and its bf16 residue (products
//            exact to 2^-17, sums in fp32), and accumulates
//            O[col l%16][32(l/16) + 8i' + c] in acc[c][i'], i' = 0..3.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

struct RowTileState {
  float m;        // base-2 reference maximum of the lane's column
  float l;        // sum of the lane's rows' weights against m
  f32x4 acc[8];   // O[col][32j + 8i + c] in acc[c][i], unnormalised
};

// Reference maximum of a column that has taken no row yet: finite, so that a
// masked row (logit -inf) weighs exp2(-inf) = 0 rather than exp2(NaN) even
// in a tile where every row of the column is masked; the first real logit
// raises it; tile_finish maps a column that took none to the empty state.
constexpr float kTileMInit = -1.0e30f;

__device__ __forceinline__ void tile_init(RowTileState& st) {
  st.m = kTileMInit;
  st.l = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c) st.acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

// B operand of the logit MFMAs: lane (col, j) holds q[col][32j + 8c .. + 8]
// for MFMA c, zero for columns past the G query heads (q: bf16 [G][128]).
template <int G>
__device__ __forceinline__ void tile_query(const uint16_t* q, int col, int j, bf16x8 (&qb)[4]) {
  const uint16_t* qr = q + min(col, G - 1) * kD + 32 * j;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint4 w = *reinterpret_cast<const uint4*>(qr + 8 * c);
    if (col >= G) w = make_uint4(0, 0, 0, 0);
    qb[c] = __builtin_bit_cast(bf16x8, w);
  }
}

// Base-2 logits of a tile of cache rows for the lane's column: kb[c] as
// described above (zero for rows that are not there); sv[i] is row 4j + i.
__device__ __forceinline__ f32x4 tile_logits(const bf16x8 (&qb)[4], const uint4 (&kb)[4],
                                             float scale_log2) {
  f32x4 sv = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < 4; ++c)
    sv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb[c]), qb[c], sv, 0,
                                                 0, 0);
  return sv * scale_log2;
}

// Online softmax of one tile: s[i] is the base-2 logit of row 4j + i for the
// lane's column (-inf: no row); returns the rows' weights against the
// column's reference maximum, which is raised (and the state rescaled) only
// when the tile exceeds it by more than 8.
__device__ __forceinline__ void tile_softmax(RowTileState& st, const float (&s)[4],
                                             float (&p)[4]) {
  float mt = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  if (__any(mt > st.m + 8.0f)) {
    // raise the column's reference maximum (uniform over its four lanes); a
    // wave-wide vote keeps the lane exchange off the common path
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    if (mt > st.m + 8.0f) {
      const float al = __builtin_amdgcn_exp2f(st.m - mt);
      st.l *= al;
#pragma unroll
      for (int c = 0; c < 8; ++c) st.acc[c] *= al;
      st.m = mt;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = __builtin_amdgcn_exp2f(s[i] - st.m);
    st.l += p[i];
  }
}

// x as a sum of two bf16 numbers, each rounded to nearest: |x - hi - lo| is
// below 2^-17 |x|, and a product of either with a bf16 value is exact in fp32.
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = (__bf16)x;
  lo = (__bf16)(x - (float)hi);
}

// B operand of the value MFMAs: the lane's four weights (rows 4j + i) at
// k = 8j + i as bf16, their rounding residues at k = 8j + 4 + i.
__device__ __forceinline__ bf16x8 tile_weights_operand(const float (&p)[4]) {
  bf16x8 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __bf16 h, l;
    split_bf16(p[i], h, l);
    w[i] = h;
    w[4 + i] = l;
  }
  return w;
}

// A operand of the value MFMA for dim offset c: element c of the lane's four
// bf16 rows (8 values each), at k = 8j + i and again at 8j + 4 + i, so that
// one MFMA takes both halves of the split weights.
__device__ __forceinline__ bf16x8 tile_values_operand(const uint4 (&v)[4], int c) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = c < 2 ? v[i].x : c < 4 ? v[i].y : c < 6 ? v[i].z : v[i].w;
    w[i] = (c & 1) ? x >> 16 : x & 0xffffu;
  }
  const uint32_t lo = w[0] | (w[1] << 16), hi = w[2] | (w[3] << 16);
  return __builtin_bit_cast(bf16x8, make_uint4(lo, hi, lo, hi));
}

// One tile of bf16 rows into the state: v[i] holds row 4j + i at dims
// 8 col .. 8 col + 7 (finite, so that a zero weight never meets a NaN).
// Values are exact bf16 and the weights are split into two bf16 terms, so
// the eight 16x16x32 bf16 MFMAs form every product to 2^-17 and sum in fp32.
__device__ __forceinline__ void tile_accumulate(RowTileState& st, const float (&s)[4],
                                                const uint4 (&v)[4]) {
  float p[4];
  tile_softmax(st, s, p);
  const bf16x8 w = tile_weights_operand(p);
#pragma unroll
  for (int c = 0; c < 8; ++c)
    st.acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tile_values_operand(v, c), w, st.acc[c],
                                                       0, 0, 0);
}

// The same for fp32 values v[i][c] (row 4j + i, dim 8 col + c): each value
// is split into two bf16 terms as well, one MFMA per term.
__device__ __forceinline__ void tile_accumulate_f32(RowTileState& st, const float (&s)[4],
                                                    const float (&v)[4][8]) {
  float p[4];
  tile_softmax(st, s, p);
  const bf16x8 w = tile_weights_operand(p);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    bf16x8 vh, vl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __bf16 h, l;
      split_bf16(v[i][c], h, l);
      vh[i] = vh[4 + i] = h;
      vl[i] = vl[4 + i] = l;
    }
    st.acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vh, w, st.acc[c], 0, 0, 0);
    st.acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vl, w, st.acc[c], 0, 0, 0);
  }
}

// The same for fp32 values on 32 16x16x4 fp32 MFMAs (for row group i and
// dim offset c, lane l supplies v[i][c] against its weight p[i]).  The dense
// step uses this form: on its HBM-bound page loop it measured faster than the
// split-weight bf16 form, although it issues more matrix work.
__device__ __forceinline__ void tile_accumulate_fp32mfma(RowTileState& st, const float (&s)[4],
                                                         const float (&v)[4][8]) {
  float p[4];
  tile_softmax(st, s, p);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 8; ++c)
      st.acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(v[i][c], p[i], st.acc[c], 0, 0, 0);
}

__device__ __forceinline__ void bf16x8_to_f32(uint4 w, float (&v)[8]) {
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}

// After the last tile: l summed over the column's four lanes, and the
// maximum of a column that took no row set to -inf (the empty state).
__device__ __forceinline__ void tile_finish(RowTileState& st) {
  st.l += __shfl_xor(st.l, 16);
  st.l += __shfl_xor(st.l, 32);
  if (st.l == 0.0f) st.m = -INFINITY;
}

// Scale factors that bring states with maxima m0 and m1 to their common max.
__device__ __forceinline__ void lse_factors(float m0, float m1, float* M, float* a0, float* a1) {
  *M = fmaxf(m0, m1);
  *a0 = (m0 == -INFINITY) ? 0.0f : exp2f(m0 - *M);
  *a1 = (m1 == -INFINITY) ? 0.0f : exp2f(m1 - *M);
}

// ---------------------------------------------------------------- launchers
// Stream and optional timing events of one kernel launch.  With events the
// launch goes through hipExtLaunchKernel, which stamps the two events with the
// kernel's own start and end (no gap to a separately recorded marker).
struct Launch {
  hipStream_t st;
  hipEvent_t start;
  hipEvent_t stop;
};

template <typename A>
inline hipError_t launch_kernel(void (*kernel)(A), dim3 grid, dim3 block, size_t lds,
                                const Launch& l, A arg) {
  void* argv[1] = {&arg};
  if (l.start)
    return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, lds, l.st,
                              l.start, l.stop, 0);
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, lds, l.st);
}

hipError_t launch_upload(const UploadArgs& a, hipStream_t st);
hipError_t launch_upload_regroup(const UploadArgs& a, hipStream_t st);
hipError_t launch_append_snapshot(const AppendArgs& a, hipStream_t st);
hipError_t launch_append_encode(const AppendArgs& a, int max_new, hipStream_t st);
hipError_t launch_append_means(const AppendArgs& a, hipStream_t st);
hipError_t launch_append_regroup(const AppendArgs& a, hipStream_t st);
hipError_t launch_tables(const StepArgs& a, const Launch& l);
hipError_t launch_scan(const StepArgs& a, const Launch& l);
hipError_t launch_collect(const StepArgs& a, const Launch& l);
hipError_t launch_select(const StepArgs& a, const Launch& l);
hipError_t launch_exact_and_background(const StepArgs& a, bool dense, const Launch& l);
hipError_t launch_merge(const StepArgs& a, const Launch& l);
hipError_t launch_exact_reuse(const StepArgs& a, const Launch& l);
hipError_t launch_reuse_search(const StepArgs& a, const Launch& l);
hipError_t launch_reuse_clear(const StepArgs& a, int seq_begin, int seq_end, hipStream_t st);
// Fused step: blocks per (b, h) that fit co-resident on the device (0 when the
// fused kernel cannot run this shape), and its launch.
int fused_blocks_per_head(const Dims& d);
size_t fused_lds_bytes(int G);
hipError_t launch_fused(const StepArgs& a, const Launch& l);

}  // namespace pqhsa
