// C ABI of libpqhsa: the entry points that launch kernels or touch device
// memory (argument checks, then launch order).  Validation, sizes and layouts
// are in pqhsa_host.cpp; the operations are documented in include/pqhsa.h.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "pqhsa_host.hpp"
#include "pqhsa_internal.hpp"

using namespace pqhsa;

namespace {

IndexPtrs index_ptrs(const Dims& d, void* buf) {
  const IndexLayout l = index_layout(d);
  char* p = static_cast<char*>(buf);
  IndexPtrs ix;
  ix.centroids = reinterpret_cast<float*>(p + l.centroids);
  ix.codebooks = reinterpret_cast<float*>(p + l.codebooks);
  ix.list_off = reinterpret_cast<int32_t*>(p + l.list_off);
  ix.codes = reinterpret_cast<uint8_t*>(p + l.codes);
  ix.pos = reinterpret_cast<int32_t*>(p + l.pos);
  ix.ent_list = reinterpret_cast<int32_t*>(p + l.ent_list);
  ix.means = reinterpret_cast<float*>(p + l.means);
  ix.n_indexed = reinterpret_cast<int32_t*>(p + l.n_indexed);
  ix.dropped = reinterpret_cast<unsigned long long*>(p + l.dropped);
  return ix;
}

WsPtrs ws_ptrs(const Dims& d, bool dense, void* buf) {
  const WsLayout l = ws_layout(d, dense);
  char* p = static_cast<char*>(buf);
  WsPtrs w;
  memset(&w, 0, sizeof(w));
  if (!dense) {
    w.lut = reinterpret_cast<float*>(p + l.lut);
    w.qc = reinterpret_cast<float*>(p + l.qc);
    w.keys = reinterpret_cast<uint32_t*>(p + l.keys);
    w.bins = reinterpret_cast<float*>(p + l.bins);
    w.hist = reinterpret_cast<uint32_t*>(p + l.hist);
    w.seg_above = reinterpret_cast<int2*>(p + l.seg_above);
    w.seg_aw = reinterpret_cast<float*>(p + l.seg_aw);
    w.seg_tie = reinterpret_cast<uint4*>(p + l.seg_tie);
    w.seg_w = reinterpret_cast<float*>(p + l.seg_w);
    w.seg_cnt = reinterpret_cast<int32_t*>(p + l.seg_cnt);
    w.wsel = reinterpret_cast<unsigned long long*>(p + l.wsel);
    w.rows = reinterpret_cast<int32_t*>(p + l.rows);
    w.n_rows = reinterpret_cast<int32_t*>(p + l.n_rows);
    w.fsync = reinterpret_cast<uint32_t*>(p + l.fsync);
    w.fflags = reinterpret_cast<uint32_t*>(p + l.fflags);
    w.fcnt = reinterpret_cast<unsigned long long*>(p + l.fcnt);
    w.fpart = reinterpret_cast<unsigned long long*>(p + l.fpart);
  }
  w.partials = reinterpret_cast<float*>(p + l.partials);
  return w;
}

inline pqhsa_status hip_status(hipError_t e) { return e == hipSuccess ? PQHSA_OK : PQHSA_ERR_HIP; }

// Launch context of stage i: with an event array, events 2i and 2i+1 take
// the kernel's start and end.
Launch stage(hipEvent_t* evs, int i, hipStream_t st) {
  if (!evs) return Launch{st, nullptr, nullptr};
  return Launch{st, evs[2 * i], evs[2 * i + 1]};
}

#define PQHSA_TRY(expr)                         \
  do {                                          \
    pqhsa_status s_ = (expr);                   \
    if (s_ != PQHSA_OK) return s_;              \
  } while (0)

pqhsa_status run_dense(const pqhsa_shape* shape, const uint16_t* q, const uint16_t* k_cache,
                       const uint16_t* v_cache, const int32_t* block_table,
                       const int32_t* context_lens, float* out, float* lse, void* workspace,
                       size_t ws_bytes, hipEvent_t* evs, int* n_kernels, hipStream_t stream) {
  PQHSA_TRY(validate(shape, true));
  if (!q || !k_cache || !v_cache || !block_table || !context_lens || !out || !workspace)
    return PQHSA_ERR_INVALID_ARG;
  const Dims d = make_dims(shape, true);
  if (ws_bytes < ws_layout(d, true).total) return PQHSA_ERR_BUFFER_TOO_SMALL;
  StepArgs a;
  memset(&a, 0, sizeof(a));
  a.d = d;
  a.ws = ws_ptrs(d, true, workspace);
  a.q = q; a.kc = k_cache; a.vc = v_cache; a.table = block_table; a.ctx = context_lens;
  a.out = out; a.lse = lse;
  PQHSA_TRY(hip_status(launch_exact_and_background(a, true, stage(evs, 0, stream))));
  PQHSA_TRY(hip_status(launch_merge(a, stage(evs, 1, stream))));
  if (n_kernels) *n_kernels = 2;
  return PQHSA_OK;
}

pqhsa_status run_step(const pqhsa_shape* shape, const void* index_buf, const uint16_t* q,
                      const uint16_t* k_cache, const uint16_t* v_cache,
                      const int32_t* block_table, const int32_t* context_lens, float* out,
                      int32_t* selected, float* lse, void* workspace, size_t ws_bytes,
                      bool staged, bool barrier_test, bool keys_out, hipEvent_t* evs,
                      int* n_kernels, hipStream_t stream) {
  PQHSA_TRY(validate(shape, false));
  if (!index_buf || !q || !k_cache || !v_cache || !block_table || !context_lens || !out ||
      !workspace)
    return PQHSA_ERR_INVALID_ARG;
  const Dims d = make_dims(shape, false);
  if (ws_bytes < ws_layout(d, false).total) return PQHSA_ERR_BUFFER_TOO_SMALL;
  StepArgs a;
  memset(&a, 0, sizeof(a));
  a.d = d;
  a.ix = index_ptrs(d, const_cast<void*>(index_buf));
  a.ws = ws_ptrs(d, false, workspace);
  a.q = q; a.kc = k_cache; a.vc = v_cache; a.table = block_table; a.ctx = context_lens;
  a.out = out; a.selected = selected; a.max_sel = max_selected(shape); a.lse = lse;
  const int fP = staged ? 0 : fused_blocks_per_head(d);
  if ((barrier_test || keys_out) && fP == 0) return PQHSA_ERR_UNSUPPORTED;
  if (fP > 0) {
    // the whole step in one kernel
    a.d.fP = fP;
    a.d.fcpb = ceil_div(d.L, fP);
    a.d.fkeys_out = keys_out ? 1 : 0;
    if (barrier_test) {
      // one arrival more than there are blocks: every barrier wait runs out
      a.d.fbar_extra = 1;
      a.d.fbar_ticks = kBarrierTestTicks;
    }
    PQHSA_TRY(hip_status(launch_fused(a, stage(evs, 0, stream))));
    if (n_kernels) *n_kernels = 1;
    return PQHSA_OK;
  }
  PQHSA_TRY(hip_status(launch_tables(a, stage(evs, PQHSA_STAGE_TABLES, stream))));
  PQHSA_TRY(hip_status(launch_scan(a, stage(evs, PQHSA_STAGE_SCAN, stream))));
  PQHSA_TRY(hip_status(launch_collect(a, stage(evs, PQHSA_STAGE_COLLECT, stream))));
  PQHSA_TRY(hip_status(launch_select(a, stage(evs, PQHSA_STAGE_SELECT, stream))));
  PQHSA_TRY(hip_status(launch_exact_and_background(a, false, stage(evs, PQHSA_STAGE_ATTEND, stream))));
  PQHSA_TRY(hip_status(launch_merge(a, stage(evs, PQHSA_STAGE_MERGE, stream))));
  if (n_kernels) *n_kernels = PQHSA_NUM_STAGES;
  return PQHSA_OK;
}

ReusePtrs reuse_ptrs(const Dims& d, int W, void* buf) {
  const ReuseLayout l = reuse_layout(d, W);
  char* p = static_cast<char*>(buf);
  ReusePtrs r;
  memset(&r, 0, sizeof(r));
  r.qs = reinterpret_cast<uint16_t*>(p + l.qs);
  r.st = reinterpret_cast<float*>(p + l.st);
  r.tj = reinterpret_cast<int32_t*>(p + l.tj);
  r.cnt = reinterpret_cast<int32_t*>(p + l.cnt);
  r.W = W;
  r.S = reuse_slabs(W);
  return r;
}

pqhsa_status run_reuse(const pqhsa_shape* shape, int32_t window, float max_dist2,
                       const uint16_t* q, const uint16_t* q_search, const uint16_t* k_cache,
                       const uint16_t* v_cache, const int32_t* block_table,
                       const int32_t* context_lens, void* reuse_buf, size_t reuse_bytes,
                       float* out, float* lse, int32_t* reused_slot, float* min_dist2,
                       void* workspace, size_t ws_bytes, hipEvent_t* evs, int* n_kernels,
                       hipStream_t stream) {
  PQHSA_TRY(validate(shape, true));
  if (!reuse_window_ok(window) || isnan(max_dist2)) return PQHSA_ERR_INVALID_ARG;
  if (!q || !q_search || !k_cache || !v_cache || !block_table || !context_lens || !reuse_buf ||
      !out || !workspace)
    return PQHSA_ERR_INVALID_ARG;
  const Dims d = reuse_dims(shape);
  if (reuse_bytes < reuse_layout(d, window).total) return PQHSA_ERR_BUFFER_TOO_SMALL;
  const ReuseWs lw = reuse_ws(d, window);
  if (ws_bytes < lw.total) return PQHSA_ERR_BUFFER_TOO_SMALL;
  char* ws = static_cast<char*>(workspace);
  StepArgs a;
  memset(&a, 0, sizeof(a));
  a.d = d;
  a.ws.partials = reinterpret_cast<float*>(ws + lw.partials);
  a.ws.n_rows = reinterpret_cast<int32_t*>(ws + lw.n_merge);
  a.ru = reuse_ptrs(d, window, reuse_buf);
  a.ru.cand = reinterpret_cast<int4*>(ws + lw.cand);
  a.ru.q_search = q_search;
  a.ru.slot_out = reused_slot;
  a.ru.d2_out = min_dist2;
  a.ru.max_d2 = max_dist2;
  a.q = q; a.kc = k_cache; a.vc = v_cache; a.table = block_table; a.ctx = context_lens;
  a.out = out; a.lse = lse;
  PQHSA_TRY(hip_status(launch_reuse_search(a, stage(evs, 0, stream))));
  PQHSA_TRY(hip_status(launch_exact_reuse(a, stage(evs, 1, stream))));
  PQHSA_TRY(hip_status(launch_merge(a, stage(evs, 2, stream))));
  if (n_kernels) *n_kernels = 3;
  return PQHSA_OK;
}

// ---------------------------------------------------------------- fixed scratch
// The workspace of pqhsa_decode_step_noalloc: one array per device, held
// until the process ends.  Host code never uses the array's name as an
// address: the device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = (size_t)PQHSA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kScratchDevices = 64;
void* g_scratch[kScratchDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch (looked up on the first
// call on that device), or nullptr with *err set.
void* scratch_ptr(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kScratchDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

// Zero two byte ranges (16-byte aligned, multiples of 16 bytes) with plain
// vector stores: a kernel rather than a memset, so that the clearing can sit
// in a captured graph.
__global__ __launch_bounds__(256) void k_zero2(uint4* a, size_t na, uint4* b, size_t nb) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < na + nb; i += stride) {
    if (i < na) a[i] = make_uint4(0, 0, 0, 0);
    else b[i - na] = make_uint4(0, 0, 0, 0);
  }
}

}  // namespace

extern "C" {





pqhsa_status pqhsa_upload_index(const pqhsa_shape* shape, const float* centroids,
                                const float* codebooks, const int32_t* list_ids,
                                const uint8_t* codes, const int32_t* n_indexed,
                                const uint16_t* v_cache, const int32_t* block_table,
                                void* index_buf, size_t index_bytes, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  PQHSA_TRY(validate(shape, false));
  if (!centroids || !codebooks || !list_ids || !codes || !n_indexed || !v_cache ||
      !block_table || !index_buf || !workspace)
    return PQHSA_ERR_INVALID_ARG;
  const Dims d = make_dims(shape, false);
  if (index_bytes < index_layout(d).total) return PQHSA_ERR_BUFFER_TOO_SMALL;
  if (workspace_bytes < upload_ws_bytes(d)) return PQHSA_ERR_BUFFER_TOO_SMALL;
  UploadArgs a;
  memset(&a, 0, sizeof(a));
  a.d = d;
  a.ix = index_ptrs(d, index_buf);
  a.list_ids = list_ids;
  a.codes = codes;
  a.n_indexed = n_indexed;
  a.vc = v_cache;
  a.table = block_table;
  a.chunk_counts = static_cast<int32_t*>(workspace);
  const size_t BH = (size_t)d.B * d.Hkv;
  PQHSA_TRY(hip_status(hipMemcpyAsync(a.ix.centroids, centroids, BH * d.L * kD * sizeof(float),
                                      hipMemcpyDeviceToDevice, stream)));
  PQHSA_TRY(hip_status(hipMemcpyAsync(a.ix.codebooks, codebooks,
                                      BH * kM * kKsub * kDsub * sizeof(float),
                                      hipMemcpyDeviceToDevice, stream)));
  PQHSA_TRY(hip_status(hipMemcpyAsync(a.ix.n_indexed, n_indexed, d.B * sizeof(int32_t),
                                      hipMemcpyDeviceToDevice, stream)));
  PQHSA_TRY(hip_status(hipMemsetAsync(a.ix.dropped, 0, sizeof(unsigned long long), stream)));
  return hip_status(launch_upload(a, stream));
}


pqhsa_status pqhsa_append_tokens(const pqhsa_shape* shape, void* index_buf,
                                 const uint16_t* k_cache, const uint16_t* v_cache,
                                 const int32_t* block_table, const int32_t* new_n_indexed,
                                 int32_t max_new, int32_t* list_ids, uint8_t* codes,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  PQHSA_TRY(validate(shape, false));
  if (!index_buf || !k_cache || !v_cache || !block_table || !new_n_indexed || !list_ids ||
      !codes || !workspace || max_new < 0)
    return PQHSA_ERR_INVALID_ARG;
  const Dims d = make_dims(shape, false);
  if (max_new > d.cap) return PQHSA_ERR_INVALID_ARG;
  const AppendWs lw = append_ws(d);
  if (workspace_bytes < lw.total) return PQHSA_ERR_BUFFER_TOO_SMALL;
  char* ws = static_cast<char*>(workspace);
  AppendArgs aa;
  memset(&aa, 0, sizeof(aa));
  aa.d = d;
  aa.ix = index_ptrs(d, index_buf);
  aa.kc = k_cache;
  aa.vc = v_cache;
  aa.table = block_table;
  aa.new_n_indexed = new_n_indexed;
  aa.list_ids = list_ids;
  aa.codes = codes;
  aa.old_off = reinterpret_cast<int32_t*>(ws + lw.old_off);
  aa.shift = reinterpret_cast<int32_t*>(ws + lw.shift);
  aa.snap_codes = reinterpret_cast<uint8_t*>(ws + lw.codes);
  aa.snap_pos = reinterpret_cast<int32_t*>(ws + lw.pos);
  aa.snap_list = reinterpret_cast<int32_t*>(ws + lw.list);
  aa.best = reinterpret_cast<unsigned long long*>(ws + lw.best);
  aa.max_new = max_new;
  // 1. snapshot the cluster offsets and the cluster-major arrays
  PQHSA_TRY(hip_status(launch_append_snapshot(aa, stream)));
  // 2. encode the new tokens (reads the index's current n_indexed)
  PQHSA_TRY(hip_status(launch_append_encode(aa, max_new, stream)));
  // 3. new offsets, new entries placed, old entries moved
  PQHSA_TRY(hip_status(launch_append_regroup(aa, stream)));
  // 4. fold the new tokens' values into the cluster means; the index now
  //    covers the new tokens
  return hip_status(launch_append_means(aa, stream));
}

pqhsa_status pqhsa_index_dropped(const pqhsa_shape* shape, const void* index_buf,
                                 int64_t* dropped, hipStream_t stream) {
  PQHSA_TRY(validate(shape, false));
  if (!index_buf || !dropped) return PQHSA_ERR_INVALID_ARG;
  const Dims d = make_dims(shape, false);
  const IndexLayout l = index_layout(d);
  unsigned long long v = 0;
  PQHSA_TRY(hip_status(hipMemcpyAsync(&v, static_cast<const char*>(index_buf) + l.dropped,
                                      sizeof(v), hipMemcpyDeviceToHost, stream)));
  PQHSA_TRY(hip_status(hipStreamSynchronize(stream)));
  *dropped = (int64_t)v;
  return PQHSA_OK;
}

pqhsa_status pqhsa_decode_step(const pqhsa_shape* shape, const void* index_buf,
                               const uint16_t* q, const uint16_t* k_cache,
                               const uint16_t* v_cache, const int32_t* block_table,
                               const int32_t* context_lens, float* out, int32_t* selected,
                               float* lse, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  return run_step(shape, index_buf, q, k_cache, v_cache, block_table, context_lens, out,
                  selected, lse, workspace, workspace_bytes, false, false, false, nullptr,
                  nullptr, stream);
}

pqhsa_status pqhsa_decode_step_noalloc(const pqhsa_shape* shape, const void* index_buf,
                                       const uint16_t* q, const uint16_t* k_cache,
                                       const uint16_t* v_cache, const int32_t* block_table,
                                       const int32_t* context_lens, float* out,
                                       int32_t* selected, float* lse, hipStream_t stream) {
  PQHSA_TRY(validate(shape, false));
  const Dims d = make_dims(shape, false);
  const WsLayout l = ws_layout(d, false);
  if (!index_buf || !q || !k_cache || !v_cache || !block_table || !context_lens || !out)
    return PQHSA_ERR_INVALID_ARG;
  if (l.total > kScratchBytes) return PQHSA_ERR_BUFFER_TOO_SMALL;
  hipError_t e = hipSuccess;
  char* ws = static_cast<char*>(scratch_ptr(&e));
  if (!ws) return PQHSA_ERR_HIP;
  // the histogram, counters and flags start at zero: the previous call on
  // this device may have used another shape (another layout of the array)
  const size_t hist_bytes = (size_t)d.B * d.Hkv * kHistStride * sizeof(uint32_t);
  const size_t ctr_bytes = l.fpart - l.fsync;
  const size_t n16 = (hist_bytes + ctr_bytes) / 16;
  const int blocks = (int)std::min<size_t>(1024, (n16 + 255) / 256);
  hipLaunchKernelGGL(k_zero2, dim3(blocks), dim3(256), 0, stream,
                     reinterpret_cast<uint4*>(ws + l.hist), hist_bytes / 16,
                     reinterpret_cast<uint4*>(ws + l.fsync), ctr_bytes / 16);
  PQHSA_TRY(hip_status(hipGetLastError()));
  return run_step(shape, index_buf, q, k_cache, v_cache, block_table, context_lens, out,
                  selected, lse, ws, kScratchBytes, false, false, false, nullptr, nullptr,
                  stream);
}

pqhsa_status pqhsa_dense_decode_step(const pqhsa_shape* shape, const uint16_t* q,
                                     const uint16_t* k_cache, const uint16_t* v_cache,
                                     const int32_t* block_table, const int32_t* context_lens,
                                     float* out, float* lse, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  return run_dense(shape, q, k_cache, v_cache, block_table, context_lens, out, lse, workspace,
                   workspace_bytes, nullptr, nullptr, stream);
}

pqhsa_status pqhsa_decode_step_profiled(const pqhsa_shape* shape, const void* index_buf,
                                        const uint16_t* q, const uint16_t* k_cache,
                                        const uint16_t* v_cache, const int32_t* block_table,
                                        const int32_t* context_lens, float* out,
                                        int32_t* selected, float* lse, void* workspace,
                                        size_t workspace_bytes, int variant,
                                        hipEvent_t* events, int32_t* n_kernels,
                                        hipStream_t stream) {
  if (!events) return PQHSA_ERR_INVALID_ARG;
  int nk = 0;
  pqhsa_status st;
  switch (variant) {
    case PQHSA_VARIANT_DEFAULT:
    case PQHSA_VARIANT_STAGED:
    case PQHSA_VARIANT_BARRIER_TEST:
    case PQHSA_VARIANT_KEYS_OUT:
      st = run_step(shape, index_buf, q, k_cache, v_cache, block_table, context_lens, out,
                    selected, lse, workspace, workspace_bytes, variant == PQHSA_VARIANT_STAGED,
                    variant == PQHSA_VARIANT_BARRIER_TEST, variant == PQHSA_VARIANT_KEYS_OUT,
                    events, &nk, stream);
      break;
    case PQHSA_VARIANT_DENSE:
      st = run_dense(shape, q, k_cache, v_cache, block_table, context_lens, out, lse, workspace,
                     workspace_bytes, events, &nk, stream);
      break;
    default:
      return PQHSA_ERR_INVALID_ARG;
  }
  if (n_kernels) *n_kernels = nk;
  return st;
}


pqhsa_status pqhsa_step_flags(const pqhsa_shape* shape, void* workspace, size_t workspace_bytes,
                              int clear, uint32_t* flags, hipStream_t stream) {
  PQHSA_TRY(validate(shape, false));
  if (!workspace || !flags) return PQHSA_ERR_INVALID_ARG;
  const Dims d = make_dims(shape, false);
  const WsLayout l = ws_layout(d, false);
  if (workspace_bytes < l.total) return PQHSA_ERR_BUFFER_TOO_SMALL;
  char* ws = static_cast<char*>(workspace);
  uint32_t v = 0;
  PQHSA_TRY(hip_status(hipMemcpyAsync(&v, ws + l.fflags, sizeof(v), hipMemcpyDeviceToHost,
                                      stream)));
  PQHSA_TRY(hip_status(hipStreamSynchronize(stream)));
  *flags = v;
  if (clear) {
    // the step's counters, per-head flags, per-block counts and histogram:
    // everything a step expects to find cleared
    PQHSA_TRY(hip_status(hipMemsetAsync(ws + l.hist, 0,
                                        (size_t)d.B * d.Hkv * kHistStride * sizeof(uint32_t),
                                        stream)));
    PQHSA_TRY(hip_status(hipMemsetAsync(ws + l.fsync, 0, l.fpart - l.fsync, stream)));
    PQHSA_TRY(hip_status(hipStreamSynchronize(stream)));
  }
  return PQHSA_OK;
}





pqhsa_status pqhsa_reuse_clear(const pqhsa_shape* shape, int32_t window, void* reuse_buf,
                               size_t reuse_bytes, int32_t seq_begin, int32_t seq_end,
                               hipStream_t stream) {
  PQHSA_TRY(validate(shape, true));
  if (!reuse_window_ok(window) || !reuse_buf) return PQHSA_ERR_INVALID_ARG;
  if (seq_begin < 0 || seq_end > shape->batch || seq_begin > seq_end) return PQHSA_ERR_INVALID_ARG;
  const Dims d = reuse_dims(shape);
  if (reuse_bytes < reuse_layout(d, window).total) return PQHSA_ERR_BUFFER_TOO_SMALL;
  StepArgs a;
  memset(&a, 0, sizeof(a));
  a.d = d;
  a.ru = reuse_ptrs(d, window, reuse_buf);
  return hip_status(launch_reuse_clear(a, seq_begin, seq_end, stream));
}

pqhsa_status pqhsa_reuse_decode_step(const pqhsa_shape* shape, int32_t window, float max_dist2,
                                     const uint16_t* q, const uint16_t* q_search,
                                     const uint16_t* k_cache, const uint16_t* v_cache,
                                     const int32_t* block_table, const int32_t* context_lens,
                                     void* reuse_buf, size_t reuse_bytes, float* out, float* lse,
                                     int32_t* reused_slot, float* min_dist2, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  return run_reuse(shape, window, max_dist2, q, q_search, k_cache, v_cache, block_table,
                   context_lens, reuse_buf, reuse_bytes, out, lse, reused_slot, min_dist2,
                   workspace, workspace_bytes, nullptr, nullptr, stream);
}

pqhsa_status pqhsa_reuse_decode_step_profiled(
    const pqhsa_shape* shape, int32_t window, float max_dist2, const uint16_t* q,
    const uint16_t* q_search, const uint16_t* k_cache, const uint16_t* v_cache,
    const int32_t* block_table, const int32_t* context_lens, void* reuse_buf, size_t reuse_bytes,
    float* out, float* lse, int32_t* reused_slot, float* min_dist2, void* workspace,
    size_t workspace_bytes, hipEvent_t* events, int32_t* n_kernels, hipStream_t stream) {
  if (!events) return PQHSA_ERR_INVALID_ARG;
  int nk = 0;
  const pqhsa_status st =
      run_reuse(shape, window, max_dist2, q, q_search, k_cache, v_cache, block_table,
                context_lens, reuse_buf, reuse_bytes, out, lse, reused_slot, min_dist2,
                workspace, workspace_bytes, events, &nk, stream);
  if (n_kernels) *n_kernels = nk;
  return st;
}


}  // extern "C"
