// C ABI of libpqhsa: argument validation, buffer layouts and launch order.
// The operations themselves are documented in include/pqhsa.h.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "pqhsa_internal.hpp"

using namespace pqhsa;

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxContextLimit = 1 << 26;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

pqhsa_status validate(const pqhsa_shape* s, bool dense) {
  if (!s) return PQHSA_ERR_INVALID_ARG;
  if (s->batch < 1 || s->num_q_heads < 1 || s->num_kv_heads < 1) return PQHSA_ERR_INVALID_ARG;
  if (s->num_q_heads % s->num_kv_heads != 0) return PQHSA_ERR_INVALID_ARG;
  if (s->head_dim < 1 || s->page_size < 1) return PQHSA_ERR_INVALID_ARG;
  if (s->num_pages < 1 || s->max_pages_per_seq < 1 || s->max_context < 1)
    return PQHSA_ERR_INVALID_ARG;
  if ((long long)s->max_context > (long long)s->max_pages_per_seq * s->page_size)
    return PQHSA_ERR_INVALID_ARG;
  if (s->max_context > kMaxContextLimit) return PQHSA_ERR_UNSUPPORTED;
  if (!(s->scale > 0.0f) || !isfinite(s->scale)) return PQHSA_ERR_INVALID_ARG;
  const int G = s->num_q_heads / s->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return PQHSA_ERR_UNSUPPORTED;
  if (s->head_dim != kD || s->page_size != kPage) return PQHSA_ERR_UNSUPPORTED;
  // the K/V cache offsets are formed in 64-bit; page indices in 32-bit
  if ((long long)s->num_pages * kPage > 0x7fffffffLL) return PQHSA_ERR_UNSUPPORTED;
  if (dense) return PQHSA_OK;
  if (s->num_lists < 1 || s->pq_m < 1 || s->pq_ksub < 1) return PQHSA_ERR_INVALID_ARG;
  if (s->n_sink < 0 || s->n_recent < 0) return PQHSA_ERR_INVALID_ARG;
  if (s->budget_bp < 0 || s->budget_bp > 10000) return PQHSA_ERR_INVALID_ARG;
  if (s->exact_only != 0 && s->exact_only != 1) return PQHSA_ERR_INVALID_ARG;
  if (s->num_lists > kMaxLists) return PQHSA_ERR_UNSUPPORTED;
  if (s->pq_m != kM || s->pq_ksub != kKsub) return PQHSA_ERR_UNSUPPORTED;
  if (s->max_context > kMaxSparseContext) return PQHSA_ERR_UNSUPPORTED;
  return PQHSA_OK;
}

int max_selected(const pqhsa_shape* s) {
  const long long k = ((long long)s->max_context * s->budget_bp + 9999) / 10000;
  return (int)(k < s->max_context ? k : s->max_context);
}

Dims make_dims(const pqhsa_shape* s, bool dense) {
  Dims d;
  memset(&d, 0, sizeof(d));
  d.B = s->batch;
  d.Hq = s->num_q_heads;
  d.Hkv = s->num_kv_heads;
  d.G = d.Hq / d.Hkv;
  d.L = dense ? 1 : s->num_lists;
  d.num_pages = s->num_pages;
  d.max_pages = s->max_pages_per_seq;
  d.cap = s->max_context;
  d.n_sink = dense ? 0 : s->n_sink;
  d.n_recent = dense ? 0 : s->n_recent;
  d.budget_bp = dense ? 0 : s->budget_bp;
  d.exact_only = dense ? 1 : s->exact_only;
  d.scale_log2 = (float)((double)s->scale * 1.4426950408889634);
  d.nwords = ceil_div(d.cap, 32);
  d.fbar_extra = 0;
  d.fbar_ticks = kBarrierTicks;
  {
    // clusters per scan block: a multiple of its 16 waves, grown until the
    // grid is about two blocks per CU, so each block's LUT copy into LDS is
    // amortised over more codes when there are many (b, h)
    const long long total = (long long)d.B * d.Hkv * d.L;
    const long long per_wave = (total + kScanWaves * 512LL - 1) / (kScanWaves * 512LL);
    d.scan_lists = kScanWaves * (int)(per_wave < 1 ? 1 : per_wave);
    d.scan_blocks = ceil_div(d.L, d.scan_lists);
  }
  d.collect_slices = ceil_div(d.cap, kCollectEntries);
  d.upload_chunks = ceil_div(d.cap, kUploadChunk);
  if (dense) {
    // about two blocks per CU in all (a multiple of 8 splits per (b, h), so
    // that a head's blocks share an XCD), at least kDenseMinRows rows per
    // split and at most 1024 partials per query head
    const int BH = d.B * d.Hkv;
    int splits = (ceil_div(kDenseBlocks, BH) + 7) / 8 * 8;
    splits = std::min(splits, std::max(1, ceil_div(d.cap, kDenseMinRows)));
    d.n_exact_splits = std::max(1, std::min(splits, 1024));
    d.n_bg_splits = 0;
  } else {
    const long long rows_est = (long long)s->n_sink + s->n_recent + max_selected(s) + 512;
    // split counts are rounded up to multiples of 8 so that the blocks of one
    // (b, h) can all be placed on one XCD
    d.n_exact_splits = std::min(512, std::max(1, ceil_div(rows_est, kExactRowsPerSplit)));
    d.n_exact_splits = (d.n_exact_splits + 7) / 8 * 8;
    // clusters per background wave: batches of 4, at most 256 blocks per (b, h)
    d.bg_per_wave = kBgBatch * std::max(1, ceil_div(d.L, kBgWaves * kBgBatch * 256));
    d.n_bg_splits = ceil_div(d.L, kBgWaves * d.bg_per_wave);
    d.n_bg_splits = (d.n_bg_splits + 7) / 8 * 8;
  }
  d.n_parts = d.n_exact_splits + d.n_bg_splits;
  return d;
}

struct IndexLayout {
  size_t centroids, codebooks, list_off, codes, pos, ent_list, means, n_indexed, dropped, total;
};

IndexLayout index_layout(const Dims& d) {
  IndexLayout l;
  const size_t BH = (size_t)d.B * d.Hkv;
  size_t o = 0;
  l.centroids = o; o = align_up(o + BH * d.L * kD * sizeof(float));
  l.codebooks = o; o = align_up(o + BH * kM * kKsub * kDsub * sizeof(float));
  l.list_off = o;  o = align_up(o + BH * (d.L + 1) * sizeof(int32_t));
  l.codes = o;     o = align_up(o + BH * d.cap * kM);
  l.pos = o;       o = align_up(o + BH * d.cap * sizeof(int32_t));
  l.ent_list = o;  o = align_up(o + BH * d.cap * sizeof(int32_t));
  l.means = o;     o = align_up(o + BH * d.L * kD * sizeof(float));
  l.n_indexed = o; o = align_up(o + (size_t)d.B * sizeof(int32_t));
  l.dropped = o;   o = align_up(o + sizeof(unsigned long long));
  l.total = o;
  return l;
}

struct WsLayout {
  size_t lut, qc, keys, bins, hist, seg_above, seg_aw, seg_tie, seg_w, seg_cnt, wsel, rows, n_rows,
      fsync, fflags, fcnt, fpart, partials, total;
};

WsLayout ws_layout(const Dims& d, bool dense) {
  WsLayout l;
  memset(&l, 0, sizeof(l));
  const size_t BH = (size_t)d.B * d.Hkv;
  size_t o = 0;
  if (!dense) {
    l.lut = o;        o = align_up(o + BH * kM * kKsub * d.G * sizeof(float));
    l.qc = o;         o = align_up(o + BH * d.L * d.G * sizeof(float));
    l.keys = o;       o = align_up(o + BH * d.cap * sizeof(uint32_t));
    l.bins = o;       o = align_up(o + BH * d.L * d.G * 2 * sizeof(float));
    l.hist = o;       o = align_up(o + BH * kHistBins * sizeof(uint32_t));
    l.seg_above = o;  o = align_up(o + BH * d.cap * sizeof(int2));
    l.seg_aw = o;     o = align_up(o + BH * d.cap * d.G * sizeof(float));
    l.seg_tie = o;    o = align_up(o + BH * d.cap * sizeof(uint4));
    l.seg_w = o;      o = align_up(o + BH * d.cap * d.G * sizeof(float));
    l.seg_cnt = o;    o = align_up(o + BH * d.collect_slices * 2 * sizeof(int32_t));
    l.wsel = o;       o = align_up(o + BH * d.L * d.G * sizeof(unsigned long long));
    l.rows = o;       o = align_up(o + BH * d.cap * sizeof(int32_t));
    l.n_rows = o;     o = align_up(o + BH * sizeof(int32_t));
    l.fsync = o;      o = align_up(o + BH * 3 * kSyncStride * sizeof(uint32_t));
    l.fflags = o;     o = align_up(o + sizeof(uint32_t));
    l.fcnt = o;       o = align_up(o + BH * kMaxFusedP * sizeof(unsigned long long));
    l.fpart = o;      o = align_up(o + BH * d.G * kMaxFusedP * kPart * sizeof(float));
  }
  l.partials = o;     o = align_up(o + (size_t)d.B * d.Hq * d.n_parts * kPart * sizeof(float));
  l.total = o;
  return l;
}

size_t upload_ws_bytes(const Dims& d) {
  return align_up((size_t)d.B * d.Hkv * d.upload_chunks * d.L * sizeof(int32_t));
}

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
    w.fpart = reinterpret_cast<float*>(p + l.fpart);
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
                      bool staged, bool barrier_test, hipEvent_t* evs, int* n_kernels,
                      hipStream_t stream) {
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
  if (barrier_test && fP == 0) return PQHSA_ERR_UNSUPPORTED;
  if (fP > 0) {
    // the whole step in one kernel
    a.d.fP = fP;
    a.d.fcpb = ceil_div(d.L, fP);
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

struct AppendWs {
  size_t old_off, shift, codes, pos, list, best, total;
};

AppendWs append_ws(const Dims& d) {
  const size_t BH = (size_t)d.B * d.Hkv;
  AppendWs w;
  size_t o = 0;
  w.old_off = o; o = align_up(o + BH * (d.L + 1) * sizeof(int32_t));
  w.shift = o;   o = align_up(o + BH * (d.L + 1) * sizeof(int32_t));
  w.codes = o;   o = align_up(o + BH * d.cap * kM);
  w.pos = o;     o = align_up(o + BH * d.cap * sizeof(int32_t));
  w.list = o;    o = align_up(o + BH * d.cap * sizeof(int32_t));
  w.best = o;    o = align_up(o + BH * d.cap * sizeof(unsigned long long));
  w.total = o;
  return w;
}

// Query reuse: the rings (caller-owned, persistent across steps) and the
// step's workspace (split-K partials plus one reused state per query head,
// then the search candidates).
struct ReuseLayout {
  size_t qs, st, tj, cnt, total;
};

ReuseLayout reuse_layout(const Dims& d, int W) {
  ReuseLayout l;
  const size_t BQ = (size_t)d.B * d.Hq;
  size_t o = 0;
  l.qs = o;  o = align_up(o + BQ * W * kD * sizeof(uint16_t));
  l.st = o;  o = align_up(o + BQ * W * kPart * sizeof(float));
  l.tj = o;  o = align_up(o + BQ * W * sizeof(int32_t));
  l.cnt = o; o = align_up(o + BQ * sizeof(int32_t));
  l.total = o;
  return l;
}

int reuse_slabs(int W) { return ceil_div(W, kReuseSlab); }

Dims reuse_dims(const pqhsa_shape* s) {
  Dims d = make_dims(s, true);
  d.n_parts = d.n_exact_splits + 1;
  return d;
}

struct ReuseWs {
  size_t partials, cand, n_merge, total;
};

ReuseWs reuse_ws(const Dims& d, int W) {
  ReuseWs w;
  size_t o = 0;
  w.partials = o; o = align_up(o + (size_t)d.B * d.Hq * d.n_parts * kPart * sizeof(float));
  w.cand = o;     o = align_up(o + (size_t)d.B * d.Hq * reuse_slabs(W) * sizeof(int4));
  w.n_merge = o;  o = align_up(o + (size_t)d.B * d.Hkv * sizeof(int32_t));
  w.total = o;
  return w;
}

bool reuse_window_ok(int W) { return W >= 1 && W <= kReuseMaxWindow; }

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

size_t pqhsa_index_bytes(const pqhsa_shape* shape) {
  if (validate(shape, false) != PQHSA_OK) return 0;
  return index_layout(make_dims(shape, false)).total;
}

size_t pqhsa_upload_workspace_bytes(const pqhsa_shape* shape) {
  if (validate(shape, false) != PQHSA_OK) return 0;
  return upload_ws_bytes(make_dims(shape, false));
}

size_t pqhsa_workspace_bytes(const pqhsa_shape* shape, int dense) {
  if (validate(shape, dense != 0) != PQHSA_OK) return 0;
  return ws_layout(make_dims(shape, dense != 0), dense != 0).total;
}

int32_t pqhsa_max_selected(const pqhsa_shape* shape) {
  if (validate(shape, false) != PQHSA_OK) return 0;
  return max_selected(shape);
}

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

size_t pqhsa_append_workspace_bytes(const pqhsa_shape* shape) {
  if (validate(shape, false) != PQHSA_OK) return 0;
  return append_ws(make_dims(shape, false)).total;
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
                  selected, lse, workspace, workspace_bytes, false, false, nullptr, nullptr,
                  stream);
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
  const size_t hist_bytes = (size_t)d.B * d.Hkv * kHistBins * sizeof(uint32_t);
  const size_t ctr_bytes = l.fpart - l.fsync;
  const size_t n16 = (hist_bytes + ctr_bytes) / 16;
  const int blocks = (int)std::min<size_t>(1024, (n16 + 255) / 256);
  hipLaunchKernelGGL(k_zero2, dim3(blocks), dim3(256), 0, stream,
                     reinterpret_cast<uint4*>(ws + l.hist), hist_bytes / 16,
                     reinterpret_cast<uint4*>(ws + l.fsync), ctr_bytes / 16);
  PQHSA_TRY(hip_status(hipGetLastError()));
  return run_step(shape, index_buf, q, k_cache, v_cache, block_table, context_lens, out,
                  selected, lse, ws, kScratchBytes, false, false, nullptr, nullptr, stream);
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
      st = run_step(shape, index_buf, q, k_cache, v_cache, block_table, context_lens, out,
                    selected, lse, workspace, workspace_bytes, variant == PQHSA_VARIANT_STAGED,
                    variant == PQHSA_VARIANT_BARRIER_TEST, events, &nk, stream);
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

pqhsa_status pqhsa_workspace_layout(const pqhsa_shape* shape, int dense, pqhsa_ws_layout* out) {
  PQHSA_TRY(validate(shape, dense != 0));
  if (!out) return PQHSA_ERR_INVALID_ARG;
  const Dims d = make_dims(shape, dense != 0);
  const WsLayout l = ws_layout(d, dense != 0);
  out->lut = l.lut; out->qc = l.qc; out->keys = l.keys; out->bins = l.bins;
  out->rows = l.rows; out->n_rows = l.n_rows; out->partials = l.partials;
  out->flags = l.fflags;
  out->n_exact_splits = d.n_exact_splits;
  out->n_bg_splits = d.n_bg_splits;
  out->n_parts = d.n_parts;
  out->hist = l.hist;
  out->hist_bytes = dense ? 0 : (size_t)d.B * d.Hkv * kHistBins * sizeof(uint32_t);
  out->counters = l.fsync;
  out->counters_bytes = dense ? 0 : l.fpart - l.fsync;
  out->total = l.total;
  return PQHSA_OK;
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
                                        (size_t)d.B * d.Hkv * kHistBins * sizeof(uint32_t),
                                        stream)));
    PQHSA_TRY(hip_status(hipMemsetAsync(ws + l.fsync, 0, l.fpart - l.fsync, stream)));
    PQHSA_TRY(hip_status(hipStreamSynchronize(stream)));
  }
  return PQHSA_OK;
}

pqhsa_status pqhsa_index_layout_of(const pqhsa_shape* shape, pqhsa_index_layout* out) {
  PQHSA_TRY(validate(shape, false));
  if (!out) return PQHSA_ERR_INVALID_ARG;
  const IndexLayout l = index_layout(make_dims(shape, false));
  out->centroids = l.centroids; out->codebooks = l.codebooks; out->list_off = l.list_off;
  out->codes = l.codes; out->pos = l.pos; out->means = l.means; out->n_indexed = l.n_indexed;
  out->dropped = l.dropped;
  return PQHSA_OK;
}

size_t pqhsa_reuse_buffer_bytes(const pqhsa_shape* shape, int32_t window) {
  if (validate(shape, true) != PQHSA_OK || !reuse_window_ok(window)) return 0;
  return reuse_layout(reuse_dims(shape), window).total;
}

size_t pqhsa_reuse_workspace_bytes(const pqhsa_shape* shape, int32_t window) {
  if (validate(shape, true) != PQHSA_OK || !reuse_window_ok(window)) return 0;
  return reuse_ws(reuse_dims(shape), window).total;
}

pqhsa_status pqhsa_reuse_layout_of(const pqhsa_shape* shape, int32_t window,
                                   pqhsa_reuse_layout* out) {
  PQHSA_TRY(validate(shape, true));
  if (!reuse_window_ok(window) || !out) return PQHSA_ERR_INVALID_ARG;
  const ReuseLayout l = reuse_layout(reuse_dims(shape), window);
  out->search = l.qs; out->states = l.st; out->context = l.tj; out->count = l.cnt;
  out->total = l.total;
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

const char* pqhsa_status_string(pqhsa_status status) {
  switch (status) {
    case PQHSA_OK: return "ok";
    case PQHSA_ERR_INVALID_ARG: return "invalid argument";
    case PQHSA_ERR_UNSUPPORTED: return "unsupported shape";
    case PQHSA_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case PQHSA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

}  // extern "C"
