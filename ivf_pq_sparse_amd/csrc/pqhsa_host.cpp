// Host logic of libpqhsa that needs no GPU (see pqhsa_host.hpp) and the C ABI
// entry points made of it alone: buffer sizes, layouts, status strings.
#include "pqhsa_host.hpp"

#include <math.h>
#include <string.h>

#include <algorithm>

namespace pqhsa {

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
    l.hist = o;       o = align_up(o + BH * kHistStride * sizeof(uint32_t));
    l.seg_above = o;  o = align_up(o + BH * d.cap * 2 * sizeof(int32_t));
    l.seg_aw = o;     o = align_up(o + BH * d.cap * d.G * sizeof(float));
    l.seg_tie = o;    o = align_up(o + BH * d.cap * 4 * sizeof(uint32_t));
    l.seg_w = o;      o = align_up(o + BH * d.cap * d.G * sizeof(float));
    l.seg_cnt = o;    o = align_up(o + BH * d.collect_slices * 2 * sizeof(int32_t));
    l.wsel = o;       o = align_up(o + BH * d.L * d.G * sizeof(unsigned long long));
    l.rows = o;       o = align_up(o + BH * d.cap * sizeof(int32_t));
    l.n_rows = o;     o = align_up(o + BH * sizeof(int32_t));
    l.fsync = o;      o = align_up(o + BH * 3 * kSyncStride * sizeof(uint32_t));
    l.fflags = o;     o = align_up(o + sizeof(uint32_t));
    l.fcnt = o;       o = align_up(o + BH * kMaxFusedP * sizeof(unsigned long long));
    // the fused step's partials: at G = 8 a 64-bit word per value (value and
    // tag), else a float
    l.fpart = o;
    o = align_up(o + BH * d.G * kMaxFusedP * kPart * (d.G == 8 ? sizeof(unsigned long long) : sizeof(float)));
  }
  l.partials = o;     o = align_up(o + (size_t)d.B * d.Hq * d.n_parts * kPart * sizeof(float));
  l.total = o;
  return l;
}

size_t upload_ws_bytes(const Dims& d) {
  return align_up((size_t)d.B * d.Hkv * d.upload_chunks * d.L * sizeof(int32_t));
}

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

ReuseWs reuse_ws(const Dims& d, int W) {
  ReuseWs w;
  size_t o = 0;
  w.partials = o; o = align_up(o + (size_t)d.B * d.Hq * d.n_parts * kPart * sizeof(float));
  w.cand = o;     o = align_up(o + (size_t)d.B * d.Hq * reuse_slabs(W) * 4 * sizeof(int32_t));
  w.n_merge = o;  o = align_up(o + (size_t)d.B * d.Hkv * sizeof(int32_t));
  w.total = o;
  return w;
}

bool reuse_window_ok(int W) { return W >= 1 && W <= kReuseMaxWindow; }

}  // namespace pqhsa

using namespace pqhsa;

#define PQHSA_TRY(expr)                         \
  do {                                          \
    pqhsa_status s_ = (expr);                   \
    if (s_ != PQHSA_OK) return s_;              \
  } while (0)

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

size_t pqhsa_append_workspace_bytes(const pqhsa_shape* shape) {
  if (validate(shape, false) != PQHSA_OK) return 0;
  return append_ws(make_dims(shape, false)).total;
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
  out->hist_bytes = dense ? 0 : (size_t)d.B * d.Hkv * kHistStride * sizeof(uint32_t);
  out->counters = l.fsync;
  out->counters_bytes = dense ? 0 : l.fpart - l.fsync;
  out->total = l.total;
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
