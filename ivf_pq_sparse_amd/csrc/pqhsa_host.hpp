// Host logic of libpqhsa that needs no GPU: shape validation, the derived
// sizes and the layouts of the index, workspace and reuse buffers.  Plain
// C++, built into the library with the kernels and, for the sanitizer test,
// on its own with a host compiler.  Not part of the ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "pqhsa.h"
#include "pqhsa_config.hpp"

namespace pqhsa {

constexpr size_t kAlign = 256;           // alignment of every array in a buffer
constexpr int kMaxContextLimit = 1 << 26;

// Byte offsets of the arrays in the index, workspace and append workspace.
struct IndexLayout {
  size_t centroids, codebooks, list_off, codes, pos, ent_list, means, n_indexed, dropped, total;
};

struct WsLayout {
  size_t lut, qc, keys, bins, hist, seg_above, seg_aw, seg_tie, seg_w, seg_cnt, wsel, rows, n_rows,
      fsync, fflags, fcnt, fpart, partials, total;
};

struct AppendWs {
  size_t old_off, shift, codes, pos, list, best, total;
};

// Query reuse: the rings (caller-owned, persistent across steps) and the
// step's workspace (split-K partials plus one reused state per query head,
// then the search candidates).
struct ReuseLayout {
  size_t qs, st, tj, cnt, total;
};

struct ReuseWs {
  size_t partials, cand, n_merge, total;
};

size_t align_up(size_t x);
int ceil_div(long long a, long long b);
pqhsa_status validate(const pqhsa_shape* s, bool dense);
int max_selected(const pqhsa_shape* s);
Dims make_dims(const pqhsa_shape* s, bool dense);
IndexLayout index_layout(const Dims& d);
WsLayout ws_layout(const Dims& d, bool dense);
size_t upload_ws_bytes(const Dims& d);
AppendWs append_ws(const Dims& d);
ReuseLayout reuse_layout(const Dims& d, int W);
int reuse_slabs(int W);
Dims reuse_dims(const pqhsa_shape* s);
ReuseWs reuse_ws(const Dims& d, int W);
bool reuse_window_ok(int W);

}  // namespace pqhsa
