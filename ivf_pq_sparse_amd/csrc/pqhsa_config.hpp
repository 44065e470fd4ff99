// Sizes and shape-derived constants of libpqhsa, shared by the kernels and
// the host code that validates shapes and lays out buffers.  Plain C++ (no
// HIP), so that the host logic also builds with a host compiler alone.
// Not part of the ABI.
#pragma once

#include <stdint.h>

namespace pqhsa {

constexpr int kD = 128;          // head_dim
constexpr int kPage = 16;        // tokens per cache page
constexpr int kM = 16;           // PQ subspaces
constexpr int kKsub = 256;       // codewords per subspace
constexpr int kDsub = 8;         // dims per subspace
constexpr int kHistBits = 12;    // top bits of a key used by the first selection pass
constexpr int kHistBins = 1 << kHistBits;
// uint32s between two heads' histograms in the workspace: 4096 bins and 4 KB
// of padding, so that the heads' hot top bins (every block of a head adds to
// them and reads them back) do not fall on the same memory channels; with a
// 16 KB stride the 128K step was 0.3-1.7 us slower depending on where the
// workspace happened to lie
constexpr int kHistStride = kHistBins + 1024;
constexpr int kPart = 132;       // floats per partial: m (base 2), l, pad, pad, acc[128]
constexpr int kMaxLists = 16384;
constexpr int kScanThreads = 1024;
constexpr int kScanWaves = kScanThreads / 64;
constexpr int kScanPrefetch = 4;         // 64-entry tiles in flight per wave
constexpr int kCollectThreads = 256;
constexpr int kCollectPerThread = 16;
constexpr int kCollectEntries = kCollectThreads * kCollectPerThread;  // entries per collect block
constexpr int kSelectThreads = 512;
constexpr int kMaxSparseContext = 1 << 20;  // position bitmap of the selection lives in LDS
constexpr int kExactRowsPerSplit = 64;  // target rows per split-K block (index-list mode)
constexpr int kDenseBlocks = 512;       // dense mode: split-K blocks to aim for in all
constexpr int kDenseMinRows = 64;       // dense mode: fewest rows per split
constexpr int kPhaseRows = 256;         // rows whose cache offsets are staged in LDS at once
constexpr int kBgWaves = 4;             // waves per background block
constexpr int kBgBatch = 4;             // clusters whose loads a background wave issues together
constexpr int kUploadChunk = 4096;      // tokens per counting-sort chunk
constexpr int kMaxFusedP = 64;          // fused step: at most this many blocks per (b, h)
constexpr int kSyncStride = 32;         // uint32s between fused-step counters (128 B)
constexpr int kFusedWselMax = 1024;     // fused step: clusters per block x G held in LDS
constexpr int kReuseSlab = 128;         // ring slots per search block
constexpr int kReuseMinRows = 64;       // query reuse: fewest rows per split-K block
constexpr int kReuseMaxWindow = 64 * kReuseSlab;   // slabs of a ring fit one wave
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kFixScale = 1099511627776.0f;   // 2^40: fixed-point unit of selected weights
constexpr float kFixInv = 1.0f / 1099511627776.0f;

// Shape-derived sizes, passed to every kernel by value.
struct Dims {
  int B, Hq, Hkv, G, L, num_pages, max_pages, cap;
  int n_sink, n_recent, budget_bp;
  int exact_only;             // 1: no background term
  float scale_log2;           // scale * log2(e): logits are kept in base 2
  int nwords;                 // ceil(cap / 32): words of a per-head bitmap
  int scan_blocks;            // scan blocks per (b, h)
  int scan_lists;             // clusters per scan block (a multiple of its 16 waves)
  int collect_slices;         // collect blocks per (b, h)
  int n_exact_splits;         // split-K blocks per (b, h)
  int n_bg_splits;            // background blocks per (b, h)
  int bg_per_wave;            // clusters per background wave (a multiple of 4)
  int n_parts;                // partials per (b, q head)
  int upload_chunks;          // counting-sort chunks per (b, h)
  int fP;                     // fused step: blocks per (b, h) (0: the staged kernels run)
  int fcpb;                   // fused step: clusters per block
  int fbar_extra;             // fused step: arrivals a barrier waits for beyond its P blocks
                              //   (0; 1 only in the barrier test, so that every wait runs out)
  unsigned int fbar_ticks;    // fused step: bound of a barrier wait in ticks of the 100 MHz clock
  int fkeys_out;              // fused step: also write the 16-bit keys to the workspace
                              //   (always done where a block's keys exceed its LDS key cache)
};

constexpr unsigned int kBarrierTicks = 200000000u;   // 2 s: the fused step's default wait bound
constexpr unsigned int kBarrierTestTicks = 2000u;    // 20 us: the barrier test's wait bound

}  // namespace pqhsa
