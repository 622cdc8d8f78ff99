// Host-side launch descriptions shared by the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

namespace dsaidx {

enum SourceKind { SRC_DENSE = 1, SRC_PAGED = 2, SRC_SPARSE = 3, SRC_PAGED_SPARSE = 4 };

// Per-device state (error word, CU count, occupancy, kernel attributes) is kept for
// device ids below this.
constexpr int kMaxDevices = 64;
enum KeyFmt { FMT_BF16 = 1, FMT_FP8 = 2, FMT_MXFP4 = 3 };

// A host-side set-up step run once per device (the current one when first needed), e.g. a
// kernel attribute; its result is kept per device. Thread-safe.
struct PerDeviceOnce {
  std::mutex mu;
  bool done[kMaxDevices] = {};
  hipError_t res[kMaxDevices] = {};
  template <class F>
  hipError_t run(F&& f) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!done[dev]) {
      res[dev] = f();
      done[dev] = true;
    }
    return res[dev];
  }
};

// idx_select's one-pass selection for rows that read their own keys (the balanced scan).
// A scan workgroup keeps the scores of its step range in LDS and builds, per row it
// meets, a histogram of the largest order key of each group of 2^gshift columns. The
// k-th largest group maximum of a row is a value that at least k entries reach, so the
// entries at or above it (the survivors) hold the row's top k. A row inside one workgroup
// is cut at once; the two rows a workgroup may share with its neighbours (its first and
// last) are cut once every workgroup of the row has published its histogram; a shared
// part may first be filtered at a lower speculative cut of its own while the row's cut is
// summed up (and again at the row's cut when that comes out lower). Each workgroup
// writes its survivors to its own region; a finish kernel selects exactly among them.
constexpr int kSelFineBins = 4096;    // histogram of the top 12 bits of the order key
constexpr int kSelCoarseBins = 256;   // and of its top 8 bits (16 fine bins each)
constexpr int kSelSlotWords = kSelFineBins / 2 + kSelCoarseBins;  // 16-bit fine counts in pairs, coarse
constexpr int kSelMaxBlocks = 1024;   // workgroups of a one-pass scan launch
constexpr int kSelMaxSpan = 32;       // workgroups a row may span and still be cut
constexpr uint32_t kSegNoCut = 0x80000000u;  // segment record: every entry was kept
struct SelectState {
  uint32_t* slots;               // [kSelMaxBlocks, 2, kSelSlotWords]: histogram of a workgroup's
                                 // first (0) and last (1) row when shared with other workgroups
  unsigned long long* arrive;    // [rows] workgroups done with the row (counts up, never cleared)
  int64_t* acc;                  // [rows + 1] first step of each row in the call's step order
  uint4* seg;                    // [steps] at a segment's first step: x = survivors, | kSegNoCut
                                 // when the segment kept every entry; y = its cut (the order key
                                 // every survivor reaches); z = the largest survivor's order key;
                                 // w = the row's cut as this segment found it (1: none), which
                                 // every entry of the row's top k reaches
  uint64_t* surv;                // [steps, 64] survivor keys from the segment's first step on
  float* spill;                  // [rows, ld] scores of ranges that do not fit in LDS
  int k;
  int gshift;                    // group size 2^gshift columns, 0..4
  int cutoff;                    // 0: every scored entry survives
  int64_t wait_ticks;            // limit of a row wait (100 MHz clock)
};

// One scoring call, validated by the C-ABI layer.
struct ScoreCall {
  int source;  // SourceKind
  int fmt;     // KeyFmt
  int rows;
  const uint8_t* q;
  const float* w;
  const uint8_t* k;       // dense / sparse: key rows; paged: pages
  const void* k_scale;
  int64_t n_keys;         // dense / sparse: key rows; paged: pages
  const int32_t* row_ks;  // dense / sparse
  const int32_t* row_ke;
  int page_size;          // paged
  const int32_t* block_table;
  int64_t bt_rows;
  int64_t bt_ld;
  const int32_t* seq_lens;
  const int32_t* row_req;
  const int32_t* cand;    // sparse and paged sparse
  int64_t cand_ld;
  const int32_t* n_cols;
  int block;
  float* logits;
  int64_t ld;
  unsigned* err;          // device error word (may be null)
  int skip_tail;          // 1: columns past a row's scored length stay unwritten (their
                          // reader knows the lengths); 0: they are set to -inf
  uint32_t* zero;         // optional: words the kernel sets to 0 (a following top-k's
  int64_t zero_words;     // histogram and counters)
  const SelectState* sel; // optional: the one-pass selection (balanced scan only)
  int32_t* lens_out;      // optional: each row's scored length (columns a top-k may read)
  int shared_keys;        // dense: 1 when the rows are one prefill chunk's queries over a
                          // shared key array (the tiled kernel may take them)
};

// One top-k call.
struct TopkCall {
  const float* logits;
  int64_t ld;
  int64_t n_cols;
  const int32_t* lens;    // optional: row length
  const int32_t* len_ks;  // optional: row length = len_ke - len_ks
  const int32_t* len_ke;
  int rows;
  int k;
  int32_t* out_idx;
  float* out_val;
  int64_t out_ld;
  int sorted;
  const int32_t* cand;    // optional column -> token map
  int64_t cand_ld;
  int block;
  int ws_zeroed;          // the workspace's zeroed prefix was cleared by the score kernel
};

hipError_t launch_score(const ScoreCall& c, hipStream_t stream);

// Rows up to this count take the balanced scan (and can take the one-pass selection).
constexpr int kBalancedMaxRows = 512;
// Workgroups of the balanced scan launch for this call (the one-pass selection's part
// boundaries depend on it); 0 if the call does not take the balanced scan.
int64_t select_scan_blocks(const ScoreCall& c);
// The finish of the one-pass selection: one workgroup per row selects among the row's
// survivors and writes the row.
hipError_t launch_select_finish(const TopkCall& t, const SelectState& s, int64_t blocks, hipStream_t stream);

// Dense fp8 calls the caller marks as a prefill chunk (shared_keys) with at least this
// many rows run the tiled prefill kernel; fewer rows (too few query tiles to fill the
// chip) and unmarked dense calls run the decode scan.
constexpr int kPrefillMinRows = 256;
bool prefill_applies(const ScoreCall& c);
hipError_t launch_prefill(const ScoreCall& c, hipStream_t stream);
size_t topk_workspace_bytes(int rows, int64_t n_cols);
// Leading bytes of the top-k workspace that must be zero when the top-k starts.
size_t topk_zeroed_bytes(int rows, int64_t n_cols);
hipError_t launch_topk(const TopkCall& c, void* workspace, hipStream_t stream);
// The top-k path launch_topk takes for rows of n_cols columns (for dispatch logging).
const char* topk_path(int rows, int64_t n_cols);
// Rows up to this width take the short-row top-k: one workgroup per row, the row in LDS.
constexpr int kTopkShortRow = 16384;
// Rows up to this width take the one-pass bucket top-k when they fit the compute units.
constexpr int kTopkWideRow = 32768;

// One key-cache write (new bf16 keys quantised into the cache at their slots).
struct KcacheCall {
  const void* k_new;      // bf16 [n_new, 128]
  const int64_t* slots;   // [n_new]; < 0: skip
  int64_t n_new;
  int fmt;                // FMT_FP8 or FMT_MXFP4
  uint8_t* cache;         // fp8 [n_slots, 128] / MXFP4 [n_slots, 64]
  void* scale;            // fp8 float [n_slots] / MXFP4 UE8M0 [n_slots, 4]
  int64_t n_slots;
  unsigned* err;
};
hipError_t launch_kcache_write(const KcacheCall& c, hipStream_t stream);

// One candidate-block publication (the candidate-source step of the two-level indexer).
struct CandCall {
  const float* logits;    // [rows, ld]
  int64_t ld;
  const int32_t* lens;    // optional: row length, clamped to [0, n_cols]
  int64_t n_cols;
  int rows;
  int block;              // tokens per block, a multiple of 64
  int n_top;
  int32_t* cand;          // [rows, cand_ld]
  int64_t cand_ld;
  int32_t* n_cand;        // [rows]
};
// Most blocks one row may have (LDS of the selection workgroup).
constexpr int kCandMaxBlocks = 16384;
size_t cand_workspace_bytes(int rows, int64_t n_cols);
hipError_t launch_candidate_blocks(const CandCall& c, void* workspace, hipStream_t stream);

// One sparse-attention call (attention over each row's selected entries).
struct AttnCall {
  const void* q;          // bf16 [rows, heads, 576]
  const void* kv;         // bf16 [n_pages, page_size, 576]
  int64_t n_pages;
  int page_size;
  const int32_t* block_table;
  int64_t bt_rows;
  int64_t bt_ld;
  const int32_t* seq_lens;
  const int32_t* row_req;
  const int32_t* indices; // [rows, idx_ld] logical positions, -1 skipped
  int64_t idx_ld;
  int k;
  int rows;
  int heads;              // 16, 32, 64 or 128
  float scale;
  float* out;             // [rows, heads, 512]
  float* lse;             // [rows, heads] or null
  unsigned* err;
};
int attn_splits(int rows, int heads, int k);
size_t attn_workspace_bytes(int rows, int heads, int k);
hipError_t launch_sparse_attn(const AttnCall& c, void* workspace, hipStream_t stream);

// Streaming-read probe (measurement aid).
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

// Per-device error word (device address) and compute-unit count.
unsigned* device_error_word();
int device_cu_count();

}  // namespace dsaidx
