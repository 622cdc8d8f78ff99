// C-ABI entry points of dsaidx: argument checks, workspace sizing and dispatch to
// the kernels. Nothing here touches the device before every host-checkable
// argument has passed.
#include "dsaidx.h"
#include "launch.h"
#include "api_internal.h"

#include <cmath>

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <set>
#include <string>

using namespace dsaidx;

namespace {

thread_local std::string g_last_error;

idx_status fail(idx_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

idx_status ok() {
  g_last_error.clear();
  return IDX_OK;
}

// IDX_LOG=1 in the environment: one stderr line per distinct dispatch decision.
bool log_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("IDX_LOG");
    return v && *v && std::strcmp(v, "0") != 0;
  }();
  return on;
}

void log_once(const char* fmt, ...) {
  if (!log_enabled()) return;
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  static std::mutex mu;
  static std::set<std::string> seen;
  std::lock_guard<std::mutex> lock(mu);
  if (seen.insert(buf).second) fprintf(stderr, "[dsaidx] %s\n", buf);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int64_t kMaxCols = 0x7FFFFFFF;
constexpr int kMaxCandBlockSize = 4096;

#define REQUIRE(cond, status, ...) \
  do {                             \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

// Format of the keys, given the dtype pair; -1 if the pair is not supported.
int key_format(int q_dtype, int k_dtype) {
  if (q_dtype == IDX_BF16 && k_dtype == IDX_BF16) return FMT_BF16;
  if (q_dtype == IDX_FP8_E4M3 && k_dtype == IDX_FP8_E4M3) return FMT_FP8;
  if (q_dtype == IDX_FP8_E4M3 && k_dtype == IDX_MXFP4) return FMT_MXFP4;
  return -1;
}

idx_status check_common(const char* fn, const void* q, int q_dtype, const float* w, const void* k,
                        const void* k_scale, int k_dtype, int rows, const float* logits, int64_t ld,
                        int* fmt) {
  REQUIRE(rows >= 0, IDX_ERR_ARG, "%s: rows = %d is negative", fn, rows);
  *fmt = key_format(q_dtype, k_dtype);
  REQUIRE(*fmt > 0, IDX_ERR_UNSUPPORTED,
          "%s: q_dtype %d with k_dtype %d is not supported (bf16/bf16, fp8/fp8 or fp8/mxfp4)", fn,
          q_dtype, k_dtype);
  if (rows == 0) return IDX_OK;
  REQUIRE(q && w && k && logits, IDX_ERR_ARG, "%s: q, w, k and logits must be non-null", fn);
  REQUIRE(*fmt == FMT_BF16 || k_scale, IDX_ERR_ARG, "%s: k_scale is required for fp8 and mxfp4 keys", fn);
  REQUIRE(aligned(q, 16) && aligned(k, 16) && aligned(w, 16), IDX_ERR_ARG,
          "%s: q, k and w must be 16-byte aligned (w is read four weights at a time)", fn);
  REQUIRE(aligned(logits, 4), IDX_ERR_ARG, "%s: logits must be 4-byte aligned", fn);
  REQUIRE(*fmt != FMT_FP8 || aligned(k_scale, 4), IDX_ERR_ARG, "%s: fp8 k_scale must be 4-byte aligned", fn);
  REQUIRE(ld >= 1 && ld <= kMaxCols, IDX_ERR_ARG, "%s: ld = %lld out of range [1, 2^31)", fn, (long long)ld);
  return IDX_OK;
}

idx_status check_ints(const char* fn, std::initializer_list<const int32_t*> ps) {
  for (const int32_t* p : ps) REQUIRE(p == nullptr || aligned(p, 4), IDX_ERR_ARG, "%s: int32 arrays must be 4-byte aligned", fn);
  return IDX_OK;
}

idx_status launched(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(IDX_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

// Checks of a problem for both the score calls and idx_select; fills ``c`` (minus
// the output pointers).
idx_status check_problem(const char* fn, const idx_problem* p, ScoreCall* c, const float* logits,
                         int64_t ld, bool need_out) {
  REQUIRE(p, IDX_ERR_ARG, "%s: problem is null", fn);
  *c = ScoreCall{};
  int fmt = 0;
  idx_status s = check_common(fn, p->q, p->q_dtype, p->w, p->k, p->k_scale, p->k_dtype, p->rows,
                              need_out ? logits : (const float*)p->w, need_out ? ld : 1, &fmt);
  if (s != IDX_OK) return s;
  c->fmt = fmt;
  c->rows = p->rows;
  c->q = (const uint8_t*)p->q;
  c->w = p->w;
  c->k = (const uint8_t*)p->k;
  c->k_scale = p->k_scale;
  c->n_keys = p->n_keys;
  c->logits = (float*)logits;
  c->ld = ld;
  if (p->mode == IDX_MODE_DENSE || p->mode == IDX_MODE_PREFILL) {
    c->source = SRC_DENSE;
    c->shared_keys = p->mode == IDX_MODE_PREFILL ? 1 : 0;
    if (p->rows == 0) return IDX_OK;
    REQUIRE(p->n_keys >= 0, IDX_ERR_ARG, "%s: n_keys is negative", fn);
    REQUIRE(p->row_ks && p->row_ke, IDX_ERR_ARG, "%s: row_ks and row_ke must be non-null", fn);
    c->row_ks = p->row_ks;
    c->row_ke = p->row_ke;
    return check_ints(fn, {p->row_ks, p->row_ke});
  }
  if (p->mode == IDX_MODE_PAGED) {
    c->source = SRC_PAGED;
    REQUIRE(fmt != FMT_BF16, IDX_ERR_UNSUPPORTED, "%s: paged keys must be fp8 or mxfp4", fn);
    REQUIRE(p->page_size >= 64 && p->page_size % 64 == 0, IDX_ERR_UNSUPPORTED,
            "%s: page_size = %d must be a positive multiple of 64", fn, p->page_size);
    if (p->rows == 0) return IDX_OK;
    REQUIRE(p->n_keys >= 1, IDX_ERR_ARG, "%s: n_pages must be >= 1", fn);
    REQUIRE(p->block_table && p->seq_lens, IDX_ERR_ARG, "%s: block_table and seq_lens must be non-null", fn);
    REQUIRE(p->bt_ld >= 1 && p->bt_ld <= kMaxCols / p->page_size, IDX_ERR_ARG,
            "%s: bt_ld = %lld out of range", fn, (long long)p->bt_ld);
    c->page_size = p->page_size;
    c->block_table = p->block_table;
    c->bt_ld = p->bt_ld;
    c->seq_lens = p->seq_lens;
    c->row_req = p->row_req;
    return check_ints(fn, {p->block_table, p->seq_lens, p->row_req});
  }
  if (p->mode == IDX_MODE_SPARSE_BLOCKS) {
    c->source = SRC_SPARSE;
    REQUIRE(fmt != FMT_BF16, IDX_ERR_UNSUPPORTED, "%s: candidate-block keys must be fp8 or mxfp4", fn);
    REQUIRE(p->block_size >= 64 && p->block_size % 64 == 0, IDX_ERR_UNSUPPORTED,
            "%s: block_size = %d must be a positive multiple of 64", fn, p->block_size);
    if (p->rows == 0) return IDX_OK;
    REQUIRE(p->n_keys >= 0, IDX_ERR_ARG, "%s: n_keys is negative", fn);
    REQUIRE(p->row_ks && p->row_ke && p->cand_blocks && p->n_cols, IDX_ERR_ARG,
            "%s: row_ks, row_ke, cand_blocks and n_cols must be non-null", fn);
    REQUIRE(p->cand_ld >= 1 && p->cand_ld <= kMaxCols / p->block_size, IDX_ERR_ARG,
            "%s: cand_ld = %lld out of range", fn, (long long)p->cand_ld);
    c->row_ks = p->row_ks;
    c->row_ke = p->row_ke;
    c->cand = p->cand_blocks;
    c->cand_ld = p->cand_ld;
    c->n_cols = p->n_cols;
    c->block = p->block_size;
    return check_ints(fn, {p->row_ks, p->row_ke, p->cand_blocks, p->n_cols});
  }
  if (p->mode == IDX_MODE_PAGED_SPARSE_BLOCKS) {
    c->source = SRC_PAGED_SPARSE;
    REQUIRE(fmt != FMT_BF16, IDX_ERR_UNSUPPORTED, "%s: paged candidate-block keys must be fp8 or mxfp4", fn);
    REQUIRE(p->page_size >= 64 && p->page_size % 64 == 0, IDX_ERR_UNSUPPORTED,
            "%s: page_size = %d must be a positive multiple of 64", fn, p->page_size);
    REQUIRE(p->block_size >= 64 && p->block_size % 64 == 0, IDX_ERR_UNSUPPORTED,
            "%s: block_size = %d must be a positive multiple of 64", fn, p->block_size);
    REQUIRE(p->page_size % p->block_size == 0, IDX_ERR_UNSUPPORTED,
            "%s: page_size = %d must be a multiple of block_size = %d", fn, p->page_size, p->block_size);
    if (p->rows == 0) return IDX_OK;
    REQUIRE(p->n_keys >= 1, IDX_ERR_ARG, "%s: n_pages must be >= 1", fn);
    REQUIRE(p->block_table && p->seq_lens && p->cand_blocks && p->n_cols, IDX_ERR_ARG,
            "%s: block_table, seq_lens, cand_blocks and n_cols must be non-null", fn);
    REQUIRE(p->bt_ld >= 1 && p->bt_ld <= kMaxCols / p->page_size, IDX_ERR_ARG,
            "%s: bt_ld = %lld out of range", fn, (long long)p->bt_ld);
    REQUIRE(p->cand_ld >= 1 && p->cand_ld <= kMaxCols / p->block_size, IDX_ERR_ARG,
            "%s: cand_ld = %lld out of range", fn, (long long)p->cand_ld);
    c->page_size = p->page_size;
    c->block_table = p->block_table;
    c->bt_ld = p->bt_ld;
    c->seq_lens = p->seq_lens;
    c->row_req = p->row_req;
    c->cand = p->cand_blocks;
    c->cand_ld = p->cand_ld;
    c->n_cols = p->n_cols;
    c->block = p->block_size;
    return check_ints(fn, {p->block_table, p->seq_lens, p->row_req, p->cand_blocks, p->n_cols});
  }
  return fail(IDX_ERR_ARG, "%s: unknown mode %d", fn, p->mode);
}

// Width of the score matrix idx_select builds for a problem.
int64_t select_width(const idx_problem* p) {
  switch (p->mode) {
    case IDX_MODE_DENSE:
    case IDX_MODE_PREFILL: return p->max_cols;
    case IDX_MODE_PAGED: return p->bt_ld * p->page_size;
    case IDX_MODE_SPARSE_BLOCKS:
    case IDX_MODE_PAGED_SPARSE_BLOCKS: return p->cand_ld * p->block_size;
  }
  return 0;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// idx_select workspace. Two layouts, the larger one sized:
//  - one-pass selection (rows that read their own keys, kSelMinRows..kBalancedMaxRows rows):
//    the histogram slots, arrival counters, row step offsets, segment records and survivor
//    regions of SelectState, then the spill score rows [rows, ldw];
//  - scores then top-k (prefill chunks, more rows): the score matrix [rows, ldw], the
//    rows' scored lengths, then the top-k workspace.
// Every region starts on a 256-byte boundary; ldw = width rounded up to 64 columns.
struct SelectLayout {
  size_t slots, arrive, acc, seg, surv, spill, total;
};

SelectLayout select_layout(const idx_problem* p) {
  const int64_t R = p->rows, ldw = round_up(select_width(p), 64), steps = R * (ldw / 64);
  SelectLayout L{};
  size_t o = 0;
  auto take = [&](int64_t bytes) {
    const size_t at = o;
    o += (size_t)round_up(bytes, 256);
    return at;
  };
  L.slots = take((int64_t)kSelMaxBlocks * 2 * kSelSlotWords * 4);
  L.arrive = take(R * 8);
  L.acc = take((R + 1) * 8);
  L.seg = take(steps * 16);
  L.surv = take(steps * 64 * 8);
  L.spill = take(R * ldw * 4);
  L.total = o;
  return L;
}

size_t select_scores_bytes(const idx_problem* p) {
  return (size_t)round_up((int64_t)p->rows * round_up(select_width(p), 64) * (int64_t)sizeof(float), 256);
}

size_t select_lens_bytes(const idx_problem* p) { return (size_t)round_up((int64_t)p->rows * 4, 256); }

// Whether the problem takes the one-pass selection (the balanced scan of rows that read
// their own keys); the launch must also fit the finish's segment table (checked per call).
// Fewer rows than this take scores then top-k: each row would span more than
// kSelMaxSpan of the CUs' workgroups, too many to exchange histograms between. Rows of
// up to kTopkShortRow columns also take scores then top-k: their one-workgroup-per-row
// top-k costs less than the one-pass epilogue and finish (two-level 64 x 8192: 31
// against 37 us), and so do rows of up to kTopkWideRow columns when there are at most
// kSelTwoPassRows of them (batched decode R x 32768, scores then top-k against one
// pass: R = 16 31.9 / 35.8 us, 32 42.6 / 43.8, 64 64.1 / 62.5, 128 106.4 / 104.3).
// Wider rows take the one pass: 256 x 32768 180 against 185 us, the 128K paged decode
// 153 against 172 us.
constexpr int kSelMinRows = 8;
constexpr int kSelTwoPassRows = 32;

// The shapes the one-pass selection can run at all (the workspace covers both layouts).
bool select_one_pass_possible(const idx_problem* p) {
  if (p->rows < kSelMinRows || p->rows > kBalancedMaxRows) return false;
  if (p->mode == IDX_MODE_PREFILL && p->q_dtype == IDX_FP8_E4M3 && p->k_dtype == IDX_FP8_E4M3 &&
      p->rows >= kPrefillMinRows)
    return false;  // a prefill chunk: the tiled prefill kernel, then the top-k
  return true;
}

// The shapes that take it by default (IDX_SELECT_ONE_PASS: every possible one).
bool select_one_pass_shape(const idx_problem* p, uint32_t flags) {
  if (!select_one_pass_possible(p)) return false;
  const int64_t w = select_width(p);
  return (flags & IDX_SELECT_ONE_PASS) || (w > kTopkShortRow && !(w <= kTopkWideRow && p->rows <= kSelTwoPassRows));
}

// Group size of the one-pass cutoff: 16 columns, halved while a row of the call's width
// would have fewer than 4k groups (the cutoff is the k-th largest group maximum).
int select_group_shift(int64_t width, int k) {
  int gs = 4;
  while (gs > 0 && (width >> gs) < 4 * (int64_t)k) --gs;
  return gs;
}

// Limit of a row wait (the device's 100 MHz real-time clock): far beyond the few
// microseconds the waves of a row finish apart.
constexpr int64_t kSelectWaitTicks = 200000;


}  // namespace

namespace dsaidx {

idx_status api_fail(idx_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

idx_status select_call(const char* fn, const idx_problem* p, int k, int32_t* out_idx, float* out_val,
                       int64_t out_ld, uint32_t flags, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  REQUIRE(p, IDX_ERR_ARG, "%s: problem is null", fn);
  REQUIRE(k >= 1 && k <= IDX_MAX_K, IDX_ERR_UNSUPPORTED, "%s: k = %d outside [1, %d]", fn, k, IDX_MAX_K);
  REQUIRE((flags & ~(IDX_TOPK_UNSORTED | IDX_SELECT_NO_CUTOFF | IDX_SELECT_ONE_PASS)) == 0, IDX_ERR_ARG,
          "%s: unknown flags 0x%x", fn, flags);
  REQUIRE(p->rows >= 0, IDX_ERR_ARG, "%s: rows = %d is negative", fn, p->rows);
  const int64_t width = select_width(p);
  ScoreCall c;
  {
    // validate the problem with a stand-in output so the score checks run
    idx_status s = check_problem(fn, p, &c, (const float*)p->w, 1, false);
    if (s != IDX_OK) return s;
  }
  if (p->rows == 0) return ok();
  REQUIRE(width >= 1 && width <= kMaxCols, IDX_ERR_ARG,
          "%s: score width %lld out of range (dense problems need max_cols >= 1)", fn, (long long)width);
  REQUIRE(out_idx && out_ld >= k, IDX_ERR_ARG, "%s: out_idx must be non-null and out_ld >= k", fn);
  REQUIRE(aligned(out_idx, 4) && (!out_val || aligned(out_val, 4)), IDX_ERR_ARG,
          "%s: outputs must be 4-byte aligned", fn);
  if (p->mode == IDX_MODE_PAGED || p->mode == IDX_MODE_PAGED_SPARSE_BLOCKS)
    REQUIRE(p->bt_rows >= 1 && (p->row_req || p->bt_rows >= p->rows), IDX_ERR_ARG,
            "%s: bt_rows = %lld too small", fn, (long long)p->bt_rows);
  const size_t need = idx_select_workspace(p, k);
  REQUIRE(workspace && workspace_bytes >= need, IDX_ERR_WORKSPACE,
          "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace ? workspace_bytes : (size_t)0);
  REQUIRE(aligned(workspace, 256), IDX_ERR_ARG, "%s: workspace must be 256-byte aligned", fn);

  const int64_t ldw = round_up(width, 64);
  uint8_t* ws = (uint8_t*)workspace;
  c.ld = ldw;
  c.bt_rows = p->bt_rows;
  c.err = device_error_word();
  c.skip_tail = 1;  // the top-k below reads each row only up to its scored length

  TopkCall t{};
  t.ld = ldw;
  t.n_cols = width;
  t.rows = p->rows;
  t.k = k;
  t.out_idx = out_idx;
  t.out_val = out_val;
  t.out_ld = out_ld;
  t.sorted = (flags & IDX_TOPK_UNSORTED) ? 0 : 1;
  if (p->mode == IDX_MODE_SPARSE_BLOCKS || p->mode == IDX_MODE_PAGED_SPARSE_BLOCKS) {
    t.cand = p->cand_blocks;
    t.cand_ld = p->cand_ld;
    t.block = p->block_size;
  }

  const int64_t blocks = select_one_pass_shape(p, flags) ? select_scan_blocks(c) : 0;
  if (blocks >= 1 && blocks <= kSelMaxBlocks) {
    const SelectLayout L = select_layout(p);
    SelectState st{};
    st.slots = (uint32_t*)(ws + L.slots);
    st.arrive = (unsigned long long*)(ws + L.arrive);
    st.acc = (int64_t*)(ws + L.acc);
    st.seg = (uint4*)(ws + L.seg);
    st.surv = (uint64_t*)(ws + L.surv);
    st.spill = (float*)(ws + L.spill);
    st.k = k;
    st.gshift = select_group_shift(ldw, k);
    st.cutoff = (flags & IDX_SELECT_NO_CUTOFF) ? 0 : 1;
    st.wait_ticks = kSelectWaitTicks;
    c.logits = st.spill;
    c.sel = &st;
    log_once("idx_select: one pass (rows %d, width %lld, k %d, groups of %d, %lld scan workgroups)", p->rows,
             (long long)width, k, 1 << st.gshift, (long long)blocks);
    hipError_t e = launch_score(c, stream);
    if (e != hipSuccess) return launched(fn, e);
    return launched(fn, launch_select_finish(t, st, blocks, stream));
  }

  // scores to the workspace, then the top-k over each row's scored length
  float* scores = (float*)ws;
  int32_t* lens = (int32_t*)(ws + select_scores_bytes(p));
  uint8_t* topk_ws = ws + select_scores_bytes(p) + select_lens_bytes(p);
  c.logits = scores;
  c.lens_out = lens;
  // the scan kernels clear the top-k's histogram and counters on their way
  const bool prefill = prefill_applies(c);
  if (!prefill) {
    c.zero = (uint32_t*)topk_ws;
    c.zero_words = (int64_t)(topk_zeroed_bytes(p->rows, width) / 4);
  }
  log_once("idx_select: %s then top-k, %s (rows %d, width %lld, k %d)", prefill ? "prefill tiles" : "scan",
           topk_path(p->rows, width), p->rows, (long long)width, k);
  hipError_t e = launch_score(c, stream);
  if (e != hipSuccess) return launched(fn, e);
  t.logits = scores;
  t.lens = lens;
  t.ws_zeroed = c.zero && c.zero_words > 0;
  return launched(fn, launch_topk(t, topk_ws, stream));
}

}  // namespace dsaidx

extern "C" {

idx_status idx_logits(const void* q, int q_dtype, const float* w, const void* k, const void* k_scale,
                      int k_dtype, int64_t n_keys, const int32_t* row_ks, const int32_t* row_ke,
                      int rows, float* logits, int64_t ld, idx_stream_t stream) {
  idx_problem p{};
  p.mode = IDX_MODE_DENSE;
  p.rows = rows;
  p.q = q;
  p.q_dtype = q_dtype;
  p.k_dtype = k_dtype;
  p.w = w;
  p.k = k;
  p.k_scale = k_scale;
  p.n_keys = n_keys;
  p.row_ks = row_ks;
  p.row_ke = row_ke;
  ScoreCall c;
  idx_status s = check_problem("idx_logits", &p, &c, logits, ld, true);
  if (s != IDX_OK) return s;
  if (rows == 0) return ok();
  c.err = device_error_word();
  log_once("idx_logits: %s (rows %d, ld %lld)",
           prefill_applies(c) ? "tiled prefill kernel" : rows <= kBalancedMaxRows ? "balanced scan" : "row-item scan",
           rows, (long long)ld);
  return launched("idx_logits", launch_score(c, (hipStream_t)stream));
}

idx_status idx_logits_prefill(const void* q, int q_dtype, const float* w, const void* k, const void* k_scale,
                              int k_dtype, int64_t n_keys, const int32_t* row_ks, const int32_t* row_ke,
                              int rows, float* logits, int64_t ld, idx_stream_t stream) {
  idx_problem p{};
  p.mode = IDX_MODE_PREFILL;
  p.rows = rows;
  p.q = q;
  p.q_dtype = q_dtype;
  p.k_dtype = k_dtype;
  p.w = w;
  p.k = k;
  p.k_scale = k_scale;
  p.n_keys = n_keys;
  p.row_ks = row_ks;
  p.row_ke = row_ke;
  ScoreCall c;
  idx_status s = check_problem("idx_logits_prefill", &p, &c, logits, ld, true);
  if (s != IDX_OK) return s;
  if (rows == 0) return ok();
  c.err = device_error_word();
  log_once("idx_logits_prefill: %s (rows %d, ld %lld)",
           prefill_applies(c) ? "tiled prefill kernel" : rows <= kBalancedMaxRows ? "balanced scan" : "row-item scan",
           rows, (long long)ld);
  return launched("idx_logits_prefill", launch_score(c, (hipStream_t)stream));
}

idx_status idx_logits_paged(const void* q, int q_dtype, const float* w, const void* k_pages,
                            const void* k_scale_pages, int k_dtype, int64_t n_pages, int page_size,
                            const int32_t* block_table, int64_t bt_rows, int64_t bt_ld,
                            const int32_t* seq_lens, const int32_t* row_req, int rows, float* logits,
                            int64_t ld, idx_stream_t stream) {
  idx_problem p{};
  p.mode = IDX_MODE_PAGED;
  p.rows = rows;
  p.q = q;
  p.q_dtype = q_dtype;
  p.k_dtype = k_dtype;
  p.w = w;
  p.k = k_pages;
  p.k_scale = k_scale_pages;
  p.n_keys = n_pages;
  p.page_size = page_size;
  p.block_table = block_table;
  p.bt_rows = bt_rows;
  p.bt_ld = bt_ld;
  p.seq_lens = seq_lens;
  p.row_req = row_req;
  ScoreCall c;
  idx_status s = check_problem("idx_logits_paged", &p, &c, logits, ld, true);
  if (s != IDX_OK) return s;
  if (rows == 0) return ok();
  REQUIRE(bt_rows >= 1 && (row_req || bt_rows >= rows), IDX_ERR_ARG,
          "idx_logits_paged: bt_rows = %lld too small", (long long)bt_rows);
  c.bt_rows = bt_rows;
  c.err = device_error_word();
  log_once("idx_logits_paged: %s (rows %d, page %d)", rows <= kBalancedMaxRows ? "balanced scan" : "row-item scan",
           rows, page_size);
  return launched("idx_logits_paged", launch_score(c, (hipStream_t)stream));
}

idx_status idx_logits_sparse_blocks(const void* q, int q_dtype, const float* w, const void* k,
                                    const void* k_scale, int k_dtype, int64_t n_keys,
                                    const int32_t* row_ks, const int32_t* row_ke,
                                    const int32_t* cand_blocks, int64_t cand_ld, const int32_t* n_cols,
                                    int block_size, int rows, float* logits, int64_t ld,
                                    idx_stream_t stream) {
  idx_problem p{};
  p.mode = IDX_MODE_SPARSE_BLOCKS;
  p.rows = rows;
  p.q = q;
  p.q_dtype = q_dtype;
  p.k_dtype = k_dtype;
  p.w = w;
  p.k = k;
  p.k_scale = k_scale;
  p.n_keys = n_keys;
  p.row_ks = row_ks;
  p.row_ke = row_ke;
  p.cand_blocks = cand_blocks;
  p.cand_ld = cand_ld;
  p.n_cols = n_cols;
  p.block_size = block_size;
  ScoreCall c;
  idx_status s = check_problem("idx_logits_sparse_blocks", &p, &c, logits, ld, true);
  if (s != IDX_OK) return s;
  if (rows == 0) return ok();
  REQUIRE(ld >= cand_ld * block_size, IDX_ERR_ARG,
          "idx_logits_sparse_blocks: ld = %lld < cand_ld * block_size = %lld", (long long)ld,
          (long long)(cand_ld * block_size));
  c.err = device_error_word();
  log_once("idx_logits_sparse_blocks: %s (rows %d, block %d)",
           rows <= kBalancedMaxRows ? "balanced scan" : "row-item scan", rows, block_size);
  return launched("idx_logits_sparse_blocks", launch_score(c, (hipStream_t)stream));
}

idx_status idx_logits_paged_sparse_blocks(const void* q, int q_dtype, const float* w, const void* k_pages,
                                          const void* k_scale_pages, int k_dtype, int64_t n_pages, int page_size,
                                          const int32_t* block_table, int64_t bt_rows, int64_t bt_ld,
                                          const int32_t* seq_lens, const int32_t* row_req,
                                          const int32_t* cand_blocks, int64_t cand_ld, const int32_t* n_cols,
                                          int block_size, int rows, float* logits, int64_t ld,
                                          idx_stream_t stream) {
  const char* fn = "idx_logits_paged_sparse_blocks";
  idx_problem p{};
  p.mode = IDX_MODE_PAGED_SPARSE_BLOCKS;
  p.rows = rows;
  p.q = q;
  p.q_dtype = q_dtype;
  p.k_dtype = k_dtype;
  p.w = w;
  p.k = k_pages;
  p.k_scale = k_scale_pages;
  p.n_keys = n_pages;
  p.page_size = page_size;
  p.block_table = block_table;
  p.bt_rows = bt_rows;
  p.bt_ld = bt_ld;
  p.seq_lens = seq_lens;
  p.row_req = row_req;
  p.cand_blocks = cand_blocks;
  p.cand_ld = cand_ld;
  p.n_cols = n_cols;
  p.block_size = block_size;
  ScoreCall c;
  idx_status s = check_problem(fn, &p, &c, logits, ld, true);
  if (s != IDX_OK) return s;
  if (rows == 0) return ok();
  REQUIRE(bt_rows >= 1 && (row_req || bt_rows >= rows), IDX_ERR_ARG, "%s: bt_rows = %lld too small", fn,
          (long long)bt_rows);
  REQUIRE(ld >= cand_ld * block_size, IDX_ERR_ARG, "%s: ld = %lld < cand_ld * block_size = %lld", fn,
          (long long)ld, (long long)(cand_ld * block_size));
  c.bt_rows = bt_rows;
  c.err = device_error_word();
  log_once("%s: %s (rows %d, page %d, block %d)", fn, rows <= kBalancedMaxRows ? "balanced scan" : "row-item scan",
           rows, page_size, block_size);
  return launched(fn, launch_score(c, (hipStream_t)stream));
}

size_t idx_topk_workspace(int rows, int64_t n_cols, int) { return topk_workspace_bytes(rows, n_cols); }

idx_status idx_topk(const float* logits, int64_t ld, const int32_t* lens, int64_t n_cols, int rows,
                    int k, int32_t* out_idx, float* out_val, int64_t out_ld, uint32_t flags,
                    void* workspace, size_t workspace_bytes, idx_stream_t stream) {
  const char* fn = "idx_topk";
  REQUIRE(rows >= 0, IDX_ERR_ARG, "%s: rows = %d is negative", fn, rows);
  REQUIRE(k >= 1 && k <= IDX_MAX_K, IDX_ERR_UNSUPPORTED, "%s: k = %d outside [1, %d]", fn, k, IDX_MAX_K);
  REQUIRE((flags & ~IDX_TOPK_UNSORTED) == 0, IDX_ERR_ARG, "%s: unknown flags 0x%x", fn, flags);
  if (rows == 0) return ok();
  REQUIRE(logits && out_idx, IDX_ERR_ARG, "%s: logits and out_idx must be non-null", fn);
  REQUIRE(n_cols >= 0 && n_cols <= kMaxCols, IDX_ERR_ARG, "%s: n_cols = %lld out of range", fn, (long long)n_cols);
  REQUIRE(ld >= n_cols && ld >= 1, IDX_ERR_ARG, "%s: ld = %lld < n_cols = %lld", fn, (long long)ld, (long long)n_cols);
  REQUIRE(out_ld >= k, IDX_ERR_ARG, "%s: out_ld = %lld < k = %d", fn, (long long)out_ld, k);
  REQUIRE(aligned(logits, 4) && aligned(out_idx, 4) && (!out_val || aligned(out_val, 4)), IDX_ERR_ARG,
          "%s: arrays must be 4-byte aligned", fn);
  idx_status s = check_ints(fn, {lens});
  if (s != IDX_OK) return s;
  const size_t need = topk_workspace_bytes(rows, n_cols);
  REQUIRE(need == 0 || (workspace && workspace_bytes >= need), IDX_ERR_WORKSPACE,
          "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace ? workspace_bytes : (size_t)0);
  REQUIRE(need == 0 || aligned(workspace, 256), IDX_ERR_ARG, "%s: workspace must be 256-byte aligned", fn);
  TopkCall c{};
  c.logits = logits;
  c.ld = ld;
  c.n_cols = n_cols;
  c.lens = lens;
  c.rows = rows;
  c.k = k;
  c.out_idx = out_idx;
  c.out_val = out_val;
  c.out_ld = out_ld;
  c.sorted = (flags & IDX_TOPK_UNSORTED) ? 0 : 1;
  log_once("idx_topk: %s (rows %d, n_cols %lld, k %d)", topk_path(rows, n_cols), rows, (long long)n_cols, k);
  return launched(fn, launch_topk(c, workspace, (hipStream_t)stream));
}

size_t idx_select_workspace(const idx_problem* p, int k) {
  (void)k;
  if (!p || p->rows <= 0) return 0;
  int64_t width = select_width(p);
  if (width <= 0) return 0;
  const size_t two_pass = select_scores_bytes(p) + select_lens_bytes(p) + topk_workspace_bytes(p->rows, width);
  if (!select_one_pass_possible(p)) return two_pass;
  return std::max(two_pass, select_layout(p).total);
}

idx_status idx_select(const idx_problem* p, int k, int32_t* out_idx, float* out_val, int64_t out_ld,
                      uint32_t flags, void* workspace, size_t workspace_bytes, idx_stream_t stream) {
  return select_call("idx_select", p, k, out_idx, out_val, out_ld, flags, workspace, workspace_bytes,
                     (hipStream_t)stream);
}

const char* idx_status_string(idx_status s) {
  switch (s) {
    case IDX_OK: return "IDX_OK";
    case IDX_ERR_ARG: return "IDX_ERR_ARG";
    case IDX_ERR_UNSUPPORTED: return "IDX_ERR_UNSUPPORTED";
    case IDX_ERR_WORKSPACE: return "IDX_ERR_WORKSPACE";
    case IDX_ERR_HIP: return "IDX_ERR_HIP";
  }
  return "IDX_ERR_UNKNOWN";
}

const char* idx_last_error(void) { return g_last_error.c_str(); }

int idx_version(void) { return 100; }

size_t idx_candidate_blocks_workspace(int rows, int64_t n_cols) { return cand_workspace_bytes(rows, n_cols); }

idx_status idx_candidate_blocks(const float* logits, int64_t ld, const int32_t* lens, int64_t n_cols, int rows,
                                int block_size, int n_top, int32_t* cand_blocks, int64_t cand_ld, int32_t* n_cand,
                                void* workspace, size_t workspace_bytes, idx_stream_t stream) {
  const char* fn = "idx_candidate_blocks";
  REQUIRE(rows >= 0, IDX_ERR_ARG, "%s: rows = %d is negative", fn, rows);
  REQUIRE(block_size >= 64 && block_size % 64 == 0 && block_size <= kMaxCandBlockSize, IDX_ERR_UNSUPPORTED,
          "%s: block_size = %d must be a multiple of 64 in [64, %d]", fn, block_size, kMaxCandBlockSize);
  REQUIRE(n_top >= 1, IDX_ERR_ARG, "%s: n_top = %d must be >= 1", fn, n_top);
  if (rows == 0) return ok();
  REQUIRE(logits && cand_blocks && n_cand, IDX_ERR_ARG, "%s: logits, cand_blocks and n_cand must be non-null", fn);
  REQUIRE(n_cols >= 0 && n_cols <= kMaxCols, IDX_ERR_ARG, "%s: n_cols = %lld out of range", fn, (long long)n_cols);
  REQUIRE(ld >= n_cols && ld >= 1, IDX_ERR_ARG, "%s: ld = %lld < n_cols = %lld", fn, (long long)ld,
          (long long)n_cols);
  REQUIRE(cand_ld >= n_top, IDX_ERR_ARG, "%s: cand_ld = %lld < n_top = %d", fn, (long long)cand_ld, n_top);
  REQUIRE((n_cols + block_size - 1) / block_size <= kCandMaxBlocks, IDX_ERR_UNSUPPORTED,
          "%s: %lld columns make more than %d blocks of %d", fn, (long long)n_cols, kCandMaxBlocks, block_size);
  REQUIRE(aligned(logits, 4) && aligned(cand_blocks, 4) && aligned(n_cand, 4), IDX_ERR_ARG,
          "%s: arrays must be 4-byte aligned", fn);
  idx_status s = check_ints(fn, {lens});
  if (s != IDX_OK) return s;
  const size_t need = cand_workspace_bytes(rows, n_cols);
  REQUIRE(need == 0 || (workspace && workspace_bytes >= need), IDX_ERR_WORKSPACE,
          "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace ? workspace_bytes : (size_t)0);
  REQUIRE(need == 0 || aligned(workspace, 256), IDX_ERR_ARG, "%s: workspace must be 256-byte aligned", fn);
  CandCall c{};
  c.logits = logits;
  c.ld = ld;
  c.lens = lens;
  c.n_cols = n_cols;
  c.rows = rows;
  c.block = block_size;
  c.n_top = n_top;
  c.cand = cand_blocks;
  c.cand_ld = cand_ld;
  c.n_cand = n_cand;
  return launched(fn, launch_candidate_blocks(c, workspace, (hipStream_t)stream));
}

size_t idx_sparse_attn_workspace(int rows, int heads, int k) {
  if (rows <= 0 || k <= 0 || heads <= 0) return 0;
  return attn_workspace_bytes(rows, heads, k);
}

idx_status idx_sparse_attn_paged(const void* q, int heads, const void* kv_pages, int64_t n_pages, int page_size,
                                 const int32_t* block_table, int64_t bt_rows, int64_t bt_ld,
                                 const int32_t* seq_lens, const int32_t* row_req, const int32_t* indices,
                                 int64_t idx_ld, int k, int rows, float scale, float* out, float* lse,
                                 void* workspace, size_t workspace_bytes, idx_stream_t stream) {
  const char* fn = "idx_sparse_attn_paged";
  REQUIRE(rows >= 0, IDX_ERR_ARG, "%s: rows = %d is negative", fn, rows);
  REQUIRE(heads == 16 || heads == 32 || heads == 64 || heads == 128, IDX_ERR_UNSUPPORTED,
          "%s: heads = %d must be 16, 32, 64 or 128", fn, heads);
  REQUIRE(page_size == 64, IDX_ERR_UNSUPPORTED, "%s: page_size = %d must be 64", fn, page_size);
  REQUIRE(k >= 1 && k <= IDX_MAX_K, IDX_ERR_UNSUPPORTED, "%s: k = %d outside [1, %d]", fn, k, IDX_MAX_K);
  if (rows == 0) return ok();
  REQUIRE(q && kv_pages && block_table && seq_lens && indices && out, IDX_ERR_ARG,
          "%s: q, kv_pages, block_table, seq_lens, indices and out must be non-null", fn);
  REQUIRE(n_pages >= 1 && bt_rows >= 1 && bt_ld >= 1 && idx_ld >= k, IDX_ERR_ARG,
          "%s: n_pages, bt_rows, bt_ld must be >= 1 and idx_ld >= k", fn);
  REQUIRE(row_req || bt_rows >= rows, IDX_ERR_ARG, "%s: bt_rows = %lld < rows without row_req", fn,
          (long long)bt_rows);
  REQUIRE(std::isfinite(scale), IDX_ERR_ARG, "%s: scale must be finite", fn);
  REQUIRE(aligned(q, 16) && aligned(kv_pages, 16), IDX_ERR_ARG, "%s: q and kv_pages must be 16-byte aligned", fn);
  REQUIRE(aligned(out, 16) && (!lse || aligned(lse, 4)), IDX_ERR_ARG,
          "%s: out must be 16-byte and lse 4-byte aligned", fn);
  idx_status s = check_ints(fn, {block_table, seq_lens, row_req, indices});
  if (s != IDX_OK) return s;
  const size_t need = idx_sparse_attn_workspace(rows, heads, k);
  REQUIRE(need == 0 || (workspace && workspace_bytes >= need), IDX_ERR_WORKSPACE,
          "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace ? workspace_bytes : (size_t)0);
  REQUIRE(need == 0 || aligned(workspace, 256), IDX_ERR_ARG, "%s: workspace must be 256-byte aligned", fn);
  AttnCall c{};
  c.q = q;
  c.kv = kv_pages;
  c.n_pages = n_pages;
  c.page_size = page_size;
  c.block_table = block_table;
  c.bt_rows = bt_rows;
  c.bt_ld = bt_ld;
  c.seq_lens = seq_lens;
  c.row_req = row_req;
  c.indices = indices;
  c.idx_ld = idx_ld;
  c.k = k;
  c.rows = rows;
  c.heads = heads;
  c.scale = scale;
  c.out = out;
  c.lse = lse;
  c.err = device_error_word();
  return launched(fn, launch_sparse_attn(c, workspace, (hipStream_t)stream));
}

idx_status idx_kcache_write(const void* k_new, int new_dtype, int64_t n_new, const int64_t* slot_mapping,
                            void* k_cache, void* k_scale, int k_dtype, int64_t n_slots, idx_stream_t stream) {
  const char* fn = "idx_kcache_write";
  REQUIRE(n_new >= 0 && n_slots >= 0, IDX_ERR_ARG, "%s: n_new = %lld and n_slots = %lld must be >= 0", fn,
          (long long)n_new, (long long)n_slots);
  REQUIRE(new_dtype == IDX_BF16, IDX_ERR_UNSUPPORTED, "%s: new keys must be IDX_BF16 (got %d)", fn, new_dtype);
  REQUIRE(k_dtype == IDX_FP8_E4M3 || k_dtype == IDX_MXFP4, IDX_ERR_UNSUPPORTED,
          "%s: the cache must be IDX_FP8_E4M3 or IDX_MXFP4 (got %d)", fn, k_dtype);
  if (n_new == 0) return ok();
  REQUIRE(k_new && slot_mapping && k_cache && k_scale, IDX_ERR_ARG,
          "%s: k_new, slot_mapping, k_cache and k_scale must be non-null", fn);
  REQUIRE(aligned(k_new, 16) && aligned(slot_mapping, 8), IDX_ERR_ARG,
          "%s: k_new must be 16-byte and slot_mapping 8-byte aligned", fn);
  REQUIRE(aligned(k_cache, 16) && aligned(k_scale, 4), IDX_ERR_ARG,
          "%s: k_cache must be 16-byte and k_scale 4-byte aligned", fn);
  KcacheCall c{};
  c.k_new = k_new;
  c.slots = slot_mapping;
  c.n_new = n_new;
  c.fmt = k_dtype == IDX_FP8_E4M3 ? FMT_FP8 : FMT_MXFP4;
  c.cache = (uint8_t*)k_cache;
  c.scale = k_scale;
  c.n_slots = n_slots;
  c.err = device_error_word();
  return launched(fn, launch_kcache_write(c, (hipStream_t)stream));
}

idx_status idx_read_probe(const void* buf, size_t bytes, uint32_t* sink, idx_stream_t stream) {
  const char* fn = "idx_read_probe";
  REQUIRE(buf && sink, IDX_ERR_ARG, "%s: buf and sink must be non-null", fn);
  REQUIRE(aligned(buf, 16) && bytes % 16 == 0, IDX_ERR_ARG, "%s: buf must be 16-byte aligned and bytes a multiple of 16",
          fn);
  REQUIRE(aligned(sink, 4), IDX_ERR_ARG, "%s: sink must be 4-byte aligned", fn);
  return launched(fn, launch_read_probe(buf, bytes, sink, (hipStream_t)stream));
}

int idx_device_errors(idx_stream_t stream) {
  unsigned* p = device_error_word();
  if (!p) {
    fail(IDX_ERR_HIP, "idx_device_errors: no device error word");
    return -1;
  }
  unsigned v = 0;
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e == hipSuccess) e = hipMemcpy(&v, p, sizeof v, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemset(p, 0, sizeof v);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    fail(IDX_ERR_HIP, "idx_device_errors: %s", hipGetErrorString(e));
    return -1;
  }
  return (int)v;
}

}  // extern "C"
