// Streaming key-cache scan: Eq. (1) of the DeepSeek-V3.2 architecture section for
// rows that each read their own keys (decode rows, paged decode, candidate blocks).
//
// Work split: an item is (row, chunk of positions); waves take items in a
// grid-stride loop. A wave scores 64 positions per step:
//   * the step's 64 key rows are loaded with 16-byte loads: fp8 rows in whole 1 KiB
//     blocks of 8 rows, then moved across lanes into the MFMA operand order (lane
//     l % 16 = token column of a 16-token tile, l / 16 = K block); MXFP4 and bf16 rows
//     directly in operand order (each load instruction reads 1 KiB of 16 rows),
//   * 16 MFMAs (4 head tiles x 4 token tiles) give S[head, token] = q_head . k,
//   * each lane applies ReLU and its 16 head weights in registers, three lane
//     swaps finish the 64-head sum, and lane l holds the score of position l,
//   * the fp8 per-token scale multiplies after the head sum (scales are >= 0, so
//     ReLU(scale * x) = scale * ReLU(x)); MXFP4 group scales enter the MFMA itself,
//   * the 64 scores (-inf where the position is not scored) go to the wave's LDS
//     slice; the item's scores leave in 1 KiB stores once it is done, so score
//     stores do not interleave with the key stream.
// The keys of step s + 1 load while step s computes (two register sets); keys are
// read once per call, so their loads are non-temporal.
#include "device.h"
#include "launch.h"
#include "topk_device.h"

#include <mutex>

namespace dsaidx {

struct ScanCommon {
  const uint8_t* q;
  const float* w;
  const uint8_t* k;
  const void* k_scale;
  float* logits;
  int64_t ld;
  int rows;
  int chunk_tiles;  // item schedule: steps per item
  int64_t n_items;
  unsigned* err;
  int skip_tail;    // columns past a row's scored steps stay unwritten
  uint32_t* zero;   // words to clear (every wave clears its share first)
  int64_t zero_words;
  int32_t* lens_out;  // optional: each row's scored length (clipped to ld)
};

// ------------------------------------------------------------------ key sources
//
// Pages and candidate blocks hold a multiple of 64 keys and steps start at multiples
// of 64 positions, so the 64 positions of a step name 64 consecutive key rows. A
// source describes step s of a row by its first key row and by how many leading
// positions of the step are scored (its valid prefix, <= 0 when none is). The lookup
// has two halves so a caller can issue the table load early and use it later:
// step_raw loads the table entry the step needs (page or candidate block id), step_desc
// turns it into the description; step is both at once.

struct StepDesc {
  int64_t kidx0;
  int32_t vlim;
};

// Contiguous range [row_ks, row_ke) of a flat key array.
struct DenseSrc {
  const int32_t* ks;
  const int32_t* ke;
  int64_t n_keys;
  struct Row {
    int64_t base, len;
  };
  __device__ Row row(int r, int64_t ld, unsigned* err, bool report) const {
    int64_t s = ks[r], e = ke[r];
    int64_t s2 = min(max(s, (int64_t)0), n_keys);
    int64_t e2 = min(max(e, s2), n_keys);
    int64_t len = min(e2 - s2, ld);
    if (report && (s2 != s || e2 != e || len != e2 - s2)) flag_error(err, kErrRange);
    return {s2, len};
  }
  __device__ int64_t bound(const Row& R) const { return R.len; }
  __device__ int64_t step_raw(const Row&, int64_t) const { return 0; }
  __device__ StepDesc step_desc(const Row& R, int64_t pos0, int64_t, unsigned*) const {
    return {R.base + pos0, (int32_t)min(R.len - pos0, (int64_t)kTileTokens)};
  }
  __device__ StepDesc step(const Row& R, int64_t pos0, unsigned* err) const {
    return step_desc(R, pos0, 0, err);
  }
};

// Logical position s of request req in page block_table[req][s / page], slot s % page.
struct PagedSrc {
  const int32_t* bt;
  int64_t bt_rows, bt_ld;
  const int32_t* seq_lens;
  const int32_t* row_req;
  int64_t n_pages;
  int page;
  struct Row {
    const int32_t* bt_row;
    int64_t len;
  };
  __device__ Row row(int r, int64_t ld, unsigned* err, bool report) const {
    int64_t req = row_req ? (int64_t)row_req[r] : (int64_t)r;
    int64_t req2 = min(max(req, (int64_t)0), bt_rows - 1);
    int64_t L = seq_lens[r];
    int64_t L2 = min(max(L, (int64_t)0), min(bt_ld * page, ld));
    if (report && (req2 != req || L2 != L)) flag_error(err, kErrRange);
    return {bt + req2 * bt_ld, L2};
  }
  __device__ int64_t bound(const Row& R) const { return R.len; }
  __device__ int64_t step_raw(const Row& R, int64_t pos0) const {
    return pos0 < R.len ? (int64_t)R.bt_row[pos0 / page] : 0;
  }
  __device__ StepDesc step(const Row& R, int64_t pos0, unsigned* err) const {
    return step_desc(R, pos0, step_raw(R, pos0), err);
  }
  __device__ StepDesc step_desc(const Row& R, int64_t pos0, int64_t pg, unsigned* err) const {
    if (pos0 >= R.len) return {0, 0};
    if (pg < 0 || pg >= n_pages) {
      flag_error(err, kErrPage);
      pg = min(max(pg, (int64_t)0), n_pages - 1);
    }
    return {pg * page + pos0 % page, (int32_t)min(R.len - pos0, (int64_t)kTileTokens)};
  }
};

// Candidate blocks: column c names token cand[r][c / block] * block + c % block of
// the row's range [row_ks, row_ke); columns at or past n_cols[r] are not scored.
struct SparseSrc {
  const int32_t* ks;
  const int32_t* ke;
  int64_t n_keys;
  const int32_t* cand;
  int64_t cand_ld;
  const int32_t* n_cols;
  int block;
  struct Row {
    int64_t base, len;
    const int32_t* cand_row;
    int64_t ncols;
  };
  __device__ Row row(int r, int64_t ld, unsigned* err, bool report) const {
    int64_t s = ks[r], e = ke[r];
    int64_t s2 = min(max(s, (int64_t)0), n_keys);
    int64_t e2 = min(max(e, s2), n_keys);
    int64_t nc = n_cols[r];
    int64_t nc2 = min(max(nc, (int64_t)0), cand_ld * block);
    if (report && (s2 != s || e2 != e || nc2 != nc)) flag_error(err, kErrRange);
    if (e2 == s2) nc2 = 0;  // no keys: nothing to score
    return {s2, e2 - s2, cand + (int64_t)r * cand_ld, nc2};
  }
  __device__ int64_t bound(const Row& R) const { return R.ncols; }
  __device__ int64_t step_raw(const Row& R, int64_t pos0) const {
    return pos0 < R.ncols ? (int64_t)R.cand_row[pos0 / block] : 0;
  }
  __device__ StepDesc step(const Row& R, int64_t pos0, unsigned* err) const {
    return step_desc(R, pos0, step_raw(R, pos0), err);
  }
  __device__ StepDesc step_desc(const Row& R, int64_t pos0, int64_t cb, unsigned* err) const {
    if (pos0 >= R.ncols) return {0, 0};
    if (cb < 0 || cb * block >= R.len) {  // no token of the block lies in the row's range
      flag_error(err, kErrBlock);
      return {0, 0};
    }
    // a row's candidate blocks must be strictly increasing (the column order then is the
    // token order, which the selection's ties follow)
    if (pos0 % block == 0 && pos0 >= block && R.cand_row[pos0 / block - 1] >= cb) flag_error(err, kErrOrder);
    const int64_t tok0 = cb * block + pos0 % block;
    const int64_t v = min(min(R.ncols - pos0, R.len - tok0), (int64_t)kTileTokens);
    return {R.base + (v > 0 ? tok0 : 0), (int32_t)v};
  }
};

// Candidate blocks of a paged row (the two-level decode layout): column c names the row's
// logical token cand[r][c / block] * block + c % block, which lives in page
// block_table[req][token / page], slot token % page; columns at or past n_cols[r] are not
// scored. Blocks and pages are multiples of 64 tokens, so a step's 64 tokens lie in one
// block and one page.
struct PagedSparseSrc {
  const int32_t* bt;
  int64_t bt_rows, bt_ld;
  const int32_t* seq_lens;
  const int32_t* row_req;
  int64_t n_pages;
  int page;
  const int32_t* cand;
  int64_t cand_ld;
  const int32_t* n_cols;
  int block;
  struct Row {
    const int32_t* bt_row;
    int64_t len;
    const int32_t* cand_row;
    int64_t ncols;
  };
  __device__ Row row(int r, int64_t ld, unsigned* err, bool report) const {
    int64_t req = row_req ? (int64_t)row_req[r] : (int64_t)r;
    int64_t req2 = min(max(req, (int64_t)0), bt_rows - 1);
    int64_t L = seq_lens[r];
    int64_t L2 = min(max(L, (int64_t)0), bt_ld * page);
    int64_t nc = n_cols[r];
    int64_t nc2 = min(max(nc, (int64_t)0), min(cand_ld * block, ld));
    if (report && (req2 != req || L2 != L || nc2 != nc)) flag_error(err, kErrRange);
    if (L2 == 0) nc2 = 0;  // no keys: nothing to score
    return {bt + req2 * bt_ld, L2, cand + (int64_t)r * cand_ld, nc2};
  }
  __device__ int64_t bound(const Row& R) const { return R.ncols; }
  __device__ int64_t step_raw(const Row& R, int64_t pos0) const {
    return pos0 < R.ncols ? (int64_t)R.cand_row[pos0 / block] : 0;
  }
  __device__ StepDesc step(const Row& R, int64_t pos0, unsigned* err) const {
    return step_desc(R, pos0, step_raw(R, pos0), err);
  }
  __device__ StepDesc step_desc(const Row& R, int64_t pos0, int64_t cb, unsigned* err) const {
    if (pos0 >= R.ncols) return {0, 0};
    if (cb < 0 || cb * block >= R.len) {  // no token of the block lies in the row
      flag_error(err, kErrBlock);
      return {0, 0};
    }
    if (pos0 % block == 0 && pos0 >= block && R.cand_row[pos0 / block - 1] >= cb) flag_error(err, kErrOrder);
    const int64_t tok0 = cb * block + pos0 % block;
    const int64_t v = min(min(R.ncols - pos0, R.len - tok0), (int64_t)kTileTokens);
    if (v <= 0) return {0, 0};
    int64_t pg = R.bt_row[tok0 / page];
    if (pg < 0 || pg >= n_pages) {
      flag_error(err, kErrPage);
      pg = min(max(pg, (int64_t)0), n_pages - 1);
    }
    return {pg * page + tok0 % page, (int32_t)v};
  }
};

// ------------------------------------------------------------------ per-format operands

template <int F>
struct QOps;
template <int F>
struct KOps;

// fp8 q, head tile h, lane l: row 16h + l%16, dims 16g .. 16g+15 and 64+16g ..
// 64+16g+15 (g = l / 16), which is the 8-bit operand's own K order (measured on gfx950
// with one-hot inputs). Against fp8 keys any K order shared by both operands would
// do (the key operand is assembled in this order from whole-row loads). Against MXFP4
// keys it is required: the fp4 operand of lane group g holds dims 32g .. 32g+31 (one
// UE8M0 group) in hardware order.
template <int F>
struct QOps {
  static_assert(F == FMT_FP8 || F == FMT_MXFP4, "8-bit q operand");
  v8i a[4];
  __device__ void load(const uint8_t* q, int r, int lane) {
    const int g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint8_t* row = q + ((int64_t)r * kHeads + 16 * h + c) * kDim;
      v4i lo = *(const v4i*)(row + 16 * g), hi = *(const v4i*)(row + 64 + 16 * g);
      a[h] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
};

// bf16 q: head tile h, K-step s, lane l -> q[16h + l%16][32s + 8g .. +7]; the keys use
// the same order (each key load instruction then reads 64 contiguous bytes per key).
template <>
struct QOps<FMT_BF16> {
  v8bf a[4][4];
  __device__ void load(const uint8_t* q, int r, int lane) {
    const int g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const v8bf* p = (const v8bf*)(q + (((int64_t)r * kHeads + 16 * h + c) * kDim + 8 * g) * 2);
#pragma unroll
      for (int s = 0; s < 4; ++s) a[h][s] = p[4 * s];
    }
  }
};

// fp8 keys are read in whole 1 KiB blocks (8 key rows; lane l takes 16 bytes: row
// l / 8, chunk l % 8), which the memory system serves faster than the operand order
// (every 16-lane quarter of a load instruction then reads two whole cache lines instead
// of pieces of 16 rows); the operand is then assembled across lanes. Tile j is blocks
// 2j (rows 0..7 of the tile) and 2j + 1 (rows 8..15); lane (g, c) of the operand needs
// chunks g and g + 4 of row c, which sit in lanes 8(c % 8) + g and + 4 of block
// 2j + c / 8. One row_shr:4 / row_shl:4 merge of the two blocks puts, in each 8-lane
// group, the low chunks of both blocks in one register and the high chunks in another,
// so that one backward permute per register fetches both halves of the operand.
template <>
struct KOps<FMT_FP8> {
  v4i raw[2];
  __device__ void load_rows(const uint8_t* k, int64_t kidx0, int j, int last, int lane) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = min(16 * j + 8 * h + (lane >> 3), last);
      raw[h] = __builtin_nontemporal_load((const v4i*)(k + (kidx0 + t) * kDim + 16 * (lane & 7)));
    }
  }
  __device__ v8i operand(int lane) const {
    const int c = lane & 15, g = lane >> 4;
    const int src = 4 * (8 * (c & 7) + g + 4 * (c >> 3));
    v8i b;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      // the merges write only the lanes of chunks 4..7 (DPP banks 1 and 3: lanes 4..7 and
      // 12..15 of each row), resp. of chunks 0..3 (banks 0 and 2); the other lanes keep
      // the first operand, so no lane-dependent branch is needed around the shifts
      const int s1 = __builtin_amdgcn_update_dpp(raw[0][d], raw[1][d], 0x114, 0xF, 0xA, false);  // row_shr:4
      const int s2 = __builtin_amdgcn_update_dpp(raw[1][d], raw[0][d], 0x104, 0xF, 0x5, false);  // row_shl:4
      b[d] = __builtin_amdgcn_ds_bpermute(src, s1);
      b[4 + d] = __builtin_amdgcn_ds_bpermute(src, s2);
    }
    return b;
  }
  static __device__ v4f mma(const QOps<FMT_FP8>& qo, int h, const v8i& b) {
    return mfma_fp8_fp8(qo.a[h], b, v4f{0.f, 0.f, 0.f, 0.f});
  }
};

template <>
struct KOps<FMT_MXFP4> {
  v4i b;
  int sc;
  __device__ void load(const uint8_t* k, const void* scale, int64_t kidx, int g) {
    b = __builtin_nontemporal_load((const v4i*)(k + kidx * (kDim / 2) + 16 * g));
    sc = ((const uint8_t*)scale)[kidx * (kDim / 32) + g];
  }
  __device__ const KOps& operand(int) const { return *this; }
  static __device__ v4f mma(const QOps<FMT_MXFP4>& qo, int h, const KOps& ko) {
    v8i bb = v8i{ko.b[0], ko.b[1], ko.b[2], ko.b[3], 0, 0, 0, 0};
    return mfma_fp8_fp4(qo.a[h], bb, ko.sc, v4f{0.f, 0.f, 0.f, 0.f});
  }
};

template <>
struct KOps<FMT_BF16> {
  v8bf b[4];
  __device__ void load(const uint8_t* k, const void*, int64_t kidx, int g) {
    const v8bf* p = (const v8bf*)(k + (kidx * kDim + 8 * g) * 2);
#pragma unroll
    for (int s = 0; s < 4; ++s) b[s] = __builtin_nontemporal_load(p + 4 * s);
  }
  __device__ const KOps& operand(int) const { return *this; }
  static __device__ v4f mma(const QOps<FMT_BF16>& qo, int h, const KOps& ko) {
    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma_bf16(qo.a[h][s], ko.b[s], acc);
    return acc;
  }
};

// ------------------------------------------------------------------ kernel

// Loads the key operands of one step (lane: column c16 of tile j, K-block g) and the
// scale of the key whose score this lane stores (position lane of the step).
template <int F>
__device__ __forceinline__ void load_step(KOps<F> (&ko)[4], float& sc, const ScanCommon& a, int64_t kidx0,
                                          int32_t vlim, int lane) {
  const int g = lane >> 4, c16 = lane & 15;
  const int last = vlim - 1;
  if constexpr (F == FMT_FP8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) ko[j].load_rows(a.k, kidx0, j, last, lane);
    sc = ((const float*)a.k_scale)[kidx0 + min(lane, last)];
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) ko[j].load(a.k, a.k_scale, kidx0 + min(16 * j + c16, last), g);
  }
}

template <int F>
__device__ __forceinline__ float score_step(const KOps<F> (&ko)[4], float sc, const QOps<F>& qo,
                                           const float (&wr)[4][4]) {
  const int lane = lane_id();
  float p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    p[j] = 0.f;
    const auto b = ko[j].operand(lane);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const v4f s = KOps<F>::mma(qo, h, b);
#pragma unroll
      for (int i = 0; i < 4; ++i) p[j] = fmaf(wr[h][i], relu(s[i]), p[j]);
    }
  }
  float v = sum_lane_groups(p[0], p[1], p[2], p[3]);
  if constexpr (F == FMT_FP8) v *= sc;
  return v;
}

__device__ __forceinline__ int64_t readlane64(int64_t v, int lane) {
  const int lo = __builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const int hi = __builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), lane);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Steps per segment: long segments start and drain the key pipeline rarely, but their
// LDS score slices (256 B per step and wave) limit the resident workgroups. MXFP4 steps
// move half the bytes of fp8 ones, so the MXFP4 kernels want more workgroups than the LDS
// of 64-step slices allows. DSAIDX_SCAN_MAX_STEPS overrides both.
#ifndef DSAIDX_SCAN_DEPTH
#define DSAIDX_SCAN_DEPTH 2
#endif
static constexpr int kBlock = 256;
template <int F>
constexpr int max_steps() {
#ifdef DSAIDX_SCAN_MAX_STEPS
  return DSAIDX_SCAN_MAX_STEPS;
#else
  return F == FMT_MXFP4 ? 32 : 64;
#endif
}
static_assert(max_steps<FMT_FP8>() >= 1 && max_steps<FMT_FP8>() <= kWave && max_steps<FMT_MXFP4>() >= 1 &&
                  max_steps<FMT_MXFP4>() <= kWave,
              "a segment describes one step per lane");

// Scores steps [s0, s0 + nsteps) of row r (nsteps <= max_steps<F>()) into sb[0, 64 nsteps)
// (LDS) and, if STORE, writes them to their columns of the score row, clipped to ld.
template <int F, class Src, bool STORE = true>
__device__ __forceinline__ void scan_segment(const ScanCommon& a, const Src& src, int r, int64_t s0, int nsteps,
                                             float* sb) {
  const int lane = lane_id();
  const int g = lane >> 4;
  const float NEG_INF = -__builtin_inff();
  const int64_t c0 = s0 * kTileTokens;
  const int64_t c1 = min(c0 + (int64_t)nsteps * kTileTokens, a.ld);
  float* out = a.logits + (int64_t)r * a.ld;
  const auto R = src.row(r, a.ld, a.err, false);
  // lane s describes step s of the segment
  StepDesc mine{0, 0};
  if (lane < nsteps) mine = src.step(R, c0 + (int64_t)kTileTokens * lane, a.err);
  QOps<F> qo;
  qo.load(a.q, r, lane);
  float wr[4][4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float4 wv = *(const float4*)(a.w + (int64_t)r * kHeads + 16 * h + 4 * g);
    wr[h][0] = wv.x;
    wr[h][1] = wv.y;
    wr[h][2] = wv.z;
    wr[h][3] = wv.w;
  }
  auto put = [&](int s, int32_t vlim, float v) { sb[s * kTileTokens + lane] = lane < vlim ? v : NEG_INF; };
#if DSAIDX_SCAN_DEPTH == 3
  // three register sets, A, B and C: the keys of steps s + 1 and s + 2 load while
  // step s computes
  KOps<F> ka[4], kb[4], kc[4];
  float sa = 1.f, sbs = 1.f, sc = 1.f;
  auto fetch = [&](KOps<F>(&ko)[4], float& scl, int s) -> int32_t {
    int32_t v = 0;
    if (s < nsteps) {
      v = __builtin_amdgcn_readlane(mine.vlim, s);
      if (v > 0) load_step<F>(ko, scl, a, readlane64(mine.kidx0, s), v, lane);
    }
    return v;
  };
  int32_t va = fetch(ka, sa, 0);
  int32_t vb = fetch(kb, sbs, 1);
  for (int s = 0; s < nsteps; s += 3) {
    const int32_t vc = fetch(kc, sc, s + 2);
    put(s, va, va > 0 ? score_step<F>(ka, sa, qo, wr) : NEG_INF);
    if (s + 1 >= nsteps) break;
    va = fetch(ka, sa, s + 3);
    put(s + 1, vb, vb > 0 ? score_step<F>(kb, sbs, qo, wr) : NEG_INF);
    if (s + 2 >= nsteps) break;
    vb = fetch(kb, sbs, s + 4);
    put(s + 2, vc, vc > 0 ? score_step<F>(kc, sc, qo, wr) : NEG_INF);
  }
#else
  // two register sets, A and B: the keys of step s + 1 load while step s computes
  KOps<F> ka[4], kb[4];
  float sa = 1.f, sbs = 1.f;
  int32_t va = __builtin_amdgcn_readlane(mine.vlim, 0);
  if (va > 0) load_step<F>(ka, sa, a, readlane64(mine.kidx0, 0), va, lane);
  for (int s = 0; s < nsteps; s += 2) {
    int32_t vb = 0;
    if (s + 1 < nsteps) {
      vb = __builtin_amdgcn_readlane(mine.vlim, s + 1);
      if (vb > 0) load_step<F>(kb, sbs, a, readlane64(mine.kidx0, s + 1), vb, lane);
    }
    put(s, va, va > 0 ? score_step<F>(ka, sa, qo, wr) : NEG_INF);
    if (s + 1 >= nsteps) break;
    va = 0;
    if (s + 2 < nsteps) {
      va = __builtin_amdgcn_readlane(mine.vlim, s + 2);
      if (va > 0) load_step<F>(ka, sa, a, readlane64(mine.kidx0, s + 2), va, lane);
    }
    put(s + 1, vb, vb > 0 ? score_step<F>(kb, sbs, qo, wr) : NEG_INF);
  }
#endif
  // LDS operations of one wave complete in order, so the lanes read what the wave
  // wrote; the columns leave four scores per lane per instruction
  __builtin_amdgcn_wave_barrier();
  if constexpr (!STORE) return;
  const int64_t cnt = c1 - c0;
  float* o = out + c0;
  const bool vec = ((uintptr_t)o & 15) == 0;
  for (int64_t i = 4 * lane; i < cnt; i += 4 * kWave) {
    const float4 v = *(const float4*)(sb + i);
    if (vec && i + 4 <= cnt) {
      *(float4*)(o + i) = v;
    } else {
      o[i] = v.x;
      if (i + 1 < cnt) o[i + 1] = v.y;
      if (i + 2 < cnt) o[i + 2] = v.z;
      if (i + 3 < cnt) o[i + 3] = v.w;
    }
  }
  __builtin_amdgcn_wave_barrier();  // the next segment's scores wait for these reads
}

// Scored columns of row r: its bound (length or valid sparse columns) clipped to ld.
template <class Src>
__device__ __forceinline__ int64_t row_cols(const ScanCommon& a, const Src& src, int r) {
  const auto R = src.row(r, a.ld, a.err, false);
  return max(min(src.bound(R), a.ld), (int64_t)0);
}

// Scored steps of row r (steps of 64 columns up to the row's bound, clipped to ld).
template <class Src>
__device__ __forceinline__ int64_t row_steps(const ScanCommon& a, const Src& src, int r, bool report) {
  const auto R = src.row(r, a.ld, a.err, report);
  const int64_t n = min(src.bound(R), a.ld);
  return n > 0 ? (n + kTileTokens - 1) / kTileTokens : 0;
}

// -inf into columns [from, ld) of row r within [f0, f1), four per lane per store.
__device__ __forceinline__ void fill_neg_inf(float* out, int64_t f0, int64_t f1) {
  const int lane = lane_id();
  const float NEG_INF = -__builtin_inff();
  if (f0 >= f1) return;
  const int64_t head = min(f1, (f0 + 3) & ~(int64_t)3);  // to a 16-byte boundary (rows are 16-byte aligned)
  if (lane < head - f0) out[f0 + lane] = NEG_INF;
  const bool vec = ((uintptr_t)out & 15) == 0;
  for (int64_t i = head + 4 * lane; i < f1; i += 4 * kWave) {
    if (vec && i + 4 <= f1) {
      *(float4*)(out + i) = make_float4(NEG_INF, NEG_INF, NEG_INF, NEG_INF);
    } else {
      for (int c = 0; c < 4 && i + c < f1; ++c) out[i + c] = NEG_INF;
    }
  }
}

// Rows beyond kBalancedMaxRows: items (row, chunk of chunk_tiles steps) taken by the waves
// in a grid-stride loop, each scored through the wave's LDS slice and stored.
template <int F, class Src>
__global__ __launch_bounds__(kBlock) void scan_items_kernel(ScanCommon a, Src src) {
  const int lane = lane_id();
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x / kWave);
  constexpr int kMaxSteps = max_steps<F>();
  __shared__ __align__(16) float sbuf[kBlock / kWave][kMaxSteps * kTileTokens];
  float* sb = sbuf[threadIdx.x / kWave];
  if (a.zero) {
    const int64_t per = (a.zero_words + nwaves - 1) / nwaves;
    const int64_t z1 = min(a.zero_words, (wave + 1) * per);
    for (int64_t i = wave * per + lane; i < z1; i += kWave) a.zero[i] = 0u;
  }
  const int64_t chunk = (int64_t)a.chunk_tiles * kTileTokens;
  for (int64_t item = wave; item < a.n_items; item += nwaves) {
    const int r = (int)(item % a.rows);
    const int64_t c0 = (item / a.rows) * chunk;
    if (c0 >= a.ld) continue;
    const int64_t c1 = min(c0 + chunk, a.ld);
    const int64_t n = row_steps(a, src, r, c0 == 0);
    if (c0 == 0 && a.lens_out && lane == 0) a.lens_out[r] = (int32_t)row_cols(a, src, r);
    const int64_t s0 = c0 / kTileTokens;
    const int64_t s1 = min(s0 + a.chunk_tiles, n);
    if (s1 > s0) scan_segment<F>(a, src, r, s0, (int)(s1 - s0), sb);
    if (!a.skip_tail) fill_neg_inf(a.logits + (int64_t)r * a.ld, max(c0, s1 * kTileTokens), c1);
  }
}

// ------------------------------------------------------------------ balanced scan
//
// Up to kBalancedMaxRows rows. The scored steps of all rows, in row order, are split into
// equal contiguous ranges, one per workgroup (one 8-wave workgroup per compute unit, so
// the ranges start and end together whatever the length mix). Inside a workgroup the
// waves do not take fixed shares: on each SIMD the older of its two waves issues first
// whenever both are ready and would finish its share well before the younger one. The
// range is cut instead into units of kUnit steps (never crossing a row) that the waves
// take from an LDS counter as they go; a wave issues the loads of its next step across
// unit boundaries, and looks up the table entries of its next unit one unit ahead.
// When the range fits the workgroup's LDS buffer (kBlockSteps steps) its scores stay
// there and leave in one burst at the end (or, for idx_select, never leave: see the
// one-pass selection below); a longer range is split evenly between the waves, each
// scoring its part in LDS-slice segments that are stored as they complete.

// Threads of a balanced workgroup: 8 waves, or 12 for MXFP4 keys, whose steps move half
// the bytes of fp8 ones and want more waves in flight (their kernels fit the 168 VGPRs
// that three waves per SIMD leave).
template <int F>
constexpr int bal_threads() {
  return F == FMT_MXFP4 ? 768 : 512;
}
constexpr int kBalMaxWaves = 768 / kWave;
constexpr int kUnit = 1;
constexpr int kBlockSteps = 512;   // steps a workgroup keeps in LDS: 128 KiB of scores
// Steps of a wave's LDS slice when the range does not fit: the slices share the buffer.
template <int NW>
constexpr int bal_slice_steps() {
  return kBlockSteps / NW >= kWave ? kWave : kBlockSteps / NW >= 32 ? 32 : 16;
}
constexpr int kMaxParts = kBalancedMaxRows;      // rows one range can meet
constexpr int kSpecSteps = 128;                  // idx_select: parts filtered at a speculative cut

// The rows meeting a workgroup's range, in order (built by wave 0).
struct BlockParts {
  int n, nunits;
  int r[kMaxParts];
  int rs0[kMaxParts];   // first step of the part within its row
  int rlen[kMaxParts];  // steps of the whole row
  int off[kMaxParts];   // first step of the part within the range
  int len[kMaxParts];   // steps of the part
  int ub[kMaxParts + 1];  // first unit of the part
};

// Step descriptors of a workgroup's LDS-resident range, step i of the range in slot i.
struct StepTab {
  int64_t kidx0[kBlockSteps];
  int32_t vlim[kBlockSteps];
  int32_t row[kBlockSteps];
};

// Block-wide: the descriptors of the range's n steps (one thread per step).
template <class Src>
__device__ __forceinline__ void build_steps(const ScanCommon& a, const Src& src, const BlockParts& P, int n,
                                            StepTab& T) {
  for (int t = threadIdx.x; t < n; t += blockDim.x) {
    int lo = 0, hi = P.n;  // the part holding step t: P.off[lo] <= t < P.off[lo + 1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (P.off[mid] <= t) lo = mid;
      else hi = mid;
    }
    const int r = P.r[lo];
    const auto R = src.row(r, a.ld, a.err, false);
    const StepDesc d = src.step(R, ((int64_t)P.rs0[lo] + (t - P.off[lo])) * kTileTokens, a.err);
    T.kidx0[t] = d.kidx0;
    T.vlim[t] = d.vlim;
    T.row[t] = r;
  }
}

// Scores the n steps of the range into buf (LDS, step i's 64 scores at buf + 64 i), taking
// units of kUnit consecutive steps from *ctr until none is left. A wave keeps the next unit
// taken one unit ahead and issues the loads of its next step across unit boundaries. With
// gmax, also the largest score of each 16 columns (step i's four at gmax + 4 i).
template <int F>
__device__ __forceinline__ void bal_stream(const ScanCommon& a, const StepTab& T, int n, uint32_t* ctr, float* buf,
                                           float* gmax) {
  const int lane = lane_id();
  const float NEG_INF = -__builtin_inff();
  const int nunits = (n + kUnit - 1) / kUnit;
  auto grab = [&]() __attribute__((always_inline)) -> int {
    int id = 0;
    if (lane == 0) id = (int)atomicAdd(ctr, 1u);
    return __builtin_amdgcn_readfirstlane(id);
  };
  int ucur = grab();
  if (ucur >= nunits) return;
  int unxt = grab();
  int sc = ucur * kUnit;  // the step being computed
  int qrow = T.row[sc];
  QOps<F> qo;
  float wr[4][4];
  auto load_qw = [&](int r) __attribute__((always_inline)) {
    qo.load(a.q, r, lane);
    const int g = lane >> 4;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float4 wv = *(const float4*)(a.w + (int64_t)r * kHeads + 16 * h + 4 * g);
      wr[h][0] = wv.x;
      wr[h][1] = wv.y;
      wr[h][2] = wv.z;
      wr[h][3] = wv.w;
    }
  };
  load_qw(qrow);
  KOps<F> ka[4], kb[4];
  float sca = 1.f, scb = 1.f;
  int32_t va = T.vlim[sc], vb = 0;
  if (va > 0) load_step<F>(ka, sca, a, T.kidx0[sc], va, lane);
  // computes step sc (keys in kc) after issuing the loads of the step after it into kn;
  // false when there is none
  auto phase = [&](KOps<F>(&kc)[4], float scc, int32_t vc, KOps<F>(&kn)[4], float& scn,
                   int32_t& vn) __attribute__((always_inline)) -> bool {
    int sn = sc + 1;
    if (sn >= n || sn % kUnit == 0) {  // the next unit's first step
      sn = unxt < nunits ? unxt * kUnit : -1;
      if (sn >= 0) unxt = grab();
    }
    vn = sn >= 0 ? T.vlim[sn] : 0;
    if (vn > 0) load_step<F>(kn, scn, a, T.kidx0[sn], vn, lane);
    const float v = vc > 0 ? score_step<F>(kc, scc, qo, wr) : NEG_INF;
    const float vs = lane < vc ? v : NEG_INF;
    buf[sc * kTileTokens + lane] = vs;
    if (gmax) {
      // the 16-lane row's maximum lands in its last lane (a lane without a source keeps
      // its own value)
      float m = vs;
      m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(m), __float_as_int(m), 0x111, 0xF, 0xF, false)));
      m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(m), __float_as_int(m), 0x112, 0xF, 0xF, false)));
      m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(m), __float_as_int(m), 0x114, 0xF, 0xF, false)));
      m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(m), __float_as_int(m), 0x118, 0xF, 0xF, false)));
      if ((lane & 15) == 15) gmax[sc * 4 + (lane >> 4)] = m;
    }
    if (sn < 0) return false;
    sc = sn;
    const int rn = T.row[sn];
    if (rn != qrow) {
      qrow = rn;
      load_qw(qrow);
    }
    return true;
  };
  for (;;) {
    if (!phase(ka, sca, va, kb, scb, vb)) break;
    if (!phase(kb, scb, vb, ka, sca, va)) break;
  }
}

// ------------------------------------------------------------------ one-pass selection
//
// idx_select on the balanced scan. After scoring its range (kept in LDS), a workgroup
// takes each row part in turn:
//   * the histogram of the part's group maxima (the largest order key of each group of
//     2^gshift columns) is built in LDS: 4096 fine bins of 16-bit counts in pairs (the
//     step table's space, free once the range is scored) and 256 coarse bins;
//   * a row inside the workgroup's range is cut at once from that histogram;
//   * a row shared with other workgroups (only the range's first and last can be) is
//     cut once each of the row's workgroups has published its histogram to its slot and
//     counted itself in the row's arrival counter: one wave per shared row adds up the
//     histograms of the row's slots, coarse bins first, while the other waves filter the
//     part at a speculative cut taken from its own histogram (almost surely at or below
//     the row's cut, checked once that is known; a part filtered too high, or without a
//     speculative cut, is filtered at the row's cut after);
//   * the cut is the lower edge of the fine bin holding the k-th largest group maximum,
//     so at least k groups, hence k entries, reach it; the part's entries at or above it
//     go, as selection keys (in any order), to the workgroup's region at the part's
//     first step * 64, the part's record (their count, the cut they reach, the largest of
//     them, the row's cut) to seg at the part's first step.
// Slots and counters are shared by all XCDs, so they are written and read with device-
// scope atomic operations only. A wait that runs past wait_ticks, or a row spanning more
// than kSelMaxSpan workgroups, keeps every entry of the part: correct in every case, only
// slower to finish. The arrival counters are never cleared: a workgroup waits for its
// row's counter to pass the value it read before scoring by the number of workgroups of
// the row (nothing of the row can have arrived then: arrivals follow a scored range).

__device__ __forceinline__ uint32_t atomic_ld(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_st(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The workgroup of the balanced split that holds step s (steps [total b / B,
// total (b + 1) / B) belong to workgroup b).
__device__ __forceinline__ int64_t sel_block_of(uint64_t s, uint64_t total, int64_t B) {
  return (int64_t)(((s + 1) * (uint64_t)B - 1) / total);
}

// One lane's float from the lane (lane ^ 1) or (lane ^ 2): DPP within each group of four.
template <int X>
__device__ __forceinline__ float quad_xor(float v) {
  static_assert(X == 1 || X == 2, "quad xor 1 or 2");
  constexpr int ctrl = X == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false));
}

// Block-wide, groups of 2^GS columns: adds the order key of each group's largest score
// (fmaxf passes over NaN) to the fine histogram. Consecutive lanes read consecutive
// float4s, four per thread in flight; a group of 8 or 16 columns spans 2 or 4 neighbouring
// lanes, whose butterfly leaves its largest score in each of them, so that lane j of a
// group can count the group of load j: every histogram add then has all lanes busy. n_ent
// is a multiple of 64, so a group's lanes are all in range or all out.
template <int GS>
__device__ __forceinline__ void sel_hist_groups(const float* sc, int64_t n_ent, uint32_t* hf) {
  constexpr int kU = 4;
  const int tid = threadIdx.x, lane = lane_id();
  const int64_t stride = 4 * (int64_t)blockDim.x;
  auto add = [&](float m) __attribute__((always_inline)) {
    const uint32_t mk = order_key(m);
    if (mk) {
      const uint32_t fb = mk >> 20;
      atomicAdd(&hf[fb >> 1], 1u << (16 * (fb & 1)));
    }
  };
  for (int64_t b0 = 0; b0 < n_ent; b0 += kU * stride) {
    float4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = b0 + u * stride + 4 * tid;
      v[u] = make_float4(-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff());
      if (i < n_ent) v[u] = *(const float4*)(sc + i);
    }
    if constexpr (GS == 0) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        add(v[u].x);
        add(v[u].y);
        add(v[u].z);
        add(v[u].w);
      }
    } else if constexpr (GS == 1) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        add(fmaxf(v[u].x, v[u].y));
        add(fmaxf(v[u].z, v[u].w));
      }
    } else {
      constexpr int R = 1 << (GS - 2);  // lanes per group
      float m[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        m[u] = fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w));
        if constexpr (GS >= 3) m[u] = fmaxf(m[u], quad_xor<1>(m[u]));
        if constexpr (GS >= 4) m[u] = fmaxf(m[u], quad_xor<2>(m[u]));
      }
      const int j = lane & (R - 1);
#pragma unroll
      for (int u0 = 0; u0 < kU; u0 += R) {
        float x = m[u0];
#pragma unroll
        for (int q = 1; q < R; ++q) x = j == q ? m[u0 + q] : x;
        add(x);
      }
    }
  }
}

// Block-wide: histogram (LDS: hf fine pairs, hc coarse) of the group maxima of the
// n_ent scores at sc (LDS or global; group i = entries i 2^gs .. (i + 1) 2^gs - 1).
__device__ __forceinline__ void sel_hist(const float* sc, int64_t n_ent, int gs, uint32_t* hf, uint32_t* hc,
                                         const float* gm = nullptr) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kSelFineBins / 2; i += blockDim.x) hf[i] = 0u;
  lds_barrier();
  if (gm && gs == 4) {
    // groups of 16 columns: their maxima were kept while scoring (gm, LDS)
    for (int64_t i = tid; i < n_ent / 16; i += blockDim.x) {
      const uint32_t mk = order_key(gm[i]);
      if (mk) {
        const uint32_t fb = mk >> 20;
        atomicAdd(&hf[fb >> 1], 1u << (16 * (fb & 1)));
      }
    }
  } else {
    switch (gs) {
      case 0: sel_hist_groups<0>(sc, n_ent, hf); break;
      case 1: sel_hist_groups<1>(sc, n_ent, hf); break;
      case 2: sel_hist_groups<2>(sc, n_ent, hf); break;
      case 3: sel_hist_groups<3>(sc, n_ent, hf); break;
      default: sel_hist_groups<4>(sc, n_ent, hf); break;
    }
  }
  lds_barrier();
  for (int c = tid; c < kSelCoarseBins; c += blockDim.x) {
    uint32_t t = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t w = hf[c * 8 + j];
      t += (w & 0xFFFFu) + (w >> 16);
    }
    hc[c] = t;
  }
  lds_barrier();
}

// Wave-wide, the coarse half of a cut: coarse4(c) gives lane l the coarse bins 255 - 4l ..
// 252 - 4l (highest first). Returns false when fewer than k groups are counted (the cut is
// then 1, every present entry); else the coarse bin holding the k-th largest group maximum
// and the count of the bins above it.
template <class Coarse4>
__device__ __forceinline__ bool sel_cut_coarse(uint32_t k, const Coarse4& coarse4, int& cbin, uint32_t& above) {
  const int lane = lane_id();
  uint32_t c[4];
  coarse4(c);
  const uint32_t t = c[0] + c[1] + c[2] + c[3];
  const uint32_t incl = wave_inclusive_sum(t);
  const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
  if (tot < k) return false;
  const uint32_t excl = incl - t;
  const uint64_t hit = __ballot(excl < k && k <= incl);
  const int hl = __builtin_ctzll(hit);
  int cb = 0;
  uint32_t ab = 0;
  if (lane == hl) {
    uint32_t cum = excl;
    bool found = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (!found && cum + c[j] >= k) {
        cb = kSelCoarseBins - 1 - 4 * lane - j;
        ab = cum;
        found = true;
      }
      cum += c[j];
    }
  }
  cbin = __builtin_amdgcn_readlane(cb, hl);
  above = (uint32_t)__builtin_amdgcn_readlane((int)ab, hl);
  return true;
}

// Wave-wide, the fine half: fine16(j) is the count of fine bin cbin * 16 + j. The cut is the
// lower edge of the fine bin holding the k-th largest group maximum.
template <class Fine16>
__device__ __forceinline__ uint32_t sel_cut_fine(uint32_t k, int cbin, uint32_t above, const Fine16& fine16) {
  const int lane = lane_id();
  const uint32_t f = lane < 16 ? fine16(15 - lane) : 0u;  // highest first
  const uint32_t fi = wave_inclusive_sum(f);
  const uint64_t fh = __ballot(lane < 16 && above + fi - f < k && k <= above + fi);
  if (!fh) return max((uint32_t)cbin << 24, 1u);  // counts out of step: the coarse edge is still a bound
  return max((uint32_t)(cbin * 16 + 15 - __builtin_ctzll(fh)) << 20, 1u);
}

// One lane: waits (bounded) until row r's arrival counter has moved `parts` past `base`.
__device__ __forceinline__ bool sel_wait(const SelectState& st, int r, unsigned long long base, int64_t parts) {
  const unsigned long long* p = st.arrive + r;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    const unsigned long long v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v - base >= (unsigned long long)parts) return true;
    if ((int64_t)(__builtin_amdgcn_s_memrealtime() - t0) > st.wait_ticks) return false;
    __builtin_amdgcn_s_sleep(8);
  }
}

// Wave-wide maximum (lanes without a source in a DPP row shift contribute 0).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));  // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));  // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));  // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));  // row_shr:8
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 15), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 47), d = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
  return max(max(a, b), max(c, d));
}

// Block-wide, as sel_filter for scores kept in LDS with their 16-column maxima gm: only the
// groups whose maximum reaches the cut are read. Those groups are listed first (list: LDS
// of n_ent / 16 entries, *lcount an LDS word), then their float4s are taken kI per thread,
// marked in a mask, counted over the block and written by each thread, as in sel_filter.
__device__ __forceinline__ uint32_t sel_filter_groups(const float* sc, const float* gm, int64_t n_ent, int64_t col0,
                                                      uint32_t T, uint64_t* out, uint16_t* list, uint32_t* lcount,
                                                      uint32_t* wsum, uint32_t* wmax, uint32_t* kmax) {
  constexpr int kI = 8;  // float4s per thread per pass
  const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave;
  const int nw = blockDim.x / kWave;
  const int nt = blockDim.x;
  const float t = T <= 1u ? -__FLT_MAX__ : key_value(T);
  const int ng = (int)(n_ent / 16);
  if (tid == 0) *lcount = 0u;
  lds_barrier();
  for (int g0 = 0; g0 < ng; g0 += nt) {
    const int g = g0 + tid;
    const bool take[1] = {g < ng && gm[g] >= t};
    const uint16_t item[1] = {(uint16_t)g};
    wave_append<1>(take, item, list, lcount, (uint32_t)ng);
  }
  lds_barrier();
  const int nq = 4 * (int)*lcount;  // float4s of the listed groups
  uint32_t done = 0;  // survivors of the earlier passes
  uint32_t mx = 0;    // this thread's largest survivor key
  for (int q0 = 0; q0 < nq; q0 += kI * nt) {
    uint32_t mask = 0;
#pragma unroll
    for (int v = 0; v < kI; ++v) {
      const int q = q0 + v * nt + tid;
      if (q < nq) {
        const float4 x = *(const float4*)(sc + 16 * list[q >> 2] + 4 * (q & 3));
        mask |= (x.x >= t ? 1u : 0u) << (4 * v);
        mask |= (x.y >= t ? 2u : 0u) << (4 * v);
        mask |= (x.z >= t ? 4u : 0u) << (4 * v);
        mask |= (x.w >= t ? 8u : 0u) << (4 * v);
      }
    }
    const uint32_t mine = (uint32_t)__popc(mask);
    const uint32_t incl = wave_inclusive_sum(mine);
    lds_barrier();  // wsum may still be read by the previous pass
    if (lane == kWave - 1) wsum[wv] = incl;
    lds_barrier();
    uint32_t before = incl - mine, tot = 0;
    for (int w = 0; w < nw; ++w) {
      const uint32_t v = wsum[w];
      before += w < wv ? v : 0u;
      tot += v;
    }
    uint64_t* o = out + done + before;
    while (mask) {
      const int bit = (int)__builtin_ctz(mask);
      mask &= mask - 1;
      const int q = q0 + (bit >> 2) * nt + tid;
      const int64_t i = 16 * (int64_t)list[q >> 2] + 4 * (q & 3) + (bit & 3);
      const uint32_t ok = order_key(sc[i]);
      mx = max(mx, ok);
      *o++ = ((uint64_t)ok << 32) | (uint32_t)(~(uint32_t)(col0 + i));
    }
    done += tot;
  }
  const uint32_t wm = wave_max_u32(mx);
  if (lane == 0) wmax[wv] = wm;
  lds_barrier();
  if (tid == 0) {
    uint32_t m = 0;
    for (int w = 0; w < nw; ++w) m = max(m, wmax[w]);
    *kmax = m;
  }
  return done;
}

// Block-wide: the n_ent scores at sc (columns col0 ..) at or above the cut T, as
// selection keys to out; returns their count, and to thread 0 in *kmax the largest order
// key among them (0 if none). An entry's order key is at least T exactly
// when its score is at least T's value (the order key is monotone; NaN compares false,
// -0 == +0); T = 1 keeps every present entry (-inf and NaN excluded). The entries go in
// chunks of 64 per thread: a thread marks which of its 64 (the float4s at 4 tid + v
// stride) survive in a 64-bit mask, the counts are scanned over the block (threads in
// order), and each thread writes its own survivors, reading back only those. n_ent is a
// multiple of 64.
__device__ __forceinline__ uint32_t sel_filter(const float* sc, int64_t n_ent, int64_t col0, uint32_t T,
                                               uint64_t* out, uint32_t* wsum, uint32_t* wmax, uint32_t* kmax) {
  constexpr int kV = 16;
  const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave;
  const int nw = blockDim.x / kWave;
  const int64_t stride = 4 * (int64_t)blockDim.x;
  const float t = T <= 1u ? -__FLT_MAX__ : key_value(T);
  uint32_t done = 0;  // survivors of the earlier chunks
  uint32_t mx = 0;    // this thread's largest survivor key
  for (int64_t c0 = 0; c0 < n_ent; c0 += kV * stride) {
    uint64_t mask = 0;
#pragma unroll
    for (int v = 0; v < kV; ++v) {
      const int64_t i = c0 + v * stride + 4 * tid;
      if (i < n_ent) {
        const float4 x = *(const float4*)(sc + i);
        mask |= (x.x >= t ? 1ull : 0ull) << (4 * v);
        mask |= (x.y >= t ? 2ull : 0ull) << (4 * v);
        mask |= (x.z >= t ? 4ull : 0ull) << (4 * v);
        mask |= (x.w >= t ? 8ull : 0ull) << (4 * v);
      }
    }
    const uint32_t mine = (uint32_t)__popcll(mask);
    const uint32_t incl = wave_inclusive_sum(mine);
    lds_barrier();  // wsum may still be read by the previous chunk or call
    if (lane == kWave - 1) wsum[wv] = incl;
    lds_barrier();
    uint32_t before = incl - mine, tot = 0;
    for (int w = 0; w < nw; ++w) {
      const uint32_t v = wsum[w];
      before += w < wv ? v : 0u;
      tot += v;
    }
    uint64_t* o = out + done + before;
    while (mask) {
      const int bit = (int)__builtin_ctzll(mask);
      mask &= mask - 1;
      const int64_t i = c0 + (bit >> 2) * stride + 4 * tid + (bit & 3);
      const uint32_t ok = order_key(sc[i]);
      mx = max(mx, ok);
      *o++ = ((uint64_t)ok << 32) | (uint32_t)(~(uint32_t)(col0 + i));
    }
    done += tot;
  }
  const uint32_t wm = wave_max_u32(mx);
  if (lane == 0) wmax[wv] = wm;
  lds_barrier();
  if (tid == 0) {
    uint32_t m = 0;
    for (int w = 0; w < nw; ++w) m = max(m, wmax[w]);
    *kmax = m;
  }
  return done;
}

// One wave: the cut of row r (as sel_cut over the sum of the slots of workgroups b_lo ..
// b_lo + nbb - 1, those with steps) once the row's counter has moved nb past base
// (bounded wait). 1 when the wait runs out or the row has fewer than k groups. Lane j
// finds slot j's index once (slot_of(bb) < 0: no steps). One round of loads takes the
// coarse bins of every slot (lane l: bins 255 - 4l .. 252 - 4l, eight slots in flight)
// and the fine bins of the four coarse bins pc - 1 .. pc + 2 around a predicted one (lane
// l: fine word l % 32 of them, of every other slot); when the coarse bin holding the k-th
// largest is not among them (or pc < 1), a second round takes its 16 fine bins.
template <class SlotOf>
__device__ __forceinline__ uint32_t sel_row_cut_wave(const SelectState& st, int r, unsigned long long base, int64_t nb,
                                                     int64_t b_lo, int nbb, const SlotOf& slot_of, int pc) {
  const int lane = lane_id();
  const int si0 = lane < nbb ? slot_of(b_lo + lane) : -1;
  int ok = 0;
  if (lane == 0) ok = sel_wait(st, r, base, nb) ? 1 : 0;
  if (!__builtin_amdgcn_readlane(ok, 0)) return 1u;
  // word w of the slot of index x (none: x < 0)
  auto word = [&](int x, int w) -> uint32_t { return x >= 0 ? atomic_ld(st.slots + (int64_t)x * kSelSlotWords + w) : 0u; };
  uint32_t c[4] = {0u, 0u, 0u, 0u};
  const int pw0 = 8 * (pc - 1);  // first fine word of the predicted coarse bins
  const bool pred = pc >= 1 && pc + 2 < kSelCoarseBins;
  uint32_t plo = 0, phi = 0;     // fine word pw0 + lane % 32 (its two counts) over slots lane / 32, + 2, ...
  for (int s0 = 0; s0 < nbb; s0 += kWave) {
    const int si = s0 == 0 ? si0 : (s0 + lane < nbb ? slot_of(b_lo + s0 + lane) : -1);
    const int ns = min(kWave, nbb - s0);
    constexpr int kS = 8;
    for (int j0 = 0; j0 < ns; j0 += kS) {
      uint32_t v[kS][4], fw[kS / 2];
#pragma unroll
      for (int u = 0; u < kS; ++u) {
        const int x = j0 + u < ns ? __builtin_amdgcn_readlane(si, j0 + u) : -1;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[u][q] = word(x, kSelFineBins / 2 + kSelCoarseBins - 1 - 4 * lane - q);
      }
#pragma unroll
      for (int u = 0; u < kS / 2; ++u) {
        const int j = j0 + 2 * u + (lane >> 5);
        const int x = __shfl(si, min(j, ns - 1));
        fw[u] = word(pred && j < ns ? x : -1, pw0 + (lane & 31));
      }
#pragma unroll
      for (int u = 0; u < kS; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) c[q] += v[u][q];
#pragma unroll
      for (int u = 0; u < kS / 2; ++u) {
        plo += fw[u] & 0xFFFFu;
        phi += fw[u] >> 16;
      }
    }
  }
  int cbin;
  uint32_t above;
  if (!sel_cut_coarse((uint32_t)st.k,
                      [&](uint32_t (&cc)[4]) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) cc[q] = c[q];
                      },
                      cbin, above))
    return 1u;
  plo += (uint32_t)__shfl_xor((int)plo, 32);
  phi += (uint32_t)__shfl_xor((int)phi, 32);
  if (pred && cbin >= pc - 1 && cbin <= pc + 2) {
    // fine bin j of cbin: half j % 2 of word 8 (cbin - pc + 1) + j / 2
    const int j = 15 - (lane & 15);  // this lane's bin
    const int src = 8 * (cbin - pc + 1) + (j >> 1);
    const uint32_t lo = (uint32_t)__shfl((int)plo, src), hi = (uint32_t)__shfl((int)phi, src);
    const uint32_t fr = (j & 1) ? hi : lo;
    return sel_cut_fine((uint32_t)st.k, cbin, above, [&](int) { return fr; });
  }
  const int fb = cbin * 16 + (lane & 15);
  uint32_t f = 0;
  for (int s0 = 0; s0 < nbb; s0 += kWave) {
    const int si = s0 == 0 ? si0 : (s0 + lane < nbb ? slot_of(b_lo + s0 + lane) : -1);
    const int ns = min(kWave, nbb - s0);
    // lane l: slots l / 16 + 4 i of this group of 64, 16 loads in flight
    uint32_t v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = 4 * i + (lane >> 4);
      const int x = __shfl(si, min(j, ns - 1));
      v[i] = word(j < ns ? x : -1, fb >> 1);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) f += (v[i] >> (16 * (fb & 1))) & 0xFFFFu;
  }
  f += (uint32_t)__shfl_xor((int)f, 16);
  f += (uint32_t)__shfl_xor((int)f, 32);
  const uint32_t fr = (uint32_t)__shfl((int)f, 15 - (lane & 15));  // bin 15 - lane % 16
  return sel_cut_fine((uint32_t)st.k, cbin, above, [&](int) { return fr; });
}

// Waves w .. w + nwv - 1 of the block (no block barrier): the n_ent scores at sc (columns
// col0 ..) at or above the cut T (T <= 1: every present entry, as sel_filter), as
// selection keys appended at out in any order (each wave takes its room from the LDS
// counter *cnt), their largest order key max'd into *kmx. With gm (each 16 columns'
// largest score, LDS) a lane takes a group of 16 and reads it only when its maximum
// reaches the cut; without, two float4s 64 apart.
template <bool GROUPS>
__device__ __forceinline__ void sel_filter_waves(const float* sc, const float* gm, int64_t n_ent, int64_t col0,
                                                 uint32_t T, uint64_t* out, uint32_t* cnt, uint32_t* kmx, int w,
                                                 int nwv) {
  constexpr int V = GROUPS ? 4 : 2;  // float4s of a lane's unit
  const int lane = lane_id();
  const float t = T <= 1u ? -__FLT_MAX__ : key_value(T);
  const int nu = (int)(n_ent / (4 * V));  // units
  uint32_t mx = 0;
  for (int u0 = w * kWave; u0 < nu; u0 += nwv * kWave) {
    const int u = u0 + lane;
    // entry j of the lane's unit: GROUPS: 16 u + j; else float4 (u0 V + lane + 64 (j / 4)), item j % 4
    auto at = [&](int j) -> int64_t {
      return GROUPS ? 16 * (int64_t)u + j : 4 * ((int64_t)u0 * V + lane + kWave * (j >> 2)) + (j & 3);
    };
    uint32_t m = 0;
    if (GROUPS ? u < nu && gm[u] >= t : true) {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        if (!GROUPS && u0 * V + lane + kWave * v >= V * nu) continue;
        const float4 x = *(const float4*)(sc + at(4 * v));
        m |= (x.x >= t ? 1u : 0u) << (4 * v);
        m |= (x.y >= t ? 2u : 0u) << (4 * v);
        m |= (x.z >= t ? 4u : 0u) << (4 * v);
        m |= (x.w >= t ? 8u : 0u) << (4 * v);
      }
    }
    const uint32_t c = (uint32_t)__popc(m);
    const uint32_t incl = wave_inclusive_sum(c);
    const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
    if (tot == 0) continue;
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(cnt, tot);
    base = (uint32_t)__builtin_amdgcn_readlane((int)base, 0);
    uint64_t* o = out + base + incl - c;
    while (m) {
      const int j = (int)__builtin_ctz(m);
      m &= m - 1;
      const int64_t i = at(j);
      const uint32_t ok = order_key(sc[i]);
      mx = max(mx, ok);
      *o++ = ((uint64_t)ok << 32) | (uint32_t)(~(uint32_t)(col0 + i));
    }
  }
  const uint32_t wm = wave_max_u32(mx);
  if (lane == 0 && wm) atomicMax(kmx, wm);
}

// ------------------------------------------------------------------ balanced kernel

template <int F, class Src, bool SELECT>
__global__ __launch_bounds__(bal_threads<F>()) void scan_bal_kernel(ScanCommon a, Src src, SelectState st) {
  constexpr int kBalThreads = bal_threads<F>();
  constexpr int kBalWaves = kBalThreads / kWave;
  constexpr int kSlice = bal_slice_steps<kBalWaves>();
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wib = tid / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * kBalWaves;
  const int64_t wave = (int64_t)blockIdx.x * kBalWaves + wib;
  const int64_t B = gridDim.x, b = blockIdx.x;
  __shared__ __align__(16) float buf[kBlockSteps * kTileTokens];
  __shared__ BlockParts P;
  __shared__ StepTab T;
  __shared__ uint32_t ctr;
  __shared__ unsigned long long sbase[2];
  __shared__ uint32_t hc[SELECT ? kSelCoarseBins : 1];
  __shared__ uint32_t wsum[kBalWaves], wmax[kBalWaves];
  __shared__ float gmax[SELECT ? kBlockSteps * 4 : 1];  // idx_select: each 16 columns' largest score
  __shared__ uint32_t s_lcount;
  __shared__ uint32_t s_T, s_ok, s_kmax;
  __shared__ int s_sp[2];                                            // idx_select: the shared parts
  __shared__ uint32_t s_spec[2], s_T2[2], s_cnt2[2], s_kmax2[2];   // and their speculative cuts
  __shared__ int s_pc[2];                                           // and predicted coarse bins
  if (!SELECT && a.zero) {
    const int64_t per = (a.zero_words + nwaves - 1) / nwaves;
    const int64_t z1 = min(a.zero_words, (wave + 1) * per);
    for (int64_t i = wave * per + lane; i < z1; i += kWave) a.zero[i] = 0u;
  }

  // total scored steps; wave 0 of workgroup 0 reports bad row metadata, the rows' scored
  // lengths and (idx_select) each row's first step
  const bool first = b == 0 && wib == 0;
  uint64_t total = 0;
  // scores alone: each lane's row steps of every 64-row pass stay in registers for the
  // parts below (the launch takes at most kBalancedMaxRows rows: kPasses passes; measured
  // 0.2-0.6 us off the two-level and batched scans, and no gain beyond noise for
  // idx_select's one pass, which reads them again)
  constexpr int kPasses = kBalancedMaxRows / kWave;
  uint32_t nk[kPasses];
  for (int r0 = 0; r0 < a.rows; r0 += kWave) {
    const int r = r0 + lane;
    const uint32_t n = r < a.rows ? (uint32_t)row_steps(a, src, r, first) : 0u;
    if constexpr (!SELECT) {
#pragma unroll
      for (int i = 0; i < kPasses; ++i)
        if (r0 == i * kWave) nk[i] = n;
    }
    const uint32_t incl = wave_inclusive_sum(n);
    if (first && r < a.rows) {
      if (a.lens_out) a.lens_out[r] = (int32_t)row_cols(a, src, r);
      if (SELECT) st.acc[r] = (int64_t)(total + incl - n);
    }
    total += (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
  }
  if (SELECT && first && lane == 0) st.acc[a.rows] = (int64_t)total;
  const uint64_t beg = total * (uint64_t)b / (uint64_t)B;
  const uint64_t end = total * (uint64_t)(b + 1) / (uint64_t)B;
  const bool resident = end - beg <= (uint64_t)kBlockSteps;

  // the rows meeting [beg, end); units of kUnit steps over them
  if (wib == 0) {
    uint64_t acc = 0;
    int np = 0;
    for (int r0 = 0; r0 < a.rows && acc < end; r0 += kWave) {
      const int r = r0 + lane;
      uint32_t n = 0u;
      if constexpr (SELECT) {
        n = r < a.rows ? (uint32_t)row_steps(a, src, r, false) : 0u;
      } else {
#pragma unroll
        for (int i = 0; i < kPasses; ++i)
          if (r0 == i * kWave) n = nk[i];
      }
      const uint32_t incl = wave_inclusive_sum(n);
      const uint64_t s = acc + incl - n, e = acc + incl;
      const uint64_t lo = max(s, beg), hi = min(e, end);
      const bool meet = r < a.rows && lo < hi;
      const uint64_t m = __ballot(meet);
      if (meet) {
        const int p = np + (int)lanes_below(m);
        P.r[p] = r;
        P.rs0[p] = (int)(lo - s);
        P.rlen[p] = (int)n;
        P.off[p] = (int)(lo - beg);
        P.len[p] = (int)(hi - lo);
      }
      np += (int)__popcll(m);
      acc += (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
    }
    int ub = 0;
    for (int p0 = 0; p0 < np; p0 += kWave) {
      const int p = p0 + lane;
      const uint32_t u = p < np ? (uint32_t)((P.len[p] + kUnit - 1) / kUnit) : 0u;
      const uint32_t incl = wave_inclusive_sum(u);
      if (p < np) P.ub[p] = ub + (int)(incl - u);
      ub += (int)__builtin_amdgcn_readlane((int)incl, kWave - 1);
    }
    if (lane == 0) {
      P.n = np;
      P.nunits = ub;
      P.ub[np] = ub;
      ctr = 0;
    }
  }
  __syncthreads();
  const int np = P.n;

  // idx_select: the arrival counters of the first and last rows, when shared with other
  // workgroups, read before scoring
  if constexpr (SELECT) {
    if (tid < 2 && np > 0) {
      const int p = tid == 0 ? 0 : np - 1;
      sbase[tid] = __hip_atomic_load(st.arrive + P.r[p], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // score the range
  if (resident) {
    build_steps(a, src, P, (int)(end - beg), T);
    __syncthreads();
    // idx_select with groups of 16 columns keeps their maxima while scoring: the histogram
    // then reads those, and the filter reads only the groups that reach the cut (with
    // smaller groups the cut passes most 16-column groups and this does not pay)
    bal_stream<F>(a, T, (int)(end - beg), &ctr, buf, SELECT && st.gshift == 4 ? gmax : nullptr);
    __syncthreads();
    if constexpr (!SELECT) {
      // the range's scores to their rows, four per thread per store
      for (int p = 0; p < np; ++p) {
        const int64_t c0 = (int64_t)P.rs0[p] * kTileTokens;
        const int64_t cnt = min((int64_t)P.len[p] * kTileTokens, a.ld - c0);
        float* o = a.logits + (int64_t)P.r[p] * a.ld + c0;
        const float* sp = buf + P.off[p] * kTileTokens;
        const bool vec = ((uintptr_t)o & 15) == 0;
        for (int64_t i = 4 * tid; i < cnt; i += 4 * kBalThreads) {
          const float4 v = *(const float4*)(sp + i);
          if (vec && i + 4 <= cnt) {
            *(float4*)(o + i) = v;
          } else {
            o[i] = v.x;
            if (i + 1 < cnt) o[i + 1] = v.y;
            if (i + 2 < cnt) o[i + 2] = v.z;
            if (i + 3 < cnt) o[i + 3] = v.w;
          }
        }
      }
    }
  } else {
    // too long for LDS: each wave an equal part of the range, in stored slice segments
    const uint64_t wbeg = beg + (end - beg) * wib / kBalWaves, wend = beg + (end - beg) * (wib + 1) / kBalWaves;
    float* sl = buf + wib * kSlice * kTileTokens;
    for (int p = 0; p < np; ++p) {
      const uint64_t ps = beg + P.off[p], pe = ps + P.len[p];
      const uint64_t lo = max(ps, wbeg), hi = min(pe, wend);
      for (uint64_t s0 = lo; s0 < hi; s0 += kSlice) {
        const int n = (int)min((uint64_t)kSlice, hi - s0);
        scan_segment<F>(a, src, P.r[p], (int64_t)(s0 - ps) + P.rs0[p], n, sl);
      }
    }
  }

  if constexpr (SELECT) {
    static_assert(sizeof(StepTab) >= kSelFineBins * 2, "the fine histogram reuses the step table");
    uint32_t* hf = (uint32_t*)&T;
    const bool use_gmax = resident && st.gshift == 4;  // the maxima of 16 columns were kept
    if (tid < 2) {
      s_sp[tid] = -1;
      s_spec[tid] = 0u;
      s_pc[tid] = -1;
    }
    __syncthreads();
    // f(scores of part p): in LDS, or in the spill rows. Two calls, so that each inlined
    // copy reads through a pointer of known memory (a pointer that may be either takes
    // generic loads, which wait like global ones)
    auto with_scores = [&](int p, auto&& f) __attribute__((always_inline)) {
      if (resident) f(buf + P.off[p] * kTileTokens);
      else f(st.spill + (int64_t)P.r[p] * a.ld + (int64_t)P.rs0[p] * kTileTokens);
    };
    auto row_first = [&](int p) -> uint64_t { return beg + P.off[p] - P.rs0[p]; };
    // the row of part p spans workgroups b_lo..b_hi; returns how many of them hold steps
    // (with fewer steps than workgroups some hold none, and every other one holds one step)
    auto span = [&](int p, int64_t& b_lo, int64_t& b_hi) -> int64_t {
      const uint64_t acc_r = row_first(p);
      b_lo = sel_block_of(acc_r, total, B);
      b_hi = sel_block_of(acc_r + P.rlen[p] - 1, total, B);
      return total >= (uint64_t)B ? b_hi - b_lo + 1 : (int64_t)P.rlen[p];
    };
    auto bbeg = [&](int64_t bb) -> uint64_t { return total * (uint64_t)bb / (uint64_t)B; };
    auto has_steps = [&](int64_t bb) -> bool { return bbeg(bb + 1) > bbeg(bb); };
    auto surv_of = [&](int p) -> uint64_t* { return st.surv + (int64_t)(beg + P.off[p]) * kTileTokens; };
    // publish the histograms of the shared first and last rows (one store drain for both),
    // then count this workgroup in their arrival counters. A part held in LDS also gets a
    // speculative cut: the lower edge of the fine bin of its own m-th largest group
    // maximum. The row's cut is the lower edge of the fine bin holding the row's k-th
    // largest, so fewer than k of the row's groups lie in higher bins, about share * k of
    // them in this part; m = share * k + 4 sqrt(share * k) + 8 puts the speculative cut
    // at or below the row's cut but for a deviation of four standard deviations (then the
    // part is filtered again). None (0) for a part of fewer than kSpecSteps steps, whose
    // filter after the cut is short, or when m passes 3/4 of the part's groups (too many
    // survivors): those parts are filtered at the row's cut once it is known
    // which of the first and last parts are shared (and published)
    auto shared_part = [&](int which) -> int {
      const int p = which == 0 ? 0 : np - 1;
      if (np == 0 || (which == 1 && np == 1)) return -1;
      int64_t b_lo, b_hi;
      const int64_t nb = span(p, b_lo, b_hi);
      return nb <= 1 || nb > kSelMaxSpan || !st.cutoff ? -1 : p;
    };
    const int sp0 = shared_part(0), sp1 = shared_part(1);
    // wave w, from the histogram of shared part `which` in f / c: the coarse bin of its own
    // share of the row's k-th largest group maximum (the row's cut is most likely in it or
    // next to it), and the speculative cut
    auto spec_cut = [&](int which, int w, const uint32_t* f, const uint32_t* c) {
      const int p = which == 0 ? sp0 : sp1;
      if (wib != w) return;
      const int64_t n_ent = (int64_t)P.len[p] * kTileTokens;
      const uint64_t groups = (uint64_t)n_ent >> st.gshift;
      const uint64_t row_groups = ((uint64_t)P.rlen[p] * kTileTokens) >> st.gshift;
      const float share = (float)st.k * (float)groups / (float)row_groups;
      auto coarse4 = [&](uint32_t (&cc)[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) cc[q] = c[kSelCoarseBins - 1 - 4 * lane - q];
      };
      int cbin;
      uint32_t above;
      const bool pc = sel_cut_coarse((uint32_t)max(share + 0.5f, 1.f), coarse4, cbin, above);
      if (lane == 0) s_pc[which] = pc ? cbin : -1;
      const uint64_t m = (uint64_t)(share + 4.f * __builtin_sqrtf(share)) + 8;
      uint32_t ts = 0u;
      if (resident && P.len[p] >= kSpecSteps && 4 * m < 3 * groups && sel_cut_coarse((uint32_t)m, coarse4, cbin, above))
        ts = sel_cut_fine((uint32_t)m, cbin, above, [&](int q) {
          const int fb = cbin * 16 + q;
          return (f[fb >> 1] >> (16 * (fb & 1))) & 0xFFFFu;
        });
      if (lane == 0) s_spec[which] = ts > 1u ? ts : 0u;
    };
    // the last part's histogram goes past the range's scores in buf when they leave room
    // (both histograms then stand until the speculative cuts are taken after the arrival
    // counters move); else it replaces the first part's, whose speculative cut is taken
    // before
    const bool room = resident && (end - beg) * kTileTokens + kSelFineBins / 2 + kSelCoarseBins <=
                                      (uint64_t)kBlockSteps * kTileTokens;
    uint32_t* hf1 = room ? (uint32_t*)(buf + (end - beg) * kTileTokens) : hf;
    uint32_t* hc1 = room ? hf1 + kSelFineBins / 2 : hc;
    for (int which = 0; which < 2; ++which) {
      const int p = which == 0 ? sp0 : sp1;
      if (p < 0) continue;
      uint32_t* f = which == 0 ? hf : hf1;
      uint32_t* c = which == 0 ? hc : hc1;
      const int64_t n_ent = (int64_t)P.len[p] * kTileTokens;
      with_scores(p, [&](const float* sc) {
        sel_hist(sc, n_ent, st.gshift, f, c, use_gmax ? gmax + 4 * P.off[p] : nullptr);
      });
      uint32_t* slot = st.slots + (b * 2 + which) * (int64_t)kSelSlotWords;
      for (int i = tid; i < kSelFineBins / 2; i += kBalThreads) atomic_st(slot + i, f[i]);
      for (int i = tid; i < kSelCoarseBins; i += kBalThreads) atomic_st(slot + kSelFineBins / 2 + i, c[i]);
      if (tid == 0) s_sp[which] = p;
      if (which == 0 && sp1 >= 0 && !room) {
        spec_cut(0, 0, hf, hc);
        lds_barrier();  // the stores and the speculative cut have read hf and hc
      }
    }
    if (sp0 >= 0 || sp1 >= 0) {
      __builtin_amdgcn_s_waitcnt(0);  // the slots are written before the workgroup counts itself
      __syncthreads();
      if (tid < 2 && s_sp[tid] >= 0)
        (void)__hip_atomic_fetch_add(st.arrive + P.r[s_sp[tid]], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (sp1 < 0) spec_cut(0, 0, hf, hc);
      else if (room && sp0 >= 0) {
        spec_cut(0, 0, hf, hc);
        spec_cut(1, 1, hf1, hc1);
      } else
        spec_cut(1, 0, hf1, hc1);
      lds_barrier();
    }
    // the parts not shared with other workgroups, one after the other
    for (int p = 0; p < np; ++p) {
      if (p == s_sp[0] || p == s_sp[1]) continue;
      int64_t b_lo, b_hi;
      const int64_t nb = span(p, b_lo, b_hi);
      const int64_t n_ent = (int64_t)P.len[p] * kTileTokens;
      if (nb == 1 && !st.cutoff) {
        if (tid == 0) {
          s_T = 1u;
          s_ok = 0u;
        }
      } else if (nb == 1) {
        // the whole row is here
        with_scores(p, [&](const float* sc) {
          sel_hist(sc, n_ent, st.gshift, hf, hc, use_gmax ? gmax + 4 * P.off[p] : nullptr);
        });
        if (wib == 0) {
          int cbin;
          uint32_t above, T2 = 1u;
          if (sel_cut_coarse(
                  (uint32_t)st.k,
                  [&](uint32_t (&c)[4]) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) c[j] = hc[kSelCoarseBins - 1 - 4 * lane - j];
                  },
                  cbin, above))
            T2 = sel_cut_fine((uint32_t)st.k, cbin, above, [&](int j) {
              const int f = cbin * 16 + j;
              return (hf[f >> 1] >> (16 * (f & 1))) & 0xFFFFu;
            });
          if (lane == 0) {
            s_T = T2;
            s_ok = 1;
          }
        }
      } else if (tid == 0) {
        s_T = 1u;  // no cutoff, or too many workgroups: every entry survives
        s_ok = 0u;
      }
      lds_barrier();
      uint32_t cnt;
      const int64_t col0 = (int64_t)P.rs0[p] * kTileTokens;
      uint64_t* so = surv_of(p);
      if (use_gmax)  // the group list reuses the step table's space (the cut is done with it)
        cnt = sel_filter_groups(buf + P.off[p] * kTileTokens, gmax + 4 * P.off[p], n_ent, col0, s_T, so,
                                (uint16_t*)&T, &s_lcount, wsum, wmax, &s_kmax);
      else
        with_scores(p, [&](const float* sc) { cnt = sel_filter(sc, n_ent, col0, s_T, so, wsum, wmax, &s_kmax); });
      if (tid == 0) st.seg[beg + P.off[p]] = make_uint4(cnt | (s_ok ? 0u : kSegNoCut), s_T, s_kmax, s_T);
      lds_barrier();
    }
    // the shared parts: waves 0 and 1 cut the first and the last part's row from the slots
    // while the other waves filter the parts that have a speculative cut at it; a part
    // without one, or whose row cut comes out below it, is filtered at the row cut after
    if (s_sp[0] >= 0 || s_sp[1] >= 0) {
      if (tid < 2) {
        s_cnt2[tid] = 0u;
        s_kmax2[tid] = 0u;
        s_T2[tid] = 1u;
      }
      lds_barrier();
      if (wib < 2) {
        const int which = wib;
        if (s_sp[which] >= 0) {
          const int p = s_sp[which];
          int64_t b_lo, b_hi;
          const int64_t nb = span(p, b_lo, b_hi);
          const uint32_t tr =
              sel_row_cut_wave(st, P.r[p], sbase[which], nb, b_lo, (int)(b_hi - b_lo + 1),
                               // the slot of part p's row in workgroup bb: slot 1 of a workgroup
                               // where the row starts inside the range (that range's last
                               // row), slot 0 where it covers the range's start
                               [&](int64_t bb) -> int {
                                 return has_steps(bb) ? (int)(bb * 2 + (row_first(p) > bbeg(bb) ? 1 : 0)) : -1;
                               },
                               s_pc[which]);
          if (lane == 0) s_T2[which] = tr;
        }
      } else {
        for (int which = 0; which < 2; ++which) {
          if (!s_spec[which]) continue;
          const int p = s_sp[which];
          const int64_t n_ent = (int64_t)P.len[p] * kTileTokens, col0 = (int64_t)P.rs0[p] * kTileTokens;
          if (use_gmax)
            sel_filter_waves<true>(buf + P.off[p] * kTileTokens, gmax + 4 * P.off[p], n_ent, col0, s_spec[which],
                                   surv_of(p), &s_cnt2[which], &s_kmax2[which], wib - 2, kBalWaves - 2);
          else
            sel_filter_waves<false>(buf + P.off[p] * kTileTokens, nullptr, n_ent, col0, s_spec[which], surv_of(p),
                                    &s_cnt2[which], &s_kmax2[which], wib - 2, kBalWaves - 2);
        }
      }
      lds_barrier();
      // the parts without a speculative cut, or whose row cut came out below it, at the
      // row cut by all waves
      auto refilter = [&](int which) { return s_sp[which] >= 0 && (!s_spec[which] || s_T2[which] < s_spec[which]); };
      if (tid < 2 && refilter(tid)) {
        s_cnt2[tid] = 0u;
        s_kmax2[tid] = 0u;
      }
      lds_barrier();
      for (int which = 0; which < 2; ++which) {
        if (!refilter(which)) continue;
        const int p = s_sp[which];
        const int64_t n_ent = (int64_t)P.len[p] * kTileTokens, col0 = (int64_t)P.rs0[p] * kTileTokens;
        if (use_gmax)
          sel_filter_waves<true>(buf + P.off[p] * kTileTokens, gmax + 4 * P.off[p], n_ent, col0, s_T2[which],
                                 surv_of(p), &s_cnt2[which], &s_kmax2[which], wib, kBalWaves);
        else
          with_scores(p, [&](const float* sc) {
            sel_filter_waves<false>(sc, nullptr, n_ent, col0, s_T2[which], surv_of(p), &s_cnt2[which],
                                    &s_kmax2[which], wib, kBalWaves);
          });
      }
      lds_barrier();
      if (tid < 2 && s_sp[tid] >= 0) {
        const uint32_t tr = s_T2[tid];
        st.seg[beg + P.off[s_sp[tid]]] =
            make_uint4(s_cnt2[tid] | (tr > 1u ? 0u : kSegNoCut), refilter(tid) ? tr : s_spec[tid], s_kmax2[tid], tr);
      }
    }
  } else if (!a.skip_tail) {
    // -inf past each row's scored steps, in 4096-column pieces spread over all waves
    constexpr int64_t kFill = 4096;
    const int64_t pieces = (a.ld + kFill - 1) / kFill;
    for (int64_t it = wave; it < pieces * a.rows; it += nwaves) {
      const int r = (int)(it % a.rows);
      const int64_t f0 = (it / a.rows) * kFill;
      const int64_t from = row_steps(a, src, r, false) * kTileTokens;
      fill_neg_inf(a.logits + (int64_t)r * a.ld, max(f0, from), min(f0 + kFill, a.ld));
    }
  }
}

// ------------------------------------------------------------------ launcher

// Launch shape: the grid holds exactly the workgroups that are resident at once (from
// the occupancy of each kernel instance on the current device), so no workgroup starts
// late and becomes a tail.
enum SchedKind { SCHED_ITEMS = 0, SCHED_BALANCED = 1, SCHED_SELECT = 2 };

template <int F, class Src, int KIND>
static const void* scan_fn() {
  if constexpr (KIND == SCHED_ITEMS) return (const void*)scan_items_kernel<F, Src>;
  else return (const void*)scan_bal_kernel<F, Src, KIND == SCHED_SELECT>;
}

template <int F, int KIND>
constexpr int sched_threads() {
  return KIND == SCHED_ITEMS ? kBlock : bal_threads<F>();
}

template <int F, class Src, int KIND>
static int resident_blocks_per_cu() {
  static std::mutex mu;
  static int cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  if (!cache[dev]) {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, scan_fn<F, Src, KIND>(), sched_threads<F, KIND>(), 0) !=
            hipSuccess ||
        b <= 0)
      b = 1;
    cache[dev] = b;
  }
  return cache[dev];
}

template <int F, class Src, int KIND>
static int64_t sched_blocks() {
  return (int64_t)device_cu_count() * resident_blocks_per_cu<F, Src, KIND>();
}

template <int F, class Src, int KIND>
static hipError_t run_sched(const ScoreCall& c, const Src& src, hipStream_t stream) {
  int64_t blocks = sched_blocks<F, Src, KIND>();
  const int64_t waves_total = blocks * (sched_threads<F, KIND>() / kWave);
  const int64_t tiles_per_row = (c.ld + kTileTokens - 1) / kTileTokens;
  const int64_t tiles = tiles_per_row * c.rows;
  int64_t ct = tiles / (2 * waves_total);
  constexpr int kMaxSteps = max_steps<F>();
  ct = ct < 1 ? 1 : (ct > kMaxSteps ? kMaxSteps : ct);
  const int64_t chunks = (tiles_per_row + ct - 1) / ct;
  ScanCommon a;
  a.q = c.q;
  a.w = c.w;
  a.k = c.k;
  a.k_scale = c.k_scale;
  a.logits = c.logits;
  a.ld = c.ld;
  a.rows = c.rows;
  a.chunk_tiles = (int)ct;
  a.n_items = chunks * c.rows;
  a.err = c.err;
  a.skip_tail = c.skip_tail;
  a.zero = c.zero;
  a.zero_words = c.zero_words;
  a.lens_out = c.lens_out;
  if constexpr (KIND == SCHED_ITEMS) {
    const int64_t need = (a.n_items + (kBlock / kWave) - 1) / (kBlock / kWave);
    if (blocks > need) blocks = need;
    hipLaunchKernelGGL((scan_items_kernel<F, Src>), dim3((unsigned)blocks), dim3(kBlock), 0, stream, a, src);
  } else if constexpr (KIND == SCHED_SELECT) {
    a.logits = c.sel->spill;
    hipLaunchKernelGGL((scan_bal_kernel<F, Src, true>), dim3((unsigned)blocks), dim3(bal_threads<F>()), 0, stream, a,
                       src, *c.sel);
  } else {
    hipLaunchKernelGGL((scan_bal_kernel<F, Src, false>), dim3((unsigned)blocks), dim3(bal_threads<F>()), 0, stream,
                       a, src, SelectState{});
  }
  return hipGetLastError();
}

template <int F, class Src>
static hipError_t run(const ScoreCall& c, const Src& src, hipStream_t stream) {
  if (c.rows <= kBalancedMaxRows) {
    if (c.sel) return run_sched<F, Src, SCHED_SELECT>(c, src, stream);
    return run_sched<F, Src, SCHED_BALANCED>(c, src, stream);
  }
  return run_sched<F, Src, SCHED_ITEMS>(c, src, stream);
}

template <class Src>
static hipError_t run_fmt(const ScoreCall& c, const Src& src, hipStream_t stream) {
  switch (c.fmt) {
    case FMT_FP8: return run<FMT_FP8>(c, src, stream);
    case FMT_MXFP4: return run<FMT_MXFP4>(c, src, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_score(const ScoreCall& c, hipStream_t stream) {
  if (c.rows <= 0 || c.ld <= 0) return hipSuccess;
  switch (c.source) {
    case SRC_DENSE: {
      if (prefill_applies(c)) return launch_prefill(c, stream);
      DenseSrc s{c.row_ks, c.row_ke, c.n_keys};
      if (c.fmt == FMT_BF16) return run<FMT_BF16>(c, s, stream);
      return run_fmt(c, s, stream);
    }
    case SRC_PAGED: {
      PagedSrc s{c.block_table, c.bt_rows, c.bt_ld, c.seq_lens, c.row_req, c.n_keys, c.page_size};
      return run_fmt(c, s, stream);
    }
    case SRC_SPARSE: {
      SparseSrc s{c.row_ks, c.row_ke, c.n_keys, c.cand, c.cand_ld, c.n_cols, c.block};
      return run_fmt(c, s, stream);
    }
    case SRC_PAGED_SPARSE: {
      PagedSparseSrc s{c.block_table, c.bt_rows, c.bt_ld, c.seq_lens, c.row_req, c.n_keys, c.page_size,
                       c.cand, c.cand_ld, c.n_cols, c.block};
      return run_fmt(c, s, stream);
    }
  }
  return hipErrorInvalidValue;
}

int64_t select_scan_blocks(const ScoreCall& c) {
  if (c.rows <= 0 || c.rows > kBalancedMaxRows) return 0;
  if (c.source == SRC_DENSE && prefill_applies(c)) return 0;
  switch (c.fmt) {
    case FMT_BF16:
      return c.source == SRC_DENSE ? sched_blocks<FMT_BF16, DenseSrc, SCHED_SELECT>() : 0;
    case FMT_FP8:
      switch (c.source) {
        case SRC_PAGED: return sched_blocks<FMT_FP8, PagedSrc, SCHED_SELECT>();
        case SRC_SPARSE: return sched_blocks<FMT_FP8, SparseSrc, SCHED_SELECT>();
        case SRC_PAGED_SPARSE: return sched_blocks<FMT_FP8, PagedSparseSrc, SCHED_SELECT>();
        default: return sched_blocks<FMT_FP8, DenseSrc, SCHED_SELECT>();
      }
    case FMT_MXFP4:
      switch (c.source) {
        case SRC_PAGED: return sched_blocks<FMT_MXFP4, PagedSrc, SCHED_SELECT>();
        case SRC_SPARSE: return sched_blocks<FMT_MXFP4, SparseSrc, SCHED_SELECT>();
        case SRC_PAGED_SPARSE: return sched_blocks<FMT_MXFP4, PagedSparseSrc, SCHED_SELECT>();
        default: return sched_blocks<FMT_MXFP4, DenseSrc, SCHED_SELECT>();
      }
  }
  return 0;
}

// ------------------------------------------------------------------ per-device state

__device__ unsigned g_device_errors;

static std::mutex g_mu;
static unsigned* g_err_ptr[kMaxDevices];
static int g_cus[kMaxDevices];

unsigned* device_error_word() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_err_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_device_errors)) != hipSuccess) return nullptr;
    g_err_ptr[dev] = (unsigned*)p;
  }
  return g_err_ptr[dev];
}

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cus[dev] = n;
  }
  return g_cus[dev];
}

}  // namespace dsaidx
