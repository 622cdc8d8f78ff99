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
};

// ------------------------------------------------------------------ key sources
//
// Pages and candidate blocks hold a multiple of 64 keys and steps start at multiples
// of 64 positions, so the 64 positions of a step name 64 consecutive key rows. A
// source describes step s of a row by its first key row and by how many leading
// positions of the step are scored (its valid prefix, <= 0 when none is).

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
  __device__ StepDesc step(const Row& R, int64_t pos0, unsigned*) const {
    return {R.base + pos0, (int32_t)min(R.len - pos0, (int64_t)kTileTokens)};
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
  __device__ StepDesc step(const Row& R, int64_t pos0, unsigned* err) const {
    if (pos0 >= R.len) return {0, 0};
    int64_t pg = R.bt_row[pos0 / page];
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
  __device__ StepDesc step(const Row& R, int64_t pos0, unsigned* err) const {
    if (pos0 >= R.ncols) return {0, 0};
    const int64_t cb = R.cand_row[pos0 / block];
    if (cb < 0) {
      flag_error(err, kErrBlock);
      return {0, 0};
    }
    const int64_t tok0 = cb * block + pos0 % block;
    const int64_t v = min(min(R.ncols - pos0, R.len - tok0), (int64_t)kTileTokens);
    return {R.base + (v > 0 ? tok0 : 0), (int32_t)v};
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
// Row counts up to this take the balanced schedule (every wave reads all row lengths).
static constexpr int kBalancedMaxRows = 512;

// Scores steps [s0, s0 + nsteps) of row r (nsteps <= max_steps<F>()) and writes their
// columns, clipped to ld. sb: the wave's LDS slice of max_steps<F>() * 64 floats.
template <int F, class Src>
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

// BALANCED: every wave sums the scored steps of all rows and takes an equal
// contiguous share of them (crossing rows where needed), in segments of at most
// max_steps<F>() steps, so all waves finish together whatever the row lengths; then the
// columns past each row's scored steps are filled with -inf in 4096-column pieces
// (unless skip_tail). Otherwise items (row, chunk of chunk_tiles steps) are taken in a
// grid-stride loop.
template <int F, class Src, bool BALANCED>
__global__ __launch_bounds__(kBlock) void scan_kernel(ScanCommon a, Src src) {
  const int lane = lane_id();
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x / kWave);
  // the scores of a segment collect in this wave's LDS slice and leave in 1 KiB bursts
  constexpr int kMaxSteps = max_steps<F>();
  __shared__ __align__(16) float sbuf[kBlock / kWave][kMaxSteps * kTileTokens];
  float* sb = sbuf[threadIdx.x / kWave];
  if (a.zero) {
    const int64_t per = (a.zero_words + nwaves - 1) / nwaves;
    const int64_t z1 = min(a.zero_words, (wave + 1) * per);
    for (int64_t i = wave * per + lane; i < z1; i += kWave) a.zero[i] = 0u;
  }

  if constexpr (BALANCED) {
    // total scored steps; wave 0 reports bad row metadata
    uint64_t total = 0;
    for (int r0 = 0; r0 < a.rows; r0 += kWave) {
      const int r = r0 + lane;
      const uint32_t n = r < a.rows ? (uint32_t)row_steps(a, src, r, wave == 0) : 0u;
      total += (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_sum(n), kWave - 1);
    }
    const uint64_t beg = total * (uint64_t)wave / (uint64_t)nwaves;
    const uint64_t end = total * (uint64_t)(wave + 1) / (uint64_t)nwaves;
    uint64_t acc = 0;  // steps of the rows before the current one
    for (int r0 = 0; r0 < a.rows && acc < end; r0 += kWave) {
      const int r = r0 + lane;
      const uint32_t n = r < a.rows ? (uint32_t)row_steps(a, src, r, false) : 0u;
      const int m = min(kWave, a.rows - r0);
      for (int j = 0; j < m && acc < end; ++j) {
        const uint64_t nj = (uint32_t)__builtin_amdgcn_readlane((int)n, j);
        const uint64_t lo = max(acc, beg), hi = min(acc + nj, end);
        for (uint64_t s = lo; s < hi; s += kMaxSteps)
          scan_segment<F>(a, src, r0 + j, (int64_t)(s - acc), (int)min((uint64_t)kMaxSteps, hi - s), sb);
        acc += nj;
      }
    }
    if (!a.skip_tail) {
      constexpr int64_t kFill = 4096;
      const int64_t pieces = (a.ld + kFill - 1) / kFill;
      for (int64_t it = wave; it < pieces * a.rows; it += nwaves) {
        const int r = (int)(it % a.rows);
        const int64_t f0 = (it / a.rows) * kFill;
        const int64_t from = row_steps(a, src, r, false) * kTileTokens;
        fill_neg_inf(a.logits + (int64_t)r * a.ld, max(f0, from), min(f0 + kFill, a.ld));
      }
    }
  } else {
    const int64_t chunk = (int64_t)a.chunk_tiles * kTileTokens;
    for (int64_t item = wave; item < a.n_items; item += nwaves) {
      const int r = (int)(item % a.rows);
      const int64_t c0 = (item / a.rows) * chunk;
      if (c0 >= a.ld) continue;
      const int64_t c1 = min(c0 + chunk, a.ld);
      const int64_t n = row_steps(a, src, r, c0 == 0);
      const int64_t s0 = c0 / kTileTokens;
      const int64_t s1 = min(s0 + a.chunk_tiles, n);
      if (s1 > s0) scan_segment<F>(a, src, r, s0, (int)(s1 - s0), sb);
      if (!a.skip_tail) fill_neg_inf(a.logits + (int64_t)r * a.ld, max(c0, s1 * kTileTokens), c1);
    }
  }
}

// ------------------------------------------------------------------ launcher

// Launch shape: the grid holds exactly the workgroups that are resident at once (from
// the occupancy of each kernel instance), so no workgroup starts late and becomes a
// tail.
template <int F, class Src, bool BALANCED>
static int resident_blocks_per_cu() {
  static std::once_flag once;
  static int n = 1;
  std::call_once(once, [] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, (const void*)scan_kernel<F, Src, BALANCED>, kBlock, 0) ==
            hipSuccess &&
        b > 0)
      n = b;
  });
  return n;
}

template <int F, class Src, bool BALANCED>
static hipError_t run_sched(const ScoreCall& c, const Src& src, hipStream_t stream) {
  const int cus = device_cu_count();
  const int64_t waves_total = (int64_t)cus * resident_blocks_per_cu<F, Src, BALANCED>() * (kBlock / kWave);
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
  int64_t blocks = waves_total / (kBlock / kWave);
  if (!BALANCED) {
    const int64_t need = (a.n_items + (kBlock / kWave) - 1) / (kBlock / kWave);
    if (blocks > need) blocks = need;
  }
  hipLaunchKernelGGL((scan_kernel<F, Src, BALANCED>), dim3((unsigned)blocks), dim3(kBlock), 0, stream, a, src);
  return hipGetLastError();
}

template <int F, class Src>
static hipError_t run(const ScoreCall& c, const Src& src, hipStream_t stream) {
  if (c.rows <= kBalancedMaxRows) return run_sched<F, Src, true>(c, src, stream);
  return run_sched<F, Src, false>(c, src, stream);
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
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ per-device state

__device__ unsigned g_device_errors;

static std::mutex g_mu;
static unsigned* g_err_ptr[64];
static int g_cus[64];

unsigned* device_error_word() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
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
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cus[dev] = n;
  }
  return g_cus[dev];
}

}  // namespace dsaidx
