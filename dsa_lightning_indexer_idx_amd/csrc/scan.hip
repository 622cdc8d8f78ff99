// Streaming key-cache scan: Eq. (1) of the DeepSeek-V3.2 architecture section for
// rows that each read their own keys (decode rows, paged decode, candidate blocks).
//
// Work split: an item is (row, chunk of positions); waves take items in a
// grid-stride loop. A wave scores 64 positions per step:
//   * each lane loads the 32 K-elements of block (lane / 16) for the token at
//     column lane % 16 of each of the four 16-token tiles (coalesced 16-byte loads;
//     the four lane groups together read each 128-byte fp8 key row once),
//   * 16 MFMAs (4 head tiles x 4 token tiles) give S[head, token] = q_head . k,
//   * each lane applies ReLU and its 16 head weights in registers, three lane
//     swaps finish the 64-head sum, and lane l holds the score of position l,
//   * the fp8 per-token scale multiplies after the head sum (scales are >= 0, so
//     ReLU(scale * x) = scale * ReLU(x)); MXFP4 group scales enter the MFMA itself,
//   * one 256-byte store per step writes 64 scores (-inf where the position is
//     not scored).
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
  int chunk_tiles;
  int64_t n_items;
  unsigned* err;
};

// ------------------------------------------------------------------ key sources

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
  __device__ bool key(const Row& R, int64_t pos, int64_t& kidx, unsigned*) const {
    bool v = pos < R.len;
    kidx = R.base + (v ? pos : R.len - 1);
    return v;
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
  __device__ bool key(const Row& R, int64_t pos, int64_t& kidx, unsigned* err) const {
    bool v = pos < R.len;
    int64_t p = v ? pos : R.len - 1;
    int64_t pg = R.bt_row[p / page];
    if (pg < 0 || pg >= n_pages) {
      if (v) flag_error(err, kErrPage);
      pg = min(max(pg, (int64_t)0), n_pages - 1);
    }
    kidx = pg * page + p % page;
    return v;
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
  __device__ bool key(const Row& R, int64_t pos, int64_t& kidx, unsigned* err) const {
    bool in = pos < R.ncols;
    int64_t cb = in ? (int64_t)R.cand_row[pos / block] : 0;
    int64_t tok = cb * block + pos % block;
    bool v = in && cb >= 0 && tok < R.len;
    if (in && cb < 0) flag_error(err, kErrBlock);
    kidx = R.base + (v ? tok : 0);
    return v;
  }
};

// ------------------------------------------------------------------ per-format operands

template <int F>
struct QOps;
template <int F>
struct KOps;

// fp8 q against fp8 keys: head tile h, lane l -> q[16h + l%16][32g .. 32g+31] (the
// keys use the same K order, so the pairing is right whatever the hardware order).
template <>
struct QOps<FMT_FP8> {
  v8i a[4];
  __device__ void load(const uint8_t* q, int r, int lane) {
    const int g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const v4i* p = (const v4i*)(q + ((int64_t)r * kHeads + 16 * h + c) * kDim + 32 * g);
      v4i lo = p[0], hi = p[1];
      a[h] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
};
// fp8 q against MXFP4 keys. Here the K order matters: the fp4 operand of lane
// group g holds elements 32g .. 32g+31 (one UE8M0 group) while the 8-bit operand of
// lane group g holds K = 16g .. 16g+15 in its low 16 bytes and K = 64+16g .. 64+16g+15
// in its high 16 bytes (measured on gfx950 with one-hot inputs). So q dims are
// loaded in that order.
template <>
struct QOps<FMT_MXFP4> {
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

// bf16 q: head tile h, K-step s, lane l -> q[16h + l%16][32g + 8s .. +7].
template <>
struct QOps<FMT_BF16> {
  v8bf a[4][4];
  __device__ void load(const uint8_t* q, int r, int lane) {
    const int g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const v8bf* p = (const v8bf*)(q + (((int64_t)r * kHeads + 16 * h + c) * kDim + 32 * g) * 2);
#pragma unroll
      for (int s = 0; s < 4; ++s) a[h][s] = p[s];
    }
  }
};

template <>
struct KOps<FMT_FP8> {
  v8i b;
  __device__ void load(const uint8_t* k, const void*, int64_t kidx, int g) {
    const v4i* p = (const v4i*)(k + kidx * kDim + 32 * g);
    v4i lo = p[0], hi = p[1];
    b = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  __device__ v4f mma(const QOps<FMT_FP8>& qo, int h) const {
    return mfma_fp8_fp8(qo.a[h], b, v4f{0.f, 0.f, 0.f, 0.f});
  }
};

template <>
struct KOps<FMT_MXFP4> {
  v4i b;
  int sc;
  __device__ void load(const uint8_t* k, const void* scale, int64_t kidx, int g) {
    b = *(const v4i*)(k + kidx * (kDim / 2) + 16 * g);
    sc = ((const uint8_t*)scale)[kidx * (kDim / 32) + g];
  }
  __device__ v4f mma(const QOps<FMT_MXFP4>& qo, int h) const {
    v8i bb = v8i{b[0], b[1], b[2], b[3], 0, 0, 0, 0};
    return mfma_fp8_fp4(qo.a[h], bb, sc, v4f{0.f, 0.f, 0.f, 0.f});
  }
};

template <>
struct KOps<FMT_BF16> {
  v8bf b[4];
  __device__ void load(const uint8_t* k, const void*, int64_t kidx, int g) {
    const v8bf* p = (const v8bf*)(k + (kidx * kDim + 32 * g) * 2);
#pragma unroll
    for (int s = 0; s < 4; ++s) b[s] = p[s];
  }
  __device__ v4f mma(const QOps<FMT_BF16>& qo, int h) const {
    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma_bf16(qo.a[h][s], b[s], acc);
    return acc;
  }
};

// ------------------------------------------------------------------ kernel

template <int F, class Src>
__global__ __launch_bounds__(256) void scan_kernel(ScanCommon a, Src src) {
  const int lane = lane_id();
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x / kWave);
  const int64_t chunk = (int64_t)a.chunk_tiles * kTileTokens;
  const float NEG_INF = -__builtin_inff();

  for (int64_t item = wave; item < a.n_items; item += nwaves) {
    const int r = (int)(item % a.rows);
    const int64_t c0 = (item / a.rows) * chunk;
    if (c0 >= a.ld) continue;
    const int64_t c1 = min(c0 + chunk, a.ld);
    float* out = a.logits + (int64_t)r * a.ld;
    const auto R = src.row(r, a.ld, a.err, c0 == 0);
    const int64_t bound = src.bound(R);
    if (c0 >= bound) {
      for (int64_t p = c0 + lane; p < c1; p += kWave) out[p] = NEG_INF;
      continue;
    }
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
    for (int64_t base = c0; base < c1; base += kTileTokens) {
      const int64_t pst = base + lane;
      if (base >= bound) {
        if (pst < c1) out[pst] = NEG_INF;
        continue;
      }
      KOps<F> ko[4];
      int64_t kidx_st = 0;
      bool valid_st = false;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int64_t kidx;
        const bool v = src.key(R, base + 16 * j + c16, kidx, a.err);
        ko[j].load(a.k, a.k_scale, kidx, g);
        if (j == g) {
          kidx_st = kidx;
          valid_st = v;
        }
      }
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = 0.f;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const v4f s = ko[j].mma(qo, h);
#pragma unroll
          for (int i = 0; i < 4; ++i) p[j] = fmaf(wr[h][i], fmaxf(s[i], 0.f), p[j]);
        }
      }
      float v = sum_lane_groups(p[0], p[1], p[2], p[3]);
      if constexpr (F == FMT_FP8) v *= ((const float*)a.k_scale)[kidx_st];
      if (pst < c1) out[pst] = valid_st ? v : NEG_INF;
    }
  }
}

// ------------------------------------------------------------------ launcher

static constexpr int kBlock = 256;
static constexpr int kWavesPerCU = 16;

template <int F, class Src>
static hipError_t run(const ScoreCall& c, const Src& src, hipStream_t stream) {
  const int cus = device_cu_count();
  const int64_t waves_total = (int64_t)cus * kWavesPerCU;
  const int64_t tiles_per_row = (c.ld + kTileTokens - 1) / kTileTokens;
  const int64_t tiles = tiles_per_row * c.rows;
  int64_t ct = tiles / (2 * waves_total);
  ct = ct < 1 ? 1 : (ct > 32 ? 32 : ct);
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
  int64_t blocks = (a.n_items + (kBlock / kWave) - 1) / (kBlock / kWave);
  const int64_t max_blocks = waves_total / (kBlock / kWave);
  if (blocks > max_blocks) blocks = max_blocks;
  hipLaunchKernelGGL((scan_kernel<F, Src>), dim3((unsigned)blocks), dim3(kBlock), 0, stream, a, src);
  return hipGetLastError();
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
