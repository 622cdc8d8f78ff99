// Prefill chunk scores: Eq. (1) of the DeepSeek-V3.2 architecture section for many
// query rows that share one key array (a prefill chunk against its context, causal
// mask carried by row_ke).
//
//   * A workgroup owns kQB consecutive queries (two per wave) and walks one of kSplit
//     pieces of the union of their key ranges in 64-key tiles; query blocks run longest
//     range first. Two pieces per block let short causal blocks' workgroups backfill
//     behind long ones (every workgroup of the chunk is resident at once otherwise, so
//     the longest block alone would set the time).
//   * Tiles are staged in LDS, three slots deep, chunk-major (chunk c of key k at
//     c * 1 KiB + k * 16, so one 64-lane load of 16 bytes per lane fills a chunk of the
//     tile and the MFMA-layout reads, 16 keys of one chunk per 16 lanes, are contiguous).
//     As tile t finishes, the waves load tile t + 3 straight from memory into tile t's
//     slot (two loads per wave, no registers); it lands while tile t + 1 computes and is
//     waited for at the end of it. One barrier per tile.
//   * Because tile t + 1 is already visible while tile t computes, a wave reads the B
//     operands of the next 16 keys (crossing into tile t + 1) while the current 16
//     compute, and no LDS read waits on a barrier.
//   * The ReLU-weighted head sum uses sum_j w_j ReLU(s_j) = (L + A) / 2 with the linear
//     part L = sum_j w_j s_j = (sum_j w_j q_j) . k and A = sum_j w_j |s_j|. A costs one
//     FMA per head (|s| is a free source modifier) instead of a max and an FMA. L is one
//     more MFMA row per piece: q' = sum_j w_j q_j (fp32) is split into five fp8 pieces
//     with power-of-two weights (each piece is the fp8 rounding of the scaled residual of
//     the previous ones, so the split is exact to 2^-20 of max |q'|), and the pieces of a
//     wave's two queries fill rows 0..9 of one extra 16-row MFMA tile.
//   * Per 16 keys and wave: 9 MFMAs (2 queries x 4 head tiles + the pieces; K = 128 in
//     one instruction), 20 FMAs per query and lane; per tile three lane swaps for the
//     head sum, the keys' fp8 scales and one 256-byte store per query, issued ahead of
//     the next tile's loads (see there).
#include "device.h"
#include "launch.h"

#include <mutex>

namespace dsaidx {

#ifndef DSAIDX_PREFILL_QW
#define DSAIDX_PREFILL_QW 2
#endif
#ifndef DSAIDX_PREFILL_SPLIT
#define DSAIDX_PREFILL_SPLIT 2
#endif
#ifndef DSAIDX_PREFILL_WAVES_PER_SIMD
#define DSAIDX_PREFILL_WAVES_PER_SIMD 2
#endif
constexpr int kQW = DSAIDX_PREFILL_QW;  // queries per wave
constexpr int kPThreads = 256;          // 4 waves
constexpr int kQB = 4 * kQW;            // queries per workgroup
constexpr int kSplit = DSAIDX_PREFILL_SPLIT;  // workgroups per query block (key-range pieces)
constexpr int kSlots = 3;        // LDS tile slots
constexpr int kTileBytes = kTileTokens * kDim;
struct PrefillArgs {
  const uint8_t* q;
  const float* w;
  const uint8_t* k;
  const float* k_scale;
  int64_t n_keys;
  const int32_t* ks;
  const int32_t* ke;
  int rows;
  float* logits;
  int64_t ld;
  unsigned* err;
  int skip_tail;  // 1: columns past a query's length stay unwritten
  int32_t* lens_out;  // optional: each query's scored length
};

constexpr int kPieces = 5;  // fp8 pieces of q' per query


// fp8 e4m3fn byte of x (RNE; |x| <= 448) and its value.
__device__ __forceinline__ uint32_t to_fp8(float x) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.f, 0, false) & 0xFFu;
}
__device__ __forceinline__ float from_fp8(uint32_t b) { return __builtin_amdgcn_cvt_f32_fp8((int)b, 0); }

// LDS byte offset of 16-byte chunk c (0..7) of key k (0..63) in a tile slot.
__device__ __forceinline__ int tile_off(int k, int c) { return c * (kTileTokens * 16) + (k << 4); }

__global__ __launch_bounds__(kPThreads, DSAIDX_PREFILL_WAVES_PER_SIMD) void prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kSlots][kTileBytes];
  __shared__ float tscale[kSlots][kTileTokens];
  __shared__ __attribute__((aligned(16))) float qlin[kPThreads / kWave][2][kDim];
  __shared__ int qexp[kPThreads / kWave][2];
  static_assert(kQW == 1 || kQW == 2, "one or two queries per wave");
  __shared__ int64_t s_lo, s_hi;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int g = lane >> 4, c16 = lane & 15;
  const int nblocks = (a.rows + kQB - 1) / kQB;
  const int qb = nblocks - 1 - (int)blockIdx.x / kSplit;  // longest ranges first (causal chunks)
  const int piece = (int)blockIdx.x % kSplit;
  const int q0 = qb * kQB;

  // key range of each of this wave's two queries, and of the whole block
  int64_t qs[2], qe[2];
  bool qv[2] = {false, false};
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = q0 + kQW * wave + u;
    qv[u] = u < kQW && r < a.rows;
    int64_t s = 0, e = 0;
    if (qv[u]) {
      const int64_t s0 = a.ks[r], e0 = a.ke[r];
      s = min(max(s0, (int64_t)0), a.n_keys);
      e = min(max(e0, s), a.n_keys);
      e = min(e, s + a.ld);
      if (lane == 0 && piece == 0 && (s != s0 || e != e0)) flag_error(a.err, kErrRange);
      if (lane == 0 && piece == 0 && a.lens_out) a.lens_out[r] = (int32_t)(e - s);
    }
    qs[u] = s;
    qe[u] = e;
  }
  if (tid == 0) {
    s_lo = INT64_MAX;
    s_hi = 0;
  }
  __syncthreads();
  if (lane == 0) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (qv[u] && qe[u] > qs[u]) {
        atomicMin((unsigned long long*)&s_lo, (unsigned long long)qs[u]);
        atomicMax((unsigned long long*)&s_hi, (unsigned long long)qe[u]);
      }
  }

  // query operands and head weights of the two queries
  v8i qa[2][4];
  float wr[2][4][4];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = qv[u] ? q0 + kQW * wave + u : 0;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const v4i* p = (const v4i*)(a.q + ((int64_t)r * kHeads + 16 * h + c16) * kDim + 32 * g);
      const v4i x = p[0], y = p[1];
      qa[u][h] = v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
      const float4 wv = *(const float4*)(a.w + (int64_t)r * kHeads + 16 * h + 4 * g);
      wr[u][h][0] = wv.x;
      wr[u][h][1] = wv.y;
      wr[u][h][2] = wv.z;
      wr[u][h][3] = wv.w;
    }
  }

  // q' = sum_j w_j q_j of the two queries: lane l sums dims 4 (l % 32) .. + 3 of query
  // l / 32 over the 64 heads, in head order
  {
    const int uu = lane >> 5, d0 = 4 * (lane & 31);
    const int r = qv[uu] ? q0 + kQW * wave + uu : 0;
    const uint8_t* qrow = a.q + (int64_t)r * kHeads * kDim + d0;
    const float* wrow = a.w + (int64_t)r * kHeads;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int j = 0; j < kHeads; ++j) {
      const float wj = wrow[j];
      const int codes = *(const int*)(qrow + j * kDim);
      acc[0] = fmaf(wj, __builtin_amdgcn_cvt_f32_fp8(codes, 0), acc[0]);
      acc[1] = fmaf(wj, __builtin_amdgcn_cvt_f32_fp8(codes, 1), acc[1]);
      acc[2] = fmaf(wj, __builtin_amdgcn_cvt_f32_fp8(codes, 2), acc[2]);
      acc[3] = fmaf(wj, __builtin_amdgcn_cvt_f32_fp8(codes, 3), acc[3]);
    }
    *(float4*)(&qlin[wave][uu][d0]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    float mx = fmaxf(fmaxf(fabsf(acc[0]), fabsf(acc[1])), fmaxf(fabsf(acc[2]), fabsf(acc[3])));
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
    // scale so the largest |q'| lands in [128, 256): e0 = 8 - E for mx = m 2^E, m in [0.5, 1)
    int E = 0;
    frexpf(mx, &E);
    if ((lane & 31) == 0) qexp[wave][uu] = mx > 0.f ? 8 - E : 0;
  }
  __syncthreads();
  const int64_t lo = s_lo, hi = s_hi;
  const int ntiles_all = hi > lo ? (int)((hi - lo + kTileTokens - 1) / kTileTokens) : 0;
  // this workgroup's piece of the block's tiles: [t_begin, ntiles)
  const int t_begin = (int)((int64_t)ntiles_all * piece / kSplit);
  const int ntiles = (int)((int64_t)ntiles_all * (piece + 1) / kSplit);

  // A operand of the pieces tile: row rho = l % 16 < 10 holds piece rho % 5 of query
  // rho / 5 (dims 32g .. 32g+31, the same K order as the keys); coefficient of the
  // lane's accumulator rows 4g + i for each query
  v8i apiece = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  float coef[2][4];
  {
    const int rho = c16;
    if (rho < kQW * kPieces) {
      const int u = rho / kPieces, m = rho % kPieces;
      const int e0 = qexp[wave][u];
      uint32_t words[8];
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        uint32_t word = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          float y = ldexpf(qlin[wave][u][32 * g + 4 * wd + b], e0);
          for (int mm = 0; mm < m; ++mm) y = (y - from_fp8(to_fp8(y))) * 16.f;
          word |= to_fp8(y) << (8 * b);
        }
        words[wd] = word;
      }
      apiece = v8i{(int)words[0], (int)words[1], (int)words[2], (int)words[3],
                   (int)words[4], (int)words[5], (int)words[6], (int)words[7]};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * g + i;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bool mine = u < kQW && row < kQW * kPieces && row / kPieces == u;
        coef[u][i] = mine ? ldexpf(1.f, -(qexp[wave][u] + 4 * (row % kPieces))) : 0.f;
      }
    }
  }

  // tile loads: wave w moves chunks w and w + 4 of the tile's 64 keys (lane l: key l,
  // the chunk-major slot layout is exactly a load's lane order) and wave 0 the scales;
  // keys past the last one repeat it (their scores are never stored)
  const int64_t last_key = a.n_keys - 1;
  auto load_tile = [&](int t) {
    const int slot = t % kSlots;
    const int64_t key = min(lo + (int64_t)t * kTileTokens + lane, last_key);
    const uint8_t* src = a.k + key * kDim + (wave << 4);
    lds_load16(src, lds_addr(&tile[slot][tile_off(0, wave)]));
    lds_load16(src + 64, lds_addr(&tile[slot][tile_off(0, wave + 4)]));
    if (wave == 0) lds_load4(a.k_scale + key, lds_addr(&tscale[slot][0]));
  };
  auto wait_tiles = [] { __builtin_amdgcn_s_waitcnt(vmcnt_enc(0)); };
  // B operand of 16-key group j of tile t: key 16j + c16, chunks 2g and 2g + 1
  auto read_b = [&](int t, int j) -> v8i {
    const int slot = t % kSlots;
    const int key = 16 * j + c16;
    const v4i y0 = *(const v4i*)(&tile[slot][tile_off(key, 2 * g)]);
    const v4i y1 = *(const v4i*)(&tile[slot][tile_off(key, 2 * g + 1)]);
    return v8i{y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
  };

  if (t_begin < ntiles) load_tile(t_begin);
  if (t_begin + 1 < ntiles) load_tile(t_begin + 1);
  wait_tiles();
  __syncthreads();
  // Per tile, the four 16-key groups are software-pipelined in source order: the 9
  // MFMAs of group j are written before the FMAs of group j - 1, so the FMAs can
  // consume results that are already complete while the matrix core works.
  v4f ra[9], rb[9];
  auto mfmas = [&](v4f (&r)[9], const v8i& kb) {
    r[0] = mfma_fp8_fp8(apiece, kb, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int h = 0; h < 4; ++h) r[1 + h] = mfma_fp8_fp8(qa[0][h], kb, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int h = 0; h < 4; ++h) r[5 + h] = mfma_fp8_fp8(qa[kQW - 1][h], kb, v4f{0.f, 0.f, 0.f, 0.f});
  };
  auto epilogue = [&](const v4f (&r)[9], float& p0, float& p1) {
    p0 = 0.f;
    p1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) p0 = fmaf(coef[0][i], r[0][i], p0);
#pragma unroll
    for (int i = 0; i < 4; ++i) p1 = fmaf(coef[1][i], r[0][i], p1);
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) p0 = fmaf(wr[0][h][i], fabsf(r[1 + h][i]), p0);
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) p1 = fmaf(wr[kQW - 1][h][i], fabsf(r[5 + h][i]), p1);
  };
  v8i kb_next = read_b(t_begin, 0);
  if (t_begin + 2 < ntiles) load_tile(t_begin + 2);  // its slot is still unused
  for (int t = t_begin; t < ntiles; ++t) {
    const int64_t t0 = lo + (int64_t)t * kTileTokens;
    const bool act0 = qv[0] && t0 < qe[0] && t0 + kTileTokens > qs[0];
    const bool act1 = qv[1] && t0 < qe[1] && t0 + kTileTokens > qs[1];
    const float sc = 0.5f * tscale[t % kSlots][lane];
    float p[2][4];
    v8i kb = kb_next;
    kb_next = read_b(t, 1);
    mfmas(ra, kb);
    kb = kb_next;
    kb_next = read_b(t, 2);
    mfmas(rb, kb);
    epilogue(ra, p[0][0], p[1][0]);
    kb = kb_next;
    kb_next = read_b(t, 3);
    mfmas(ra, kb);
    epilogue(rb, p[0][1], p[1][1]);
    kb = kb_next;
    // the first 16 keys of tile t + 1 (already visible). Read unconditionally: after the
    // last tile the slot holds stale keys that are never used, and a conditional read
    // would make the compiler copy the previous operand into its registers, which
    // waits for that operand's LDS read at once.
    kb_next = read_b(t + 1, 0);
    mfmas(rb, kb);
    epilogue(ra, p[0][2], p[1][2]);
    epilogue(rb, p[0][3], p[1][3]);
    const int64_t key = t0 + lane;
    float vv[kQW];
#pragma unroll
    for (int u = 0; u < kQW; ++u) vv[u] = sum_lane_groups(p[u][0], p[u][1], p[u][2], p[u][3]) * sc;
    // Tile t + 2 (loaded since the end of iteration t - 1) is complete and visible after
    // this wait and barrier, and every wave is done with tile t. The stores go out before
    // the next tile's loads: the wait at the end of the next iteration then covers both
    // without counting the (conditional) stores. The scores are written once and not read
    // again by this kernel: non-temporal stores keep them from displacing the key tiles in
    // the cache.
    wait_tiles();
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kQW; ++u)
      if ((u == 0 ? act0 : act1) && key >= qs[u] && key < qe[u])
        __builtin_nontemporal_store(vv[u], &a.logits[(int64_t)(q0 + kQW * wave + u) * a.ld + (key - qs[u])]);
    if (t + 3 < ntiles) load_tile(t + 3);  // into tile t's slot
  }

  // columns past each query's length
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (!qv[u] || a.skip_tail || piece != 0) continue;
    float* out = a.logits + (int64_t)(q0 + kQW * wave + u) * a.ld;
    for (int64_t c = (qe[u] - qs[u]) + lane; c < a.ld; c += kWave) __builtin_nontemporal_store(-__builtin_inff(), &out[c]);
  }
}

bool prefill_applies(const ScoreCall& c) {
  return c.source == SRC_DENSE && c.shared_keys && c.fmt == FMT_FP8 && c.rows >= kPrefillMinRows;
}

hipError_t launch_prefill(const ScoreCall& c, hipStream_t stream) {
  PrefillArgs a;
  a.q = c.q;
  a.w = c.w;
  a.k = c.k;
  a.k_scale = (const float*)c.k_scale;
  a.n_keys = c.n_keys;
  a.ks = c.row_ks;
  a.ke = c.row_ke;
  a.rows = c.rows;
  a.logits = c.logits;
  a.ld = c.ld;
  a.err = c.err;
  a.skip_tail = c.skip_tail;
  a.lens_out = c.lens_out;
  const int nblocks = (c.rows + kQB - 1) / kQB;
  hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)(nblocks * kSplit)), dim3(kPThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsaidx
