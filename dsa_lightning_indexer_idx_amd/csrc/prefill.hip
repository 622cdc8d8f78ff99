// Prefill chunk scores: Eq. (1) of the DeepSeek-V3.2 architecture section for many
// query rows that share one key array (a prefill chunk against its context, causal
// mask carried by row_ke).
//
// Unlike the decode scan, rows here read the same keys, so keys are staged once per
// workgroup and reused by every query of the workgroup:
//   * a workgroup owns kQB consecutive queries (two per wave) and walks the union of
//     their key ranges in 64-key tiles; query blocks run longest range first;
//   * each tile (8 KiB of fp8 keys + 256 B of scales) is loaded by all 256 threads with
//     full-line 16-byte loads and stored to LDS with the 16-byte chunks of every key
//     rotated by XOR with (key % 8), so the MFMA-layout reads that follow (16 keys of
//     one 16-byte chunk column per instruction) hit distinct banks;
//   * the next tile's global loads are in flight while the current tile computes;
//   * per query and tile: 16 MFMAs (4 head tiles x 4 key tiles, K = 128 in one
//     instruction), ReLU and head weights in registers, three lane swaps for the head
//     sum, the key's fp8 scale, one 256-byte store;
//   * tiles past a query's range are masked; a query block stops at its longest
//     range, so tiles above the causal diagonal of the whole block are never loaded.
#include "device.h"
#include "launch.h"

#include <mutex>

namespace dsaidx {

constexpr int kQB = 8;               // queries per workgroup
constexpr int kPThreads = 256;       // 4 waves, 2 queries each
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
};

// LDS byte offset of 16-byte chunk c (0..7) of key t (0..63) in a tile.
__device__ __forceinline__ int tile_off(int t, int c) { return t * kDim + ((c ^ (t & 7)) << 4); }

__global__ __launch_bounds__(kPThreads, 2) void prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[2][kTileBytes];
  __shared__ float tscale[2][kTileTokens];
  __shared__ int64_t s_lo, s_hi;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int g = lane >> 4, c16 = lane & 15;
  const int nblocks = (a.rows + kQB - 1) / kQB;
  const int qb = nblocks - 1 - (int)blockIdx.x;  // longest ranges first (causal chunks)
  const int q0 = qb * kQB;

  // key range of each of this wave's two queries, and of the whole block
  int64_t qs[2], qe[2];
  bool qv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = q0 + 2 * wave + u;
    qv[u] = r < a.rows;
    int64_t s = 0, e = 0;
    if (qv[u]) {
      const int64_t s0 = a.ks[r], e0 = a.ke[r];
      s = min(max(s0, (int64_t)0), a.n_keys);
      e = min(max(e0, s), a.n_keys);
      e = min(e, s + a.ld);
      if (lane == 0 && (s != s0 || e != e0)) flag_error(a.err, kErrRange);
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
  __syncthreads();
  const int64_t lo = s_lo, hi = s_hi;
  const int ntiles = hi > lo ? (int)((hi - lo + kTileTokens - 1) / kTileTokens) : 0;

  // query operands and head weights of the two queries
  v8i qa[2][4];
  float wr[2][4][4];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = qv[u] ? q0 + 2 * wave + u : 0;
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

  // cooperative tile load: thread t moves chunks t and t + 256 (key = chunk / 8)
  const int64_t last_key = a.n_keys - 1;
  auto fetch = [&](int t, v4i& x0, v4i& x1, float& sc) {
    const int64_t base = lo + (int64_t)t * kTileTokens;
    const int64_t k0 = min(base + (tid >> 3), last_key);
    const int64_t k1 = min(base + 32 + (tid >> 3), last_key);
    x0 = *(const v4i*)(a.k + k0 * kDim + ((tid & 7) << 4));
    x1 = *(const v4i*)(a.k + k1 * kDim + ((tid & 7) << 4));
    sc = tid < kTileTokens ? a.k_scale[min(base + tid, last_key)] : 0.f;
  };
  auto stash = [&](int slot, const v4i& x0, const v4i& x1, float sc) {
    *(v4i*)(&tile[slot][tile_off(tid >> 3, tid & 7)]) = x0;
    *(v4i*)(&tile[slot][tile_off(32 + (tid >> 3), tid & 7)]) = x1;
    if (tid < kTileTokens) tscale[slot][tid] = sc;
  };

  v4i x0, x1;
  float xs = 0.f;
  if (ntiles > 0) {
    fetch(0, x0, x1, xs);
    stash(0, x0, x1, xs);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int slot = t & 1;
    if (t + 1 < ntiles) fetch(t + 1, x0, x1, xs);
    // B operands of the four 16-key tiles: key 16j + c16, chunks 2g and 2g + 1
    v8i kb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = 16 * j + c16;
      const v4i y0 = *(const v4i*)(&tile[slot][tile_off(key, 2 * g)]);
      const v4i y1 = *(const v4i*)(&tile[slot][tile_off(key, 2 * g + 1)]);
      kb[j] = v8i{y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
    }
    const float sc = tscale[slot][lane];
    const int64_t key = lo + (int64_t)t * kTileTokens + lane;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (!qv[u]) continue;
      if (lo + (int64_t)t * kTileTokens >= qe[u] || lo + (int64_t)(t + 1) * kTileTokens <= qs[u]) continue;
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = 0.f;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const v4f s = mfma_fp8_fp8(qa[u][h], kb[j], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int i = 0; i < 4; ++i) p[j] = fmaf(wr[u][h][i], relu(s[i]), p[j]);
        }
      }
      const float v = sum_lane_groups(p[0], p[1], p[2], p[3]) * sc;
      const int r = q0 + 2 * wave + u;
      if (key >= qs[u] && key < qe[u]) a.logits[(int64_t)r * a.ld + (key - qs[u])] = v;
    }
    // slot ^ 1 was last read in iteration t - 1, before the barrier that ended it
    if (t + 1 < ntiles) stash(slot ^ 1, x0, x1, xs);
    __syncthreads();
  }

  // columns past each query's length
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (!qv[u]) continue;
    const int r = q0 + 2 * wave + u;
    float* out = a.logits + (int64_t)r * a.ld;
    for (int64_t c = (qe[u] - qs[u]) + lane; c < a.ld; c += kWave) out[c] = -__builtin_inff();
  }
}

bool prefill_applies(const ScoreCall& c) {
  return c.source == SRC_DENSE && c.fmt == FMT_FP8 && c.rows >= kPrefillMinRows;
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
  const int nblocks = (c.rows + kQB - 1) / kQB;
  hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)nblocks), dim3(kPThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsaidx
