// Candidate-source step of the two-level indexer: from the scores of a layer that scored
// its whole context, publish each row's candidate blocks for the consuming layers (the
// vLLM sparse_indexer page: a candidate-source layer hands candidate_topk_blocks blocks
// of candidate_block_size tokens to the layers after it; the DeepGEMM release note:
// consumers score only those blocks). The pages do not give the ranking rule; the
// reading: a block's score is the largest score of its tokens, and the n_top best
// blocks (higher score first, equal scores by lower block id) are published in
// ascending id, the order the consumers need, then -1 up to n_top.
//
// Two launches, both bound by reading the scores once:
//   piece_max_kernel   one 32-bit order key per 64-token piece: the largest key of the
//                      piece's valid tokens (0 = no token with a score). A wave reads
//                      four 256-token chunks (16 bytes per lane each), reduces each
//                      16-lane row with DPP and stores one key per row.
//   selection          block keys (the largest piece key of the block's pieces), the
//                      n_top-th largest key T, then one pass in block order that takes
//                      the keys above T and ranks those equal to T by id, writing the
//                      chosen ids at prefix-sum positions, so they come out ascending.
//                      Rows of up to 1024 blocks: one wave per row with the keys in
//                      registers (cand_select_wave_kernel); longer rows: one workgroup
//                      per row with the keys in LDS and a 4-pass 8-bit radix select
//                      (cand_select_kernel).
// Keys compare as the selection order does: order_key maps higher scores to larger
// integers and folds -0.0 onto +0.0, so equal maxima tie and go to the lower id.
#include "device.h"
#include "launch.h"

#include <algorithm>
#include <mutex>

namespace dsaidx {

constexpr int kPieceTokens = 64;
constexpr int kChunkTokens = 256;              // one wave-wide 16-byte-per-lane read
constexpr int kPieceThreads = 256;
constexpr int kChunksPerWave = 4;
constexpr int kGroupTokens = kChunkTokens * kChunksPerWave * (kPieceThreads / kWave);  // 4096
constexpr int kSelectThreads = 256;
static_assert(kSelectThreads == 256, "one radix bin per thread");

struct CandArgs {
  const float* logits;
  int64_t ld;
  const int32_t* lens;
  int64_t n_cols;
  int rows;
  int block;           // tokens per block, a multiple of 64
  int n_top;
  int32_t* cand;
  int64_t cand_ld;
  int32_t* n_cand;
  uint32_t* pieces;    // [rows, pieces_ld]
  int64_t pieces_ld;
};

__device__ __forceinline__ int64_t cand_row_len(const CandArgs& a, int r) {
  return a.lens ? min(a.n_cols, (int64_t)max(a.lens[r], 0)) : a.n_cols;
}

// Largest value of each 16-lane row, in the row's last lane: a max-scan with DPP row
// shifts (lanes without a source take 0, the smallest key).
__device__ __forceinline__ uint32_t row_max_to_last(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));  // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));  // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));  // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));  // row_shr:8
  return v;
}

template <bool V4>
__global__ __launch_bounds__(kPieceThreads) void piece_max_kernel(CandArgs a, int64_t groups) {
  const int r = (int)(blockIdx.x / groups);
  const int64_t g = blockIdx.x % groups;
  const int64_t len = cand_row_len(a, r);
  if (g * kGroupTokens >= len) return;
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const float* row = a.logits + (int64_t)r * a.ld;
  const int64_t chunk0 = g * (kGroupTokens / kChunkTokens) + (int64_t)w * kChunksPerWave;
  float x[kChunksPerWave][4];
#pragma unroll
  for (int u = 0; u < kChunksPerWave; ++u) {
    const int64_t col = (chunk0 + u) * kChunkTokens + 4 * lane;
    if (V4) {
      // rows start on 16-byte boundaries and ld % 4 == 0: col < len <= ld keeps the
      // whole group of four inside the row
      v4f v = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (col < len) v = *(const v4f*)(row + col);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[u][i] = v[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[u][i] = col + i < len ? row[col + i] : -INFINITY;
    }
  }
#pragma unroll
  for (int u = 0; u < kChunksPerWave; ++u) {
    const int64_t col = (chunk0 + u) * kChunkTokens + 4 * lane;
    uint32_t k = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) k = max(k, col + i < len ? order_key(x[u][i]) : 0u);
    k = row_max_to_last(k);
    const int64_t piece = (chunk0 + u) * (kChunkTokens / kPieceTokens) + lane / 16;
    if ((lane & 15) == 15 && piece * kPieceTokens < len) a.pieces[(int64_t)r * a.pieces_ld + piece] = k;
  }
}

// Exclusive prefix sum over the workgroup in thread order; ``total`` gets the sum.
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const uint32_t incl = wave_inclusive_sum(v);
  const int w = threadIdx.x / kWave;
  if (lane_id() == kWave - 1) wsum[w] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kSelectThreads / kWave; ++i) {
    const uint32_t s = wsum[i];
    base += i < w ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return base + incl - v;
}

__global__ __launch_bounds__(kSelectThreads) void cand_select_kernel(CandArgs a) {
  extern __shared__ uint32_t keys[];  // [n_blocks] block keys
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wsum[kSelectThreads / kWave];
  __shared__ uint32_t s_digit, s_rem, s_n;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t len = cand_row_len(a, r);
  const int64_t n_pieces = (len + kPieceTokens - 1) / kPieceTokens;
  const int per = a.block / kPieceTokens;
  const int nblk = (int)((len + a.block - 1) / a.block);
  const uint32_t* pc = a.pieces + (int64_t)r * a.pieces_ld;
  for (int b = tid; b < nblk; b += kSelectThreads) {
    uint32_t k = 0;
    const int64_t p0 = (int64_t)b * per;
    for (int i = 0; i < per; ++i)
      if (p0 + i < n_pieces) k = max(k, pc[p0 + i]);
    keys[b] = k;
  }
  __syncthreads();

  // radix select: the rem-th largest key among those that match the digits found so
  // far; absent blocks (key 0) are never counted
  uint32_t prefix = 0, rem = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int sh = 24 - 8 * pass;
    hist[tid] = 0;  // kSelectThreads == 256 bins
    __syncthreads();
    for (int b = tid; b < nblk; b += kSelectThreads) {
      const uint32_t k = keys[b];
      if (k != 0 && ((uint64_t)k >> (sh + 8)) == ((uint64_t)prefix >> (sh + 8))) atomicAdd(&hist[(k >> sh) & 0xFFu], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      // lane l takes bins 255 - 4l .. 252 - 4l: counts from the top down
      uint32_t c[4], s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hist[255 - 4 * tid - j];
        s += c[j];
      }
      const uint32_t incl = wave_inclusive_sum(s);
      uint32_t want = rem;
      if (pass == 0) {
        const uint32_t present = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
        want = min((uint32_t)a.n_top, present);
        if (tid == 0) s_n = want;
      }
      const uint32_t excl = incl - s;
      if (want > 0 && excl < want && incl >= want) {
        uint32_t cum = excl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (cum < want && cum + c[j] >= want) {
            s_digit = 255u - 4u * tid - j;
            s_rem = want - cum;
          }
          cum += c[j];
        }
      }
      if (want == 0 && tid == 0) {
        s_digit = 0;
        s_rem = 0;
      }
    }
    __syncthreads();
    prefix |= s_digit << sh;
    rem = s_rem;
    if (s_n == 0) break;
  }
  const uint32_t n = s_n;
  int32_t* out = a.cand + (int64_t)r * a.cand_ld;
  if (n > 0) {
    // every key above the threshold, and the first ``rem`` (by id) equal to it
    const uint32_t thr = prefix;
    uint32_t eq_seen = 0, written = 0;
    for (int b0 = 0; b0 < nblk && written < n; b0 += kSelectThreads) {
      const int b = b0 + tid;
      const uint32_t k = b < nblk ? keys[b] : 0u;
      const uint32_t eq = k == thr ? 1u : 0u;  // thr > 0, so no absent block
      uint32_t eq_tot;
      const uint32_t eq_rank = eq_seen + block_exclusive_sum(eq, wsum, eq_tot);
      const uint32_t sel = (k > thr || (eq && eq_rank < rem)) ? 1u : 0u;
      uint32_t sel_tot;
      const uint32_t pos = written + block_exclusive_sum(sel, wsum, sel_tot);
      if (sel) out[pos] = b;
      eq_seen += eq_tot;
      written += sel_tot;
    }
  }
  for (int i = (int)n + tid; i < a.n_top; i += kSelectThreads) out[i] = -1;
  if (tid == 0) a.n_cand[r] = (int32_t)n;
}

// Rows of at most kWaveBlocks blocks: one wave per row, kKeysPerLane block keys per lane
// in registers (lane l holds blocks kKeysPerLane * l + j, so lane order is block order),
// no barriers. The threshold T, the n-th largest key, is found by bisection over its
// 32 bits: T is the largest value with at least n keys >= T, each count a sum of
// ballots. Then the keys above T and the first (by id) of those equal to it are
// written at positions given by wave prefix sums. PER > 0 fixes the pieces per block.
constexpr int kKeysPerLane = 16;
constexpr int kWaveBlocks = kKeysPerLane * kWave;  // 1024
constexpr int kWaveSelectThreads = 256;            // four rows per workgroup

// Keys >= t over the wave. The 16 compares are scheduled as one group ahead of the
// scalar popcounts: a popcount waits for the vector compare that wrote its mask, and
// interleaved pairs would pay that wait 16 times in a row.
__device__ __forceinline__ uint32_t count_at_least(const uint32_t (&key)[kKeysPerLane], uint32_t t) {
  uint64_t m[kKeysPerLane];
#pragma unroll
  for (int j = 0; j < kKeysPerLane; ++j) m[j] = __ballot(key[j] >= t);
  __builtin_amdgcn_sched_group_barrier(0x2, kKeysPerLane, 0);      // VALU: the compares
  __builtin_amdgcn_sched_group_barrier(0x4, 2 * kKeysPerLane, 0);  // SALU: popcounts, adds
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < kKeysPerLane; ++j) c += (uint32_t)__popcll(m[j]);
  return c;
}

template <int PER>
__global__ __launch_bounds__(kWaveSelectThreads) void cand_select_wave_kernel(CandArgs a) {
  const int r = blockIdx.x * (kWaveSelectThreads / kWave) + threadIdx.x / kWave;
  if (r >= a.rows) return;
  const int lane = lane_id();
  const int per = PER > 0 ? PER : a.block / kPieceTokens;
  const uint32_t* pc = a.pieces + (int64_t)r * a.pieces_ld;
  uint32_t key[kKeysPerLane];
  if constexpr (PER > 0) {
    // the lane's PER * 16 pieces are contiguous: 16-byte loads from addresses clamped
    // into the row (pieces_ld is a multiple of 4), all issued before the first use and
    // before the row length; pieces at or past n_pieces are masked after the load
    constexpr int kLoads = kKeysPerLane * PER / 4;
    const int64_t p0 = (int64_t)kKeysPerLane * PER * lane;
    v4i v[kLoads];
    // pieces_ld == 0 (no columns, no workspace): nothing to read
#pragma unroll
    for (int q = 0; q < kLoads; ++q)
      v[q] = a.pieces_ld > 0 ? *(const v4i*)(pc + min(p0 + 4 * q, a.pieces_ld - 4)) : v4i{0, 0, 0, 0};
    const int64_t n_pieces = (cand_row_len(a, r) + kPieceTokens - 1) / kPieceTokens;
#pragma unroll
    for (int j = 0; j < kKeysPerLane; ++j) {
      uint32_t k = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = j * PER + i;
        k = max(k, p0 + e < n_pieces ? (uint32_t)v[e / 4][e % 4] : 0u);
      }
      key[j] = k;
    }
  } else {
    const int64_t n_pieces = (cand_row_len(a, r) + kPieceTokens - 1) / kPieceTokens;
#pragma unroll
    for (int j = 0; j < kKeysPerLane; ++j) {
      const int64_t b0 = (int64_t)(kKeysPerLane * lane + j) * per;
      uint32_t k = 0;
      for (int i = 0; i < per && a.pieces_ld > 0; ++i) {
        const int64_t p = b0 + i;
        const uint32_t x = pc[min(p, a.pieces_ld - 1)];
        k = max(k, p < n_pieces ? x : 0u);
      }
      key[j] = k;
    }
  }
  const uint32_t n = min((uint32_t)a.n_top, count_at_least(key, 1u));
  int32_t* out = a.cand + (int64_t)r * a.cand_ld;
  if (n > 0) {
    uint32_t t = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = t | (1u << bit);
      if (count_at_least(key, c) >= n) t = c;
    }
    // keys above t; t + 1 cannot wrap: no key exceeds that of +inf, 0xFF800000
    const uint32_t need_eq = n - count_at_least(key, t + 1u);
    uint32_t n_eq = 0;
#pragma unroll
    for (int j = 0; j < kKeysPerLane; ++j) n_eq += key[j] == t ? 1u : 0u;
    uint32_t eq_rank = wave_inclusive_sum(n_eq) - n_eq;
    uint32_t sel = 0, cnt = 0;
#pragma unroll
    for (int j = 0; j < kKeysPerLane; ++j) {
      const bool eq = key[j] == t;
      const bool take = key[j] > t || (eq && eq_rank < need_eq);
      eq_rank += eq ? 1u : 0u;
      sel |= take ? 1u << j : 0u;
      cnt += take ? 1u : 0u;
    }
    uint32_t pos = wave_inclusive_sum(cnt) - cnt;
    for (; sel != 0; sel &= sel - 1) out[pos++] = kKeysPerLane * lane + __builtin_ctz(sel);
  }
  for (int i = (int)n + lane; i < a.n_top; i += kWave) out[i] = -1;
  if (lane == 0) a.n_cand[r] = (int32_t)n;
}

// Pieces per workspace row: a multiple of 4, so every row starts on 16 bytes.
static int64_t pieces_ld(int64_t n_cols) { return ((n_cols + kPieceTokens - 1) / kPieceTokens + 3) / 4 * 4; }

size_t cand_workspace_bytes(int rows, int64_t n_cols) {
  if (rows <= 0 || n_cols <= 0) return 0;
  const int64_t bytes = (int64_t)rows * pieces_ld(n_cols) * 4;
  return (size_t)((bytes + 255) / 256 * 256);
}

hipError_t launch_candidate_blocks(const CandCall& c, void* workspace, hipStream_t stream) {
  if (c.rows <= 0) return hipSuccess;
  CandArgs a{c.logits, c.ld, c.lens, c.n_cols, c.rows, c.block, c.n_top, c.cand, c.cand_ld, c.n_cand,
             (uint32_t*)workspace, pieces_ld(c.n_cols)};
  if (c.n_cols > 0) {
    const int64_t groups = (c.n_cols + kGroupTokens - 1) / kGroupTokens;
    const dim3 grid((unsigned)(groups * c.rows));
    const bool v4 = ((uintptr_t)c.logits % 16 == 0) && (c.ld % 4 == 0);
    if (v4)
      hipLaunchKernelGGL(piece_max_kernel<true>, grid, dim3(kPieceThreads), 0, stream, a, groups);
    else
      hipLaunchKernelGGL(piece_max_kernel<false>, grid, dim3(kPieceThreads), 0, stream, a, groups);
  }
  const int64_t nblk = (c.n_cols + c.block - 1) / c.block;
  if (nblk <= kWaveBlocks) {
    const dim3 grid((unsigned)((c.rows + kWaveSelectThreads / kWave - 1) / (kWaveSelectThreads / kWave)));
    if (c.block == 2 * kPieceTokens)
      hipLaunchKernelGGL(cand_select_wave_kernel<2>, grid, dim3(kWaveSelectThreads), 0, stream, a);
    else if (c.block == kPieceTokens)
      hipLaunchKernelGGL(cand_select_wave_kernel<1>, grid, dim3(kWaveSelectThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(cand_select_wave_kernel<0>, grid, dim3(kWaveSelectThreads), 0, stream, a);
    return hipGetLastError();
  }
  static PerDeviceOnce once;
  const hipError_t attr = once.run([] {
    return hipFuncSetAttribute((const void*)cand_select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                               kCandMaxBlocks * (int)sizeof(uint32_t));
  });
  if (attr != hipSuccess) return attr;
  const size_t lds = (size_t)std::max<int64_t>(nblk, 1) * sizeof(uint32_t);
  hipLaunchKernelGGL(cand_select_kernel, dim3((unsigned)c.rows), dim3(kSelectThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace dsaidx
