// Sparse attention over the selected entries, the step the indexer feeds (Eq. (2) of the
// DeepSeek-V3.2 architecture section: the output attends only the key-value entries
// whose index scores are in the row's top-k). MLA keeps one 576-element entry per token,
// shared by every head (the 512- and 576-element vectors of the llama.cpp thread); head
// h scores entry c as scale * (q_h . c) and reads its first 512 elements as the value.
//
// attn_partial_kernel: one workgroup per (row, group of up to 64 heads, split of the
// row's selected positions), one wave per 16 heads, one wave per SIMD: the wave holds Q
// (72 VGPRs), O (128), the next tile's gather and a batch of operand reads, more than
// two waves per SIMD could (which would serialise every MFMA on its LDS read). The
// head groups of one (row, split) go to the same XCD (workgroup ids 8 apart), so the
// second gather of a tile mostly hits that XCD's L2. Per 32-position tile:
//   * gather: the 32 entries (paged, through the block table) land in LDS token-major.
//     The scores read B operands (8 consecutive dims of one token) with 16-byte loads;
//     the value product needs 8 consecutive tokens of one dim, which gfx950's
//     transposing LDS read delivers from the same layout (in each 16-lane group, lane j
//     reads 4 dims of token j / 4 and lane i receives 4 tokens of dim i). The loads of
//     tile t + 1 are issued into registers before tile t computes; the split's entry
//     addresses are resolved once, up front.
//   * scores S[16 heads x 32 tokens] = Q K^T: v_mfma_f32_16x16x32_bf16 over the 576 dims
//     (18 K-steps, two 16-token columns), Q held in registers as A operands.
//   * online softmax in the base-2 domain (scale folded with log2 e): per head the tile
//     maximum and sum across the 16 lanes of a row by DPP, rescaling of the running sum
//     and of the output.
//   * O[16 heads x 512] += P V: P (bf16) goes through a small per-wave LDS buffer into
//     the A-operand layout; 32 MFMAs, one per 16 value dims.
// The split's (O, m, l) go to the workspace; attn_combine_kernel merges the splits into
// the output and the log-sum-exp. With one split the partial kernel writes both itself.
#include "device.h"
#include "launch.h"

#include <algorithm>
#include <mutex>

namespace dsaidx {

constexpr int kAttnD = 576;          // entry / query length
constexpr int kAttnDV = 512;         // value length (the entry's first 512 elements)
constexpr int kAttnT = 32;           // positions per tile
constexpr int kKPitch = kAttnD + 48;  // token-major tile row (bf16): 1248 B (fewest bank conflicts of the pads tried)
constexpr int kPPitch = kAttnT + 8;  // per-wave P rows (bf16)
constexpr int kTail = kAttnD - kAttnDV;  // dims 512..575 of a token: 128 B, 8 chunks of 16 B
constexpr int kChunks = kAttnT * kAttnD / 8;  // 16-byte pieces of a tile (2304)
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
  const uint16_t* q;       // [rows, heads, 576] bf16
  const uint16_t* kv;      // [n_pages, page_size, 576] bf16
  int64_t n_pages;
  int page_size;
  const int32_t* bt;
  int64_t bt_rows;
  int64_t bt_ld;
  const int32_t* seq_lens;
  const int32_t* row_req;
  const int32_t* idx;      // [rows, idx_ld]
  int64_t idx_ld;
  int k;
  int rows;
  int heads;
  float scale2;            // scale * log2(e)
  int nsplit;
  int split_len;           // selected positions per split (a multiple of kAttnT)
  int hgroups;             // head groups (workgroups) per (row, split)
  float* out;              // [rows, heads, 512]
  float* lse;              // [rows, heads] or null
  float* part_o;           // [rows, nsplit, heads, 512]
  float* part_ml;          // [rows, nsplit, heads, 2]
  unsigned* err;
};

// The entry a position without a valid cache entry reads: zeros, so that its zero
// softmax weight times its values is 0 (a cache slot could hold Inf or NaN).
__device__ const uint16_t g_attn_zero_entry[kAttnD] = {};

__device__ __forceinline__ const uint16_t* entry_or_zero(const uint16_t* kv, int64_t e) {
  return e >= 0 ? kv + e * kAttnD : g_attn_zero_entry;
}

__device__ __forceinline__ float dpp_row_max(float v) {
  // butterfly over the 16 lanes of a row: quad xor 1, xor 2, half-row mirror, row mirror
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true)));
  return v;
}

__device__ __forceinline__ float dpp_row_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));
  return v;
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  // round to nearest even (scores and weights are finite here)
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <int NW>
__global__ __launch_bounds__(NW * kWave, 1) void attn_partial_kernel(AttnArgs a) {
  constexpr int NT = NW * kWave;
  constexpr int kPer = (kChunks + NT - 1) / NT;  // 16-byte pieces each thread gathers per tile
  __shared__ __align__(16) uint16_t kt[kAttnT * kKPitch];
  __shared__ __align__(16) uint16_t pb[NW][16 * kPPitch];
  extern __shared__ int64_t ent[];  // the split's entry rows (-1: not a valid entry)

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int g = lane >> 4, c16 = lane & 15;
  // (row, split) unit p and head group hg: ids 8 apart share an XCD
  const int b = blockIdx.x;
  const int p = (b / (8 * a.hgroups)) * 8 + (b % 8);
  const int hg = (b / 8) % a.hgroups;
  if (p >= a.rows * a.nsplit) return;
  const int r = p / a.nsplit;
  const int split = p % a.nsplit;
  const int i0 = split * a.split_len;
  const int i1 = min(a.k, i0 + a.split_len);
  const int ntok = max(i1 - i0, 0);
  const int ntiles = (ntok + kAttnT - 1) / kAttnT;

  // entry rows of the split's positions
  {
    const int64_t req = a.row_req ? (int64_t)a.row_req[r] : (int64_t)r;
    const bool req_ok = req >= 0 && req < a.bt_rows;
    const int64_t len = a.seq_lens[r];
    for (int i = tid; i < ntiles * kAttnT; i += NT) {
      int64_t e = -1;
      if (i < ntok && req_ok) {
        const int64_t pos = a.idx[(int64_t)r * a.idx_ld + i0 + i];
        if (pos >= 0 && pos < len && pos / a.page_size < a.bt_ld) {
          const int64_t page = a.bt[req * a.bt_ld + pos / a.page_size];
          if (page >= 0 && page < a.n_pages)
            e = page * a.page_size + pos % a.page_size;
          else
            flag_error(a.err, kErrPage);
        }
      }
      ent[i] = e;
    }
    if (tid == 0 && !req_ok && ntok > 0) flag_error(a.err, kErrRange);
  }
  __syncthreads();

  // the wave's 16 heads: A operands of the 18 K-steps (row c16 = head, dims 32s + 8g ..)
  const int head0 = hg * 16 * NW + 16 * wave;
  const uint16_t* qrow = a.q + ((int64_t)r * a.heads + head0 + c16) * kAttnD + 8 * g;
  v8bf qa[kAttnD / 32];
#pragma unroll
  for (int s = 0; s < kAttnD / 32; ++s) qa[s] = *(const v8bf*)(qrow + 32 * s);

  // gather: piece c of the tile is 16-byte chunk c % 72 of token c / 72, so a wave's
  // load reads 1 KiB of one entry (8 cache lines) rather than 16 bytes of 32 entries
  v4i pre[kPer];
  auto fetch = [&](int t) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int c = tid + u * NT;
      if (c < kChunks) {
        const int64_t e = ent[t * kAttnT + c / (kAttnD / 8)];
        pre[u] = *(const v4i*)(entry_or_zero(a.kv, e) + 8 * (c % (kAttnD / 8)));
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int c = tid + u * NT;
      if (c < kChunks) *(v4i*)(&kt[(c / (kAttnD / 8)) * kKPitch + 8 * (c % (kAttnD / 8))]) = pre[u];
    }
  };
  // value operand of dims 16n .. 16n + 15: lane (g, c16) gets tokens 8g .. 8g + 7 of dim
  // 16n + c16, from two transposing reads (tokens 8g + c16 / 4 and 8g + 4 + c16 / 4, dims
  // 16n + 4 (c16 % 4) .. + 3)
  typedef __attribute__((address_space(3))) v4bf lds_v4bf;
  const int tr_off = (8 * g + (c16 >> 2)) * kKPitch + 4 * (c16 & 3);
  auto read_v = [&](int n) -> v8bf {
    const v4bf lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(&kt[tr_off + 16 * n]));
    const v4bf hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(&kt[tr_off + 4 * kKPitch + 16 * n]));
    return v8bf{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };

  float m[4], l[4];
  v4f o[kAttnDV / 16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -__builtin_inff();
    l[i] = 0.f;
  }
#pragma unroll
  for (int n = 0; n < kAttnDV / 16; ++n) o[n] = v4f{0.f, 0.f, 0.f, 0.f};

  if (ntiles > 0) fetch(0);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();  // every wave is done with tile t - 1
    stash();
    __syncthreads();
    if (t + 1 < ntiles) fetch(t + 1);

    // scores of the tile's two 16-token columns: all 36 operand reads are issued before
    // the MFMAs, which then wait for them in order instead of one LDS round trip each
    v4f sc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
    v8bf kb[2][kAttnD / 32];
#pragma unroll
    for (int s = 0; s < kAttnD / 32; ++s)
#pragma unroll
      for (int j = 0; j < 2; ++j) kb[j][s] = *(const v8bf*)(&kt[(16 * j + c16) * kKPitch + 32 * s + 8 * g]);
#pragma unroll
    for (int s = 0; s < kAttnD / 32; ++s)
#pragma unroll
      for (int j = 0; j < 2; ++j) sc[j] = mfma_bf16(qa[s], kb[j][s], sc[j]);
    // lane (g, c16): heads 4g + i, tokens c16 and 16 + c16 of the tile
    const bool v0 = ent[t * kAttnT + c16] >= 0, v1 = ent[t * kAttnT + 16 + c16] >= 0;
    float p[2][4], alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float s0 = v0 ? sc[0][i] * a.scale2 : -__builtin_inff();
      const float s1 = v1 ? sc[1][i] * a.scale2 : -__builtin_inff();
      const float mt = dpp_row_max(fmaxf(s0, s1));
      const float mn = fmaxf(m[i], mt);
      // all -inf so far: keep weights 0 (exp2(-inf) = 0, and no -inf - -inf)
      const float base = mn == -__builtin_inff() ? 0.f : mn;
      // v_exp_f32 directly (exp2f adds a denormal-range fix): arguments are <= 0 or
      // -inf, and a weight below 2^-126 of the row maximum may flush to 0
      alpha[i] = __builtin_amdgcn_exp2f(m[i] - base);
      p[0][i] = __builtin_amdgcn_exp2f(s0 - base);
      p[1][i] = __builtin_amdgcn_exp2f(s1 - base);
      l[i] = l[i] * alpha[i] + dpp_row_sum(p[0][i] + p[1][i]);
      m[i] = mn;
    }
#pragma unroll
    for (int n = 0; n < kAttnDV / 16; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[n][i] *= alpha[i];
    // P into the A-operand layout: row = head, 8 consecutive tokens per lane group
    uint16_t* pw = pb[wave];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) pw[(4 * g + i) * kPPitch + 16 * j + c16] = f32_to_bf16(p[j][i]);
    __builtin_amdgcn_wave_barrier();  // one wave's LDS operations complete in order
    const v8bf pa = *(const v8bf*)(&pw[c16 * kPPitch + 8 * g]);
    // value operands in two batches of 16 reads, each ahead of its MFMAs
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v8bf vb[kAttnDV / 32];
#pragma unroll
      for (int n = 0; n < kAttnDV / 32; ++n) vb[n] = read_v(16 * h + n);
#pragma unroll
      for (int n = 0; n < kAttnDV / 32; ++n) o[16 * h + n] = mfma_bf16(pa, vb[n], o[16 * h + n]);
    }
    __builtin_amdgcn_wave_barrier();  // the P reads finish before the next tile's writes
  }

  // lane (g, c16) holds O[head 4g + i][dim 16n + c16]
  if (a.nsplit == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = head0 + 4 * g + i;
      const float inv = l[i] > 0.f ? 1.f / l[i] : 0.f;
      float* orow = a.out + ((int64_t)r * a.heads + h) * kAttnDV;
#pragma unroll
      for (int n = 0; n < kAttnDV / 16; ++n) orow[16 * n + c16] = o[n][i] * inv;
      if (a.lse && c16 == 0)
        a.lse[(int64_t)r * a.heads + h] = l[i] > 0.f ? (m[i] + log2f(l[i])) * 0.69314718055994531f : -__builtin_inff();
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = head0 + 4 * g + i;
      const int64_t slot = ((int64_t)r * a.nsplit + split) * a.heads + h;
      float* orow = a.part_o + slot * kAttnDV;
#pragma unroll
      for (int n = 0; n < kAttnDV / 16; ++n) orow[16 * n + c16] = o[n][i];
      if (c16 == 0) {
        a.part_ml[2 * slot] = m[i];
        a.part_ml[2 * slot + 1] = l[i];
      }
    }
  }
}

// ---- 16 heads: one wave per (row, split), gathering with direct-to-LDS loads
//
// A single wave staging a whole tile in registers would need 144 of them; instead the
// entries go from memory straight into LDS (no registers), dims 0..511 token-major as
// above and dims 512..575 in a side array.

__global__ __launch_bounds__(kWave, 1) void attn_partial_1w_kernel(AttnArgs a) {
  constexpr int NW = 1, NT = kWave;
  __shared__ __align__(16) uint16_t kt[1][kAttnT * kKPitch];  // dims 0..511, token-major
  __shared__ __align__(16) uint16_t kl[1][kAttnT * kTail];     // dims 512..575, swizzled
  __shared__ __align__(16) uint16_t pb[NW][16 * kPPitch];
  extern __shared__ int64_t ent[];  // the split's entry rows (-1: not a valid entry)

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = lane >> 4, c16 = lane & 15;
  // (row, split) unit p and head group hg: ids 8 apart share an XCD
  const int b = blockIdx.x;
  const int p = (b / (8 * a.hgroups)) * 8 + (b % 8);
  const int hg = (b / 8) % a.hgroups;
  if (p >= a.rows * a.nsplit) return;
  const int r = p / a.nsplit;
  const int split = p % a.nsplit;
  const int i0 = split * a.split_len;
  const int i1 = min(a.k, i0 + a.split_len);
  const int ntok = max(i1 - i0, 0);
  const int ntiles = (ntok + kAttnT - 1) / kAttnT;

  // entry rows of the split's positions
  {
    const int64_t req = a.row_req ? (int64_t)a.row_req[r] : (int64_t)r;
    const bool req_ok = req >= 0 && req < a.bt_rows;
    const int64_t len = a.seq_lens[r];
    for (int i = tid; i < ntiles * kAttnT; i += NT) {
      int64_t e = -1;
      if (i < ntok && req_ok) {
        const int64_t pos = a.idx[(int64_t)r * a.idx_ld + i0 + i];
        if (pos >= 0 && pos < len && pos / a.page_size < a.bt_ld) {
          const int64_t page = a.bt[req * a.bt_ld + pos / a.page_size];
          if (page >= 0 && page < a.n_pages)
            e = page * a.page_size + pos % a.page_size;
          else
            flag_error(a.err, kErrPage);
        }
      }
      ent[i] = e;
    }
    if (tid == 0 && !req_ok && ntok > 0) flag_error(a.err, kErrRange);
  }
  __syncthreads();

  // the wave's 16 heads: A operands of the 18 K-steps (row c16 = head, dims 32s + 8g ..)
  const int head0 = hg * 16 * NW + 16 * wave;
  const uint16_t* qrow = a.q + ((int64_t)r * a.heads + head0 + c16) * kAttnD + 8 * g;
  v8bf qa[kAttnD / 32];
#pragma unroll
  for (int s = 0; s < kAttnD / 32; ++s) qa[s] = *(const v8bf*)(qrow + 32 * s);

  // gather: tile t's entries go from memory straight into tile buffer bs (16-byte loads
  // that write LDS at the wave-uniform base + 16 l for lane l). Wave w moves dims 0..511
  // of tokens w, w + NW, ... (one 1 KiB load each) and dims 512..575 of 8 tokens per load
  // (lane l: token 8q + l / 8, chunk (l % 8) ^ (token % 8), so the 16 rows a score read
  // touches spread over the banks). Positions without a valid entry read a zero entry:
  // their weights are exactly 0, and 0 times its values is 0 whatever the cache holds.
  // (the entry rows are read ahead of the loads, up to 8 tokens at a time: the loads
  // are ordered with LDS accesses, so a read between two of them costs a round trip)
  auto dma = [&](int t, int bs) {
    constexpr int kMain = kAttnT / NW, kChunk = kMain < 8 ? kMain : 8;
    const uint32_t mbase = lds_addr(kt[bs]), tbase = lds_addr(kl[bs]);
    int64_t tv[4 / NW];
#pragma unroll
    for (int v = 0; v < 4 / NW; ++v) tv[v] = ent[t * kAttnT + 8 * (wave + v * NW) + (lane >> 3)];
#pragma unroll
    for (int c = 0; c < kMain; c += kChunk) {
      int64_t ev[kChunk];
#pragma unroll
      for (int u = 0; u < kChunk; ++u) ev[u] = ent[t * kAttnT + wave + (c + u) * NW];
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const int j = wave + (c + u) * NW;
        lds_load16(entry_or_zero(a.kv, ev[u]) + 8 * lane, mbase + 2 * j * kKPitch);
      }
    }
#pragma unroll
    for (int v = 0; v < 4 / NW; ++v) {
      const int q = wave + v * NW;
      const int j = 8 * q + (lane >> 3);
      lds_load16(entry_or_zero(a.kv, tv[v]) + kAttnDV + 8 * ((lane & 7) ^ (j & 7)), tbase + 1024 * q);
    }
  };
  // value operand of dims 16n .. 16n + 15: lane (g, c16) gets tokens 8g .. 8g + 7 of dim
  // 16n + c16, from two transposing reads (tokens 8g + c16 / 4 and 8g + 4 + c16 / 4, dims
  // 16n + 4 (c16 % 4) .. + 3)
  typedef __attribute__((address_space(3))) v4bf lds_v4bf;
  const int tr_off = (8 * g + (c16 >> 2)) * kKPitch + 4 * (c16 & 3);
  auto read_v = [&](const uint16_t* kt, int n) -> v8bf {
    const v4bf lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(&kt[tr_off + 16 * n]));
    const v4bf hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(&kt[tr_off + 4 * kKPitch + 16 * n]));
    return v8bf{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };

  float m[4], l[4];
  v4f o[kAttnDV / 16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -__builtin_inff();
    l[i] = 0.f;
  }
#pragma unroll
  for (int n = 0; n < kAttnDV / 16; ++n) o[n] = v4f{0.f, 0.f, 0.f, 0.f};

  auto tile = [&](const uint16_t* km, const uint16_t* kd, bool v0, bool v1) {

    // scores of the tile's two 16-token columns: all 36 operand reads are issued before
    // the MFMAs, which then wait for them in order instead of one LDS round trip each
    v4f sc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
    v8bf kb[2][kAttnD / 32];
#pragma unroll
    for (int s = 0; s < kAttnD / 32; ++s)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int tok = 16 * j + c16;
        kb[j][s] = s < kAttnDV / 32 ? *(const v8bf*)(&km[tok * kKPitch + 32 * s + 8 * g])
                                    : *(const v8bf*)(&kd[tok * kTail + 8 * ((4 * (s - kAttnDV / 32) + g) ^ (c16 & 7))]);
      }
#pragma unroll
    for (int s = 0; s < kAttnD / 32; ++s)
#pragma unroll
      for (int j = 0; j < 2; ++j) sc[j] = mfma_bf16(qa[s], kb[j][s], sc[j]);
    // lane (g, c16): heads 4g + i, tokens c16 and 16 + c16 of the tile
    float p[2][4], alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float s0 = v0 ? sc[0][i] * a.scale2 : -__builtin_inff();
      const float s1 = v1 ? sc[1][i] * a.scale2 : -__builtin_inff();
      const float mt = dpp_row_max(fmaxf(s0, s1));
      const float mn = fmaxf(m[i], mt);
      // all -inf so far: keep weights 0 (exp2(-inf) = 0, and no -inf - -inf)
      const float base = mn == -__builtin_inff() ? 0.f : mn;
      alpha[i] = __builtin_amdgcn_exp2f(m[i] - base);
      p[0][i] = __builtin_amdgcn_exp2f(s0 - base);
      p[1][i] = __builtin_amdgcn_exp2f(s1 - base);
      l[i] = l[i] * alpha[i] + dpp_row_sum(p[0][i] + p[1][i]);
      m[i] = mn;
    }
#pragma unroll
    for (int n = 0; n < kAttnDV / 16; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[n][i] *= alpha[i];
    // P into the A-operand layout: row = head, 8 consecutive tokens per lane group
    uint16_t* pw = pb[wave];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) pw[(4 * g + i) * kPPitch + 16 * j + c16] = f32_to_bf16(p[j][i]);
    __builtin_amdgcn_wave_barrier();  // one wave's LDS operations complete in order
    const v8bf pa = *(const v8bf*)(&pw[c16 * kPPitch + 8 * g]);
    // value operands in two batches of 16 reads, each ahead of its MFMAs
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v8bf vb[kAttnDV / 32];
#pragma unroll
      for (int n = 0; n < kAttnDV / 32; ++n) vb[n] = read_v(km, 16 * h + n);
#pragma unroll
      for (int n = 0; n < kAttnDV / 32; ++n) o[16 * h + n] = mfma_bf16(pa, vb[n], o[16 * h + n]);
    }
    __builtin_amdgcn_wave_barrier();  // the P reads finish before the next tile's writes
  };
  // One tile buffer (three workgroups share a compute unit, so their loads and math
  // overlap one another's). The fence before each load completes this wave's LDS reads
  // of the previous tile; the one after the wait orders the tile's reads behind it.
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    dma(t, 0);
    __builtin_amdgcn_s_waitcnt(vmcnt_enc(0));
    __syncthreads();
    const bool v0 = ent[t * kAttnT + c16] >= 0;
    const bool v1 = ent[t * kAttnT + 16 + c16] >= 0;
    tile(kt[0], kl[0], v0, v1);
  }

  // lane (g, c16) holds O[head 4g + i][dim 16n + c16]
  if (a.nsplit == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = head0 + 4 * g + i;
      const float inv = l[i] > 0.f ? 1.f / l[i] : 0.f;
      float* orow = a.out + ((int64_t)r * a.heads + h) * kAttnDV;
#pragma unroll
      for (int n = 0; n < kAttnDV / 16; ++n) orow[16 * n + c16] = o[n][i] * inv;
      if (a.lse && c16 == 0)
        a.lse[(int64_t)r * a.heads + h] = l[i] > 0.f ? (m[i] + log2f(l[i])) * 0.69314718055994531f : -__builtin_inff();
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = head0 + 4 * g + i;
      const int64_t slot = ((int64_t)r * a.nsplit + split) * a.heads + h;
      float* orow = a.part_o + slot * kAttnDV;
#pragma unroll
      for (int n = 0; n < kAttnDV / 16; ++n) orow[16 * n + c16] = o[n][i];
      if (c16 == 0) {
        a.part_ml[2 * slot] = m[i];
        a.part_ml[2 * slot + 1] = l[i];
      }
    }
  }
}

// One wave per (row, head): merges the splits' (O, m, l).
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Lane s reads split s's (m, l) (at most 64 splits; the split count never exceeds 16),
// then the splits' output rows are read up to four at a time, all their loads issued
// before any is used.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int64_t wv = ((int64_t)blockIdx.x * 256 + threadIdx.x) / kWave;
  if (wv >= (int64_t)a.rows * a.heads) return;
  const int lane = lane_id();
  const int64_t r = wv / a.heads, h = wv % a.heads;
  const int ns = a.nsplit;
  float ms = -__builtin_inff(), ls = 0.f;
  if (lane < ns) {
    const int64_t slot = (r * ns + lane) * a.heads + h;
    ms = a.part_ml[2 * slot];
    ls = a.part_ml[2 * slot + 1];
  }
  const float mx = wave_max_f(ms);
  const float base = mx == -__builtin_inff() ? 0.f : mx;
  const float ws = lane < ns ? exp2f(ms - base) : 0.f;  // 0 for a split without entries
  const float L = wave_sum_f(ws * ls);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < ns; s0 += 4) {
    float4 x[4][2];
    float w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // past the last split: nothing read, weight 0 (the condition is wave-uniform)
      w[q] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ws), s0 + q));
      x[q][0] = x[q][1] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (s0 + q < ns) {
        const float4* src = (const float4*)(a.part_o + ((r * ns + s0 + q) * a.heads + h) * kAttnDV) + 2 * lane;
        x[q][0] = src[0];
        x[q][1] = src[1];
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[0] += w[q] * x[q][0].x; acc[1] += w[q] * x[q][0].y; acc[2] += w[q] * x[q][0].z; acc[3] += w[q] * x[q][0].w;
      acc[4] += w[q] * x[q][1].x; acc[5] += w[q] * x[q][1].y; acc[6] += w[q] * x[q][1].z; acc[7] += w[q] * x[q][1].w;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float4* dst = (float4*)(a.out + (r * a.heads + h) * kAttnDV) + 2 * lane;
  dst[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  dst[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  if (a.lse && lane == 0) a.lse[r * a.heads + h] = L > 0.f ? (mx + log2f(L)) * 0.69314718055994531f : -__builtin_inff();
}

static int head_waves(int heads) { return std::min(heads, 64) / 16; }

int attn_splits(int rows, int heads, int k) {
  // enough workgroups to fill the MI355X's 256 compute units once: one 4-wave group per
  // CU (registers), two 2-wave groups, three 1-wave groups (LDS); each split at least
  // four tiles (a fixed count keeps the workspace size independent of the device)
  const int nw = head_waves(heads);
  const int kTargetGroups = nw == 1 ? 768 : nw == 2 ? 512 : 256;
  const int hgroups = heads / (16 * nw);
  const int want = (kTargetGroups + rows * hgroups - 1) / (rows * hgroups);
  const int most = std::max(1, (k + 4 * kAttnT - 1) / (4 * kAttnT));
  return std::max(1, std::min(want, most));
}

static int split_len(int k, int nsplit) {
  const int per = (k + nsplit - 1) / nsplit;
  return (per + kAttnT - 1) / kAttnT * kAttnT;
}

size_t attn_workspace_bytes(int rows, int heads, int k) {
  const int ns = attn_splits(rows, heads, k);
  if (ns <= 1 || rows <= 0) return 0;
  const size_t o = (size_t)rows * ns * heads * kAttnDV * sizeof(float);
  const size_t ml = (size_t)rows * ns * heads * 2 * sizeof(float);
  return (o + 255) / 256 * 256 + (ml + 255) / 256 * 256;
}

// The entry list is dynamic LDS (up to IDX_MAX_K rows) next to ~88 KB of static LDS.
static hipError_t launch_partial_1w(dim3 grid, size_t ent_bytes, hipStream_t stream, const AttnArgs& a) {
  hipLaunchKernelGGL(attn_partial_1w_kernel, grid, dim3(kWave), ent_bytes, stream, a);
  return hipGetLastError();
}

template <int NW>
static hipError_t launch_partial(dim3 grid, size_t ent_bytes, hipStream_t stream, const AttnArgs& a) {
  static PerDeviceOnce once;
  const hipError_t attr = once.run([] {
    return hipFuncSetAttribute((const void*)attn_partial_kernel<NW>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               2048 * (int)sizeof(int64_t));
  });
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(attn_partial_kernel<NW>, grid, dim3(NW * kWave), ent_bytes, stream, a);
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const AttnCall& c, void* workspace, hipStream_t stream) {
  if (c.rows <= 0) return hipSuccess;
  AttnArgs a{};
  a.q = (const uint16_t*)c.q;
  a.kv = (const uint16_t*)c.kv;
  a.n_pages = c.n_pages;
  a.page_size = c.page_size;
  a.bt = c.block_table;
  a.bt_rows = c.bt_rows;
  a.bt_ld = c.bt_ld;
  a.seq_lens = c.seq_lens;
  a.row_req = c.row_req;
  a.idx = c.indices;
  a.idx_ld = c.idx_ld;
  a.k = c.k;
  a.rows = c.rows;
  a.heads = c.heads;
  a.scale2 = c.scale * kLog2e;
  a.nsplit = attn_splits(c.rows, c.heads, c.k);
  a.split_len = split_len(c.k, a.nsplit);
  if (a.nsplit > kWave) return hipErrorInvalidValue;  // the combine gives each split a lane
  const int nw = head_waves(c.heads);
  a.hgroups = c.heads / (16 * nw);
  a.out = c.out;
  a.lse = c.lse;
  a.err = c.err;
  if (a.nsplit > 1) {
    const size_t o = (size_t)c.rows * a.nsplit * c.heads * kAttnDV * sizeof(float);
    a.part_o = (float*)workspace;
    a.part_ml = (float*)((uint8_t*)workspace + (o + 255) / 256 * 256);
  }
  const int64_t units = (int64_t)c.rows * a.nsplit;
  const dim3 grid((unsigned)((units + 7) / 8 * 8 * a.hgroups));
  const size_t ent_bytes = (size_t)a.split_len * sizeof(int64_t);
  hipError_t e = hipSuccess;
  switch (nw) {
    case 1: e = launch_partial_1w(grid, ent_bytes, stream, a); break;
    case 2: e = launch_partial<2>(grid, ent_bytes, stream, a); break;
    default: e = launch_partial<4>(grid, ent_bytes, stream, a); break;
  }
  if (e != hipSuccess || a.nsplit == 1) return e;
  const int64_t waves = (int64_t)c.rows * c.heads;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsaidx
