// Exact top-k per row (the fine-grained token selection of the DeepSeek-V3.2
// architecture section).
//
// Selection key. Every entry gets a 64-bit key: the order-preserving image of its
// fp32 score in the high word and the bitwise complement of its column in the low
// word, so "larger key" means "higher score, then lower column" and no two entries
// tie. The k winners are exactly the keys >= the k-th largest key.
//
// Both paths first build a 12-bit histogram of the value keys, which fixes the bin
// that holds the k-th largest entry (the "cut" bin): every entry above it is a
// winner, entries below it are not, and only the entries in the cut bin (the
// candidates) need a closer look. The missing winners are found among the candidates
// by MSB-first radix select with 8-bit digits, starting below the 12 bits the bin
// already fixes; ties between equal scores are settled by the column word. This is
// the sampled-filtering idea of the persistent top-k on the pages with an exact
// histogram instead of a sample, so the cut estimate is never wrong.
//
// Short rows (n_cols <= kShortRow) take one workgroup per row with the row's value
// keys cached in LDS, so the row is read from memory once. Long rows use the whole
// chip: segments of every row add into a global row histogram (hist), then every
// segment streams out its winners and candidates (filter), then one workgroup per
// row selects among the candidates and writes the row (finish). A cut bin with more
// candidates than the lists hold (e.g. a row of equal scores) is resolved by radix
// passes over the whole row instead.
//
// Sorted output is ordered by a bitonic network over registers: strides inside a
// thread compare registers, strides inside a wave exchange through DPP and
// permlane moves, and only strides across waves go through LDS.
#include "device.h"
#include "launch.h"
#include "topk_device.h"

#include <algorithm>
#include <mutex>

namespace dsaidx {

// ------------------------------------------------------------------ loads

// Four row entries starting at i (a multiple of 4) of a row of n entries: one 16-byte
// load when all four exist and the row is 16-byte aligned, -inf past the end. LAST:
// the last read of the data (a non-temporal load).
template <bool V4, bool LAST>
__device__ __forceinline__ float4 load4(const float* row, int64_t i, int64_t n) {
  if (V4 && i + 4 <= n) {
    const v4f* p = (const v4f*)(row + i);
    const v4f x = LAST ? __builtin_nontemporal_load(p) : *p;
    return make_float4(x[0], x[1], x[2], x[3]);
  }
  float4 v;
  v.x = i < n ? row[i] : -__builtin_inff();
  v.y = i + 1 < n ? row[i + 1] : -__builtin_inff();
  v.z = i + 2 < n ? row[i + 2] : -__builtin_inff();
  v.w = i + 3 < n ? row[i + 3] : -__builtin_inff();
  return v;
}

// ------------------------------------------------------------------ short rows

template <bool V4, int NT>
__global__ __launch_bounds__(NT) void topk_short_kernel(TopkCall a) {
  extern __shared__ uint4 dyn[];                 // the row's value keys (n_cols rounded up to 4, at
                                                 // least kMaxK keys' worth), then the sorted keys
  uint32_t* vkeys = (uint32_t*)dyn;
  // value histogram, then the cut bin's columns and the radix select's digit counts,
  // then the bucket counts (LDS small enough for three workgroups per CU at 8192 columns)
  __shared__ __align__(16) union {
    uint32_t hist[kHistBins];
    struct {
      uint16_t cand[kShortCandCap];
      uint32_t rh[256];
    } c;
  } u;
  __shared__ uint16_t sel[kMaxK];                // selected columns
  __shared__ RadixShared sh;
  __shared__ CutInfo ci;
  __shared__ SortShared ss;
  __shared__ uint32_t n_sel, n_cand;
  __shared__ unsigned long long n_list;  // the filter's winners << 32 | candidates
  const int tid = threadIdx.x;
  const int r = blockIdx.x;
  const int64_t n = row_len(a, r);
  for (int i = tid; i < kHistBins; i += NT) u.hist[i] = 0;
  if (tid == 0) {
    n_sel = 0;
    n_cand = 0;
    n_list = 0;
  }
  __syncthreads();

  // 1. value keys into LDS and the histogram
  const float* row = a.logits + (int64_t)r * a.ld;
  constexpr int U = 4;  // four-entry groups per thread per pass
  for (int64_t b = 0; b < n; b += (int64_t)NT * 4 * U) {
    float4 v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) v[j] = load4<V4, true>(row, b + ((int64_t)j * NT + tid) * 4, n);
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t i = b + ((int64_t)j * NT + tid) * 4;
      if (i < n) {
        uint4 kk;
        kk.x = order_key(v[j].x);
        kk.y = order_key(v[j].y);
        kk.z = order_key(v[j].z);
        kk.w = order_key(v[j].w);
        dyn[i / 4] = kk;
        if (kk.x) atomicAdd(&u.hist[kk.x >> kBinShift], 1u);
        if (kk.y) atomicAdd(&u.hist[kk.y >> kBinShift], 1u);
        if (kk.z) atomicAdd(&u.hist[kk.z >> kBinShift], 1u);
        if (kk.w) atomicAdd(&u.hist[kk.w >> kBinShift], 1u);
      }
    }
  }
  __syncthreads();

  // 2. the cut bin
  find_cut<NT>(u.hist, a.k, ci);
  const int cut = ci.bin;
  const bool compact = ci.count <= (uint32_t)kShortCandCap;
  const uint32_t keff = min((uint32_t)a.k, ci.total);

  // 3. winners above the cut, candidates in it
  // each lane marks its winners and candidates in two bit masks (bit j: entry
  // b + j NT + tid); one wave prefix sum of the packed counts (winners << 16 |
  // candidates, at most 8 each per lane) and one LDS atomic place both lists
  constexpr int U2 = 8;
  for (int64_t b = 0; b < n; b += (int64_t)NT * U2) {
    uint32_t wbits = 0u, cbits = 0u;
#pragma unroll
    for (int j = 0; j < U2; ++j) {
      const int64_t i = b + (int64_t)j * NT + tid;
      const uint32_t v = i < n ? vkeys[i] : 0u;
      const int bin = v ? (int)(v >> kBinShift) : -2;
      wbits |= bin > cut ? 1u << j : 0u;
      cbits |= compact && bin == cut ? 1u << j : 0u;
    }
    const uint32_t mine = ((uint32_t)__popc(wbits) << 16) | (uint32_t)__popc(cbits);
    const uint32_t incl = wave_inclusive_sum(mine);
    const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
    if (tot != 0u) {
      unsigned long long base = 0;
      if (lane_id() == 0) base = atomicAdd(&n_list, ((unsigned long long)(tot >> 16) << 32) | (tot & 0xFFFFu));
      const uint32_t bw = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32));
      const uint32_t bc = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base);
      const uint32_t excl = incl - mine;
      auto col = [&](int bit) { return (uint32_t)(b + (int64_t)bit * NT + tid); };
      uint32_t ws = bw + (excl >> 16), cs = bc + (excl & 0xFFFFu);
      for (; wbits != 0u; wbits &= wbits - 1u, ++ws)
        if (ws < (uint32_t)kMaxK) sel[ws] = (uint16_t)col(__builtin_ctz(wbits));
      for (; cbits != 0u; cbits &= cbits - 1u, ++cs)
        if (cs < (uint32_t)kShortCandCap) u.c.cand[cs] = (uint16_t)col(__builtin_ctz(cbits));
    }
  }
  __syncthreads();
  if (tid == 0) {
    n_sel = (uint32_t)(n_list >> 32);
    n_cand = (uint32_t)n_list;
  }
  __syncthreads();

  // 4. the rest of the winners from the cut bin
  const uint32_t have = n_sel;
  const uint32_t need = keff - have;
  if (need > 0) {
    const uint64_t pre = (uint64_t)cut << kKeyBinShift;
    if (compact) {
      const uint32_t nc = n_cand;
      auto get = [&](int64_t i) -> uint64_t {
        const uint32_t c = u.c.cand[i];
        return sel_key(vkeys[c], c);
      };
      const uint64_t thr = need == nc ? 1ull : radix_threshold<NT>(get, nc, need, sh, u.c.rh, pre, kKeyBinShift);
      gather_at_least<NT, uint16_t>(get, [&](int64_t i) { return u.c.cand[i]; }, nc, thr, sel, &n_sel,
                                    (uint32_t)kMaxK);
    } else {
      auto get = [&](int64_t i) -> uint64_t {
        const uint32_t v = vkeys[i];
        return (int)(v >> kBinShift) == cut ? sel_key(v, i) : 0ull;
      };
      const uint64_t thr = radix_threshold<NT>(get, n, need, sh, u.c.rh, pre, kKeyBinShift);
      gather_at_least<NT, uint16_t>(get, [&](int64_t i) { return (uint16_t)i; }, n, thr, sel, &n_sel,
                                    (uint32_t)kMaxK);
    }
  }
  __syncthreads();

  // 5. the row
  auto key = [&](int i) -> uint64_t {
    const uint32_t c = sel[i];
    return sel_key(vkeys[c], c);
  };
  // the sort's bounds from the histogram: every selected key lies in bins cut .. top
  uint32_t lo_key = 0u, hi_key = 0u;
  if (cut >= 0) bin_bounds(cut, ci.top, lo_key, hi_key);
  if (a.sorted)
    bucket_sort_write<NT>(a, r, key, (int)keff, u.hist, (uint64_t*)dyn, ss, lo_key, hi_key);
  else
    write_list<NT>(a, r, key, (int)keff);
}

// ------------------------------------------------------------------ short rows, one pass

// Rows of up to NT * PER entries, each thread's PER of them held in registers: the
// row's buckets, linear in the score between its smallest and largest entry (a
// monotone map), both pick the k-th largest entry and order the winners. Every entry
// counts itself into its bucket; an exclusive scan of the counts from the highest
// bucket down gives each bucket's first position and the cut bucket, the one holding
// the k-th largest entry. Every entry in the cut bucket or above takes a position of its
// bucket in LDS, and its place in the row is its bucket's first position plus the
// number of larger keys in the same bucket; places past k are not written. A bucket at
// or above the cut holding more than kBucketCap entries (equal or clustered scores, a
// far outlier) sends the row to an exact path instead: a radix threshold over the row's
// keys (in LDS, or read again from memory for rows wider than 8192), the columns at or
// above it, and a bitonic sort of those.
template <bool V4, int NT, int PER>
__global__ __launch_bounds__(NT, PER <= 16 ? 8 : 4) void topk_lin_kernel(TopkCall a) {
  static_assert(PER % 4 == 0 && kBuckets % (4 * NT) == 0, "four entries per load, four counts per read");
  constexpr int kTmp = kMaxK + kBucketCap;    // keys at or above the cut bucket
  constexpr int per = kBuckets / NT;          // buckets a thread scans
  constexpr int waves = NT / kWave;
  // bucket counts (then first positions) and the keys at or above the cut bucket; for a
  // row the buckets cannot sort, the row's value keys (rows of up to 8192 entries; longer
  // ones are read again from memory)
  constexpr bool kKeysInLds = NT * PER <= 8192;
  __shared__ __align__(16) union {
    struct {
      uint32_t cnt[kBuckets];
      uint64_t tmp[kTmp];
    } b;
    uint32_t vk[kKeysInLds ? NT * PER : 1];
  } u;
  static_assert(sizeof(u.vk) <= sizeof(u.b) && kTmp >= kMaxK && NT * PER <= 65536,
                "the row's keys fit the bucket space; columns fit 16 bits");
  uint32_t* cnt = u.b.cnt;
  uint64_t* tmp = u.b.tmp;
  __shared__ uint16_t sel[kMaxK];                    // exact path: the winners' columns
  __shared__ uint32_t rh[256];
  __shared__ RadixShared sh;
  __shared__ uint32_t wmx[waves], wmn[waves], wsum[waves];
  __shared__ uint32_t s_cut, s_fill, s_big, n_sel;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wv = tid / kWave;
  const int r = blockIdx.x;
  const int64_t n = row_len(a, r);
  const float* row = a.logits + (int64_t)r * a.ld;

  // entry e of this thread: column 4 (e / 4 * NT + tid) + e % 4 (plain loads: the scores
  // were mostly just written by the score kernel, and non-temporal loads of them measured
  // 2 us slower on the prefill chunk's 4096 rows)
  uint32_t key[PER];
#pragma unroll
  for (int g = 0; g < PER / 4; ++g) {
    const float4 v = load4<V4, false>(row, ((int64_t)g * NT + tid) * 4, n);
    key[4 * g] = order_key(v.x);
    key[4 * g + 1] = order_key(v.y);
    key[4 * g + 2] = order_key(v.z);
    key[4 * g + 3] = order_key(v.w);
  }
  for (int i = tid; i < kBuckets / 4; i += NT) ((uint4*)cnt)[i] = make_uint4(0u, 0u, 0u, 0u);
  if (tid == 0) {
    s_big = 0u;
    n_sel = 0u;
  }
  // the smallest and largest present key
  uint32_t mx = 0u, mn = ~0u;  // the smallest key less one (absent keys wrap to the top)
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    mx = max(mx, key[e]);
    mn = min(mn, key[e] - 1u);
  }
#pragma unroll
  for (int lb = 0; lb < 6; ++lb) {
    mx = max(mx, xor_lane(mx, lb));
    mn = min(mn, xor_lane(mn, lb));
  }
  if (lane == 0) {
    wmx[wv] = mx;
    wmn[wv] = mn;
  }
  __syncthreads();
  uint32_t lo_key = ~0u, hi_key = 0u;
#pragma unroll
  for (int w = 0; w < waves; ++w) {
    lo_key = min(lo_key, wmn[w]);
    hi_key = max(hi_key, wmx[w]);
  }
  ++lo_key;
  int32_t* oi = a.out_idx + (int64_t)r * a.out_ld;
  float* ov = a.out_val ? a.out_val + (int64_t)r * a.out_ld : nullptr;
  if (hi_key == 0u) {  // nothing present
    for (int i = tid; i < a.k; i += NT) {
      oi[i] = -1;
      if (ov) ov[i] = -__builtin_inff();
    }
    return;
  }
  // bucket of a key, highest first: (v - lo) * scale, clamped (NaN, only from 0 * inf,
  // goes to the lowest); an absent key gets kBuckets, past every bucket
  const float lo = key_value(lo_key);
  const float d = key_value(hi_key) - lo;
  const float scale = (d > 0.f && d <= 3.0e38f) ? (float)(kBuckets - 0.01) / d : 0.f;
  auto bucket = [&](uint32_t k) -> uint32_t {
    const float f = (key_value(k) - lo) * scale;
    const int b = f >= 1.f ? min((int)f, kBuckets - 1) : 0;
    return k ? (uint32_t)(kBuckets - 1 - b) : (uint32_t)kBuckets;
  };
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const uint32_t b = bucket(key[e]);
    if (b < (uint32_t)kBuckets) atomicAdd(&cnt[b], 1u);
  }
  __syncthreads();

  // exclusive scan of the counts (thread t: buckets per t ..), the cut bucket, and
  // whether a bucket at or above it is too full
  uint32_t c[per], sum = 0u;
#pragma unroll
  for (int j = 0; j < per; j += 4) {
    const uint4 q = ((const uint4*)cnt)[per / 4 * tid + j / 4];
    c[j] = q.x;
    c[j + 1] = q.y;
    c[j + 2] = q.z;
    c[j + 3] = q.w;
  }
#pragma unroll
  for (int j = 0; j < per; ++j) sum += c[j];
  const uint32_t incl = wave_inclusive_sum(sum);
  if (lane == kWave - 1) wsum[wv] = incl;
  __syncthreads();
  uint32_t off = incl - sum, total = 0u;
#pragma unroll
  for (int w = 0; w < waves; ++w) {
    off += w < wv ? wsum[w] : 0u;
    total += wsum[w];
  }
  const uint32_t keff = min((uint32_t)a.k, total);
  {
    uint32_t o = off, jc = ~0u, fc = 0u;
    bool big = false;
#pragma unroll
    for (int j = 0; j < per; ++j) {
      big |= o < keff && c[j] > (uint32_t)kBucketCap;
      const bool here = o < keff && keff <= o + c[j];
      jc = here ? (uint32_t)j : jc;
      fc = here ? o + c[j] : fc;
      o += c[j];
    }
    if (jc != ~0u) {
      s_cut = (uint32_t)per * tid + jc;
      s_fill = fc;
    }
    if (big) s_big = 1u;
  }
#pragma unroll
  for (int j = 0; j < per; j += 4) {
    uint4 q;
    q.x = off;
    q.y = q.x + c[j];
    q.z = q.y + c[j + 1];
    q.w = q.z + c[j + 2];
    off = q.w + c[j + 3];
    ((uint4*)cnt)[per / 4 * tid + j / 4] = q;
  }
  __syncthreads();
  const uint32_t cut = s_cut, fill = s_fill;
  const int32_t* cand_row = a.cand ? a.cand + (int64_t)r * a.cand_ld : nullptr;

  if (!s_big) {
    // the entries at or above the cut bucket to their bucket's positions (each bucket's
    // first position counts up to the next bucket's); the buckets are computed again
    // rather than kept from the count (the empty asm hides that they are the same)
    int t4 = 4 * tid;
    asm volatile("" : "+v"(t4));  // nor the columns kept from the start
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      asm volatile("" : "+v"(key[e]));
      const uint32_t b = bucket(key[e]);
      if (b <= cut) {
        const int64_t col = (int64_t)(e / 4) * NT * 4 + t4 + (e & 3);
        tmp[atomicAdd(&cnt[b], 1u)] = sel_key(key[e], col);
      }
    }
    __syncthreads();
    // each one's place: its bucket's first position (the end of the bucket above) plus
    // the larger keys of its bucket
    for (uint32_t i = tid; i < fill; i += NT) {
      const uint64_t x = tmp[i];
      const uint32_t b = bucket((uint32_t)(x >> 32));
      const uint32_t st = b > 0 ? cnt[b - 1] : 0u;
      const uint32_t len = cnt[b] - st;
      uint32_t pos = st;
      for (uint32_t j = 0; j < len; j += 4) {
        uint64_t v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = tmp[st + min(j + q, len - 1)];
#pragma unroll
        for (int q = 0; q < 4; ++q) pos += (j + q < len) & (v[q] > x);
      }
      if (pos < keff) {
        oi[pos] = out_index(a, cand_row, key_col(x));
        if (ov) ov[pos] = key_value((uint32_t)(x >> 32));
      }
    }
    for (int i = (int)keff + tid; i < a.k; i += NT) {
      oi[i] = -1;
      if (ov) ov[i] = -__builtin_inff();
    }
    return;
  }

  // a full bucket: the row's value keys to LDS, the exact threshold by radix passes over
  // them, then the columns at or above it, bitonic-sorted (the sort's exchange space
  // overlaps the keys, which it reads before its first barrier)
  if constexpr (kKeysInLds) {
    for (int g = 0; g < PER / 4; ++g) {
      const float4 v = load4<V4, false>(row, ((int64_t)g * NT + tid) * 4, n);
      ((uint4*)u.vk)[g * NT + tid] = make_uint4(order_key(v.x), order_key(v.y), order_key(v.z), order_key(v.w));
    }
    __syncthreads();
  }
  auto get = [&](int64_t i) -> uint64_t {
    const uint32_t v = kKeysInLds ? u.vk[i] : order_key(row[i]);
    return v ? sel_key(v, i) : 0ull;
  };
  const uint64_t thr = keff == total ? 1ull : radix_threshold<NT>(get, n, keff, sh, rh);
  gather_at_least<NT, uint16_t>(get, [&](int64_t i) { return (uint16_t)i; }, n, thr, sel, &n_sel,
                                (uint32_t)kMaxK);
  auto keyf = [&](int i) -> uint64_t { return get(sel[i]); };
  if (a.sorted)
    sort_and_write<NT>(a, r, keyf, (int)keff, tmp);
  else
    write_list<NT>(a, r, keyf, (int)keff);
}

// ------------------------------------------------------------------ long rows

struct LongWs {
  uint32_t* hist;    // [rows, kHistBins]
  uint32_t* counts;  // [rows, 2]: winners above the cut, candidates
  uint64_t* win;     // [rows, kMaxK]
  uint64_t* cand;    // [rows, kCandCap]
};

__global__ __launch_bounds__(kSegThreads) void topk_zero_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kSegThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kSegThreads)
    p[i] = 0u;
}

// Four-entry groups per thread per pass of the segment loops: independent loads issued
// together so the loop is not bound by one memory latency per load.
constexpr int kSegGroups = 4;  // 16 entries per thread: one 16-bit mask per list in the filter
static_assert(kSegGroups * 4 <= 16, "the filter packs per-lane counts into 16-bit halves");
constexpr int kSegStep = kSegThreads * 4 * kSegGroups;

// Histogram bin of a present score (not -inf or NaN): order_key's bin with
// branch-free arithmetic (-0 is folded onto +0 by adding +0).
__device__ __forceinline__ uint32_t hist_bin(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  return (u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u)) >> kBinShift;
}

template <bool V4>
__global__ __launch_bounds__(kSegThreads) void topk_hist_kernel(TopkCall a, LongWs ws, int64_t seg, int segs) {
  __shared__ uint32_t hist[kHistBins];
  const int r = (int)(blockIdx.x / (unsigned)segs);
  const int64_t n = row_len(a, r);
  const int64_t s0 = (int64_t)(blockIdx.x % (unsigned)segs) * seg;
  const int64_t s1 = min(s0 + seg, n);
  if (s0 >= s1) return;
  for (int i = threadIdx.x; i < kHistBins; i += kSegThreads) hist[i] = 0;
  __syncthreads();
  const float* row = a.logits + (int64_t)r * a.ld;
  for (int64_t b = s0; b < s1; b += kSegStep) {
    float4 v[kSegGroups];
#pragma unroll
    for (int j = 0; j < kSegGroups; ++j) v[j] = load4<V4, false>(row, b + ((int64_t)j * kSegThreads + threadIdx.x) * 4, s1);
#pragma unroll
    for (int j = 0; j < kSegGroups; ++j) {
      const float e[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (e[c] > -__builtin_inff()) atomicAdd(&hist[hist_bin(e[c])], 1u);
    }
  }
  __syncthreads();
  uint32_t* g = ws.hist + (int64_t)r * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += kSegThreads)
    if (hist[i]) atomicAdd(&g[i], hist[i]);
}

// Candidates one filter workgroup stages in LDS; a segment with more forces its row
// onto the full-row path (the candidate count is pushed past kCandCap). The LDS lists
// hold columns (4 bytes), so a workgroup needs 24 KiB and every segment of the
// workloads' shapes is resident at once.
constexpr int kSegCandCap = 4096;

// Appends the columns of the set bits of bits (bit j = entry j of the lane's group
// pattern, col(j)) to an LDS list at slot, one lane-serial store per set bit.
template <class Col>
__device__ __forceinline__ void append_bits(uint32_t bits, uint32_t slot, uint32_t* list, uint32_t cap, const Col& col) {
  for (; bits != 0u; bits &= bits - 1u, ++slot)
    if (slot < cap) list[slot] = col(__builtin_ctz(bits));
}

template <bool V4>
__global__ __launch_bounds__(kSegThreads) void topk_filter_kernel(TopkCall a, LongWs ws, int64_t seg, int segs) {
  __shared__ CutInfo ci;
  __shared__ uint32_t lwin[kMaxK];
  __shared__ uint32_t lcand[kSegCandCap];
  __shared__ unsigned long long n_list;  // winners << 32 | candidates
  __shared__ uint32_t base_win, base_cand;
  const int r = (int)(blockIdx.x / (unsigned)segs);
  const int64_t n = row_len(a, r);
  const int64_t s0 = (int64_t)(blockIdx.x % (unsigned)segs) * seg;
  const int64_t s1 = min(s0 + seg, n);
  if (s0 >= s1) return;
  if (threadIdx.x == 0) n_list = 0;
  find_cut<kSegThreads>(ws.hist + (int64_t)r * kHistBins, a.k, ci);
  const int cut = ci.bin;
  // a cut bin too large for the workspace is resolved from the row itself
  const bool keep_cand = ci.count <= (uint32_t)kCandCap;
  // The cut bin as value bounds, so that classifying an entry takes two compares: it
  // is a winner when its bin is above the cut, x >= t_hi (the smallest value of bin
  // cut + 1), and a candidate when it is in the cut bin, x >= t_lo and not a winner.
  // -inf and NaN compare false and -0 == +0, as in order_key. Bins below 8 hold only
  // the keys of NaN and -inf, which are never counted, so a cut bin's bounds are real
  // values; past +inf's bin nothing is a winner (a NaN bound compares false).
  const float no_bound = __builtin_nanf("");
  float t_hi, t_lo;
  if (cut < 0) {  // at most k present entries: all are winners
    t_hi = -__FLT_MAX__;
    t_lo = no_bound;
  } else {
    const uint64_t hk = (uint64_t)(cut + 1) << kBinShift;
    t_hi = hk > 0xFF800000ull ? no_bound : key_value((uint32_t)hk);
    t_lo = keep_cand ? key_value((uint32_t)cut << kBinShift) : no_bound;
  }
  const float* row = a.logits + (int64_t)r * a.ld;
  // every thread runs the same number of iterations so whole waves vote together
  for (int64_t b = s0; b < s1; b += kSegStep) {
    float4 v[kSegGroups];
#pragma unroll
    for (int j = 0; j < kSegGroups; ++j) v[j] = load4<V4, false>(row, b + ((int64_t)j * kSegThreads + threadIdx.x) * 4, s1);
    // bit 4j + c of a lane's masks: entry c of its group j
    uint32_t wbits = 0u, cbits = 0u;
#pragma unroll
    for (int j = 0; j < kSegGroups; ++j) {
      const float e[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool w = e[c] >= t_hi;
        wbits |= w ? 1u << (4 * j + c) : 0u;
        cbits |= (!w && e[c] >= t_lo) ? 1u << (4 * j + c) : 0u;
      }
    }
    // one wave prefix sum and one LDS atomic place both lists' entries (a lane holds
    // at most 16 of each, so the packed halves winners << 16 | candidates never carry)
    const uint32_t mine = ((uint32_t)__popc(wbits) << 16) | (uint32_t)__popc(cbits);
    const uint32_t incl = wave_inclusive_sum(mine);
    const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
    if (tot != 0u) {
      unsigned long long base = 0;
      if (lane_id() == 0) base = atomicAdd(&n_list, ((unsigned long long)(tot >> 16) << 32) | (tot & 0xFFFFu));
      const uint32_t bw = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32));
      const uint32_t bc = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base);
      const uint32_t excl = incl - mine;
      auto col = [&](int bit) {
        return (uint32_t)(b + ((int64_t)(bit >> 2) * kSegThreads + threadIdx.x) * 4 + (bit & 3));
      };
      append_bits(wbits, bw + (excl >> 16), lwin, (uint32_t)kMaxK, col);
      append_bits(cbits, bc + (excl & 0xFFFFu), lcand, (uint32_t)kSegCandCap, col);
    }
  }
  __syncthreads();
  uint32_t* cnt = ws.counts + 2 * (int64_t)r;
  const unsigned long long nl = n_list;
  const uint32_t nw = min((uint32_t)(nl >> 32), (uint32_t)kMaxK);
  const uint32_t nc = (uint32_t)nl;
  if (threadIdx.x == 0) {
    base_win = nw ? atomicAdd(&cnt[0], nw) : 0u;
    // an overflowing segment, or a cut bin too large to keep, pushes the row's count
    // past the cap: the finish kernel then works from the row itself
    const bool over = !keep_cand || nc > (uint32_t)kSegCandCap;
    base_cand = over ? atomicAdd(&cnt[1], (uint32_t)kCandCap + 1u) : (nc ? atomicAdd(&cnt[1], nc) : 0u);
  }
  __syncthreads();
  uint64_t* win = ws.win + (int64_t)r * kMaxK;
  uint64_t* cand = ws.cand + (int64_t)r * kCandCap;
  // the selection keys, rebuilt from the (cached) row entries
  auto key_of = [&](uint32_t c) { return sel_key(order_key(row[c]), c); };
  for (uint32_t i = threadIdx.x; i < nw; i += kSegThreads)
    if (base_win + i < (uint32_t)kMaxK) win[base_win + i] = key_of(lwin[i]);
  if (keep_cand && nc <= (uint32_t)kSegCandCap)
    for (uint32_t i = threadIdx.x; i < nc; i += kSegThreads)
      if (base_cand + i < (uint32_t)kCandCap) cand[base_cand + i] = key_of(lcand[i]);
}

__global__ __launch_bounds__(kFinishThreads) void topk_finish_kernel(TopkCall a, LongWs ws) {
  constexpr int NT = kFinishThreads;
  __shared__ uint64_t sel[kMaxK];
  __shared__ __align__(16) uint64_t cand[kCandCap];  // then the sort's bucket counts and keys
  __shared__ RadixShared sh;
  __shared__ uint32_t rh[256];  // the radix select's digit counts
  __shared__ SortShared ss;
  __shared__ uint32_t count;
  const int r = blockIdx.x;
  const int64_t n = row_len(a, r);
  const uint32_t n_win = min(ws.counts[2 * (int64_t)r], (uint32_t)kMaxK);
  const uint32_t n_cand = ws.counts[2 * (int64_t)r + 1];
  int cnt;
  if (n_cand <= (uint32_t)kCandCap) {
    const uint64_t* gw = ws.win + (int64_t)r * kMaxK;
    const uint64_t* gc = ws.cand + (int64_t)r * kCandCap;
    for (uint32_t i = threadIdx.x; i < n_win; i += NT) sel[i] = gw[i];
    for (uint32_t i = threadIdx.x; i < n_cand; i += NT) cand[i] = gc[i];
    if (threadIdx.x == 0) count = n_win;
    __syncthreads();
    // every present entry is a winner or a candidate, so the winners still missing are
    // min(k, total) - n_win and they all come from the candidates, which share the bits
    // of the cut bin
    const uint32_t need = min((uint32_t)a.k - n_win, n_cand);
    auto get = [&](int64_t i) -> uint64_t { return cand[i]; };
    if (need > 0) {
      const uint64_t pre = cand[0];
      const uint64_t thr = need == n_cand ? 1ull : radix_threshold<NT>(get, n_cand, need, sh, rh, pre, kKeyBinShift);
      gather_at_least<NT, uint64_t>(get, get, n_cand, thr, sel, &count, (uint32_t)kMaxK);
    }
    cnt = (int)(n_win + need);
  } else {
    // the cut bin did not fit the lists: select from the row itself
    const float* row = a.logits + (int64_t)r * a.ld;
    auto get = [&](int64_t i) -> uint64_t {
      const uint32_t v = order_key(row[i]);
      return v ? sel_key(v, i) : 0ull;
    };
    const uint32_t total = count_present<NT>(get, n, sh);
    const uint32_t keff = min((uint32_t)a.k, total);
    const uint64_t thr = keff == 0 ? ~0ull : (keff == total ? 1ull : radix_threshold<NT>(get, n, keff, sh, rh));
    if (threadIdx.x == 0) count = 0;
    __syncthreads();
    gather_at_least<NT, uint64_t>(get, get, n, thr, sel, &count, (uint32_t)kMaxK);
    cnt = (int)keff;
  }
  __syncthreads();
  auto key = [&](int i) -> uint64_t { return sel[i]; };
  if (a.sorted)
    bucket_sort_write<NT>(a, r, key, cnt, (uint32_t*)cand, cand + kBuckets / 2, ss);
  else
    write_list<NT>(a, r, key, cnt);
}

// ------------------------------------------------------------------ one-pass selection: finish kernel

struct SelFinishArgs {
  const int64_t* acc;
  const uint4* seg;
  const uint64_t* surv;
  int64_t blocks;
};

// One workgroup per row, after the scan.
__global__ __launch_bounds__(kFinishThreads) void select_finish_kernel(TopkCall a, SelFinishArgs f) {
  __shared__ FinishLds<kFinishThreads> L;
  const int r = blockIdx.x;
  const uint64_t total = (uint64_t)f.acc[a.rows];
  const uint64_t s0 = (uint64_t)f.acc[r], s1 = (uint64_t)f.acc[r + 1];
  if (s1 <= s0) {
    write_list<kFinishThreads>(a, r, [](int) { return 0ull; }, 0);
    return;
  }
  finish_survivors<kFinishThreads>(a, r, total, s0, s1, (uint64_t)f.blocks, f.seg, f.surv, L);
}

hipError_t launch_select_finish(const TopkCall& t, const SelectState& s, int64_t blocks, hipStream_t stream) {
  if (t.rows <= 0) return hipSuccess;
  SelFinishArgs f{s.acc, s.seg, s.surv, blocks};
  hipLaunchKernelGGL(select_finish_kernel, dim3((unsigned)t.rows), dim3(kFinishThreads), 0, stream, t, f);
  return hipGetLastError();
}

// ------------------------------------------------------------------ host side

static int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

size_t topk_workspace_bytes(int rows, int64_t n_cols) {
  if (rows <= 0 || n_cols <= kShortRow) return 0;
  const int64_t R = rows;
  return (size_t)(round_up(R * kHistBins * 4, 256) + round_up(R * 2 * 4, 256) + R * kMaxK * 8 +
                  R * kCandCap * 8);
}

size_t topk_zeroed_bytes(int rows, int64_t n_cols) {
  if (rows <= 0 || n_cols <= kShortRow || (n_cols <= kWideRow && rows <= device_cu_count())) return 0;
  const int64_t R = rows;
  return (size_t)(round_up(R * kHistBins * 4, 256) + round_up(R * 2 * 4, 256));
}

// NT = kShortThreads for rows up to kShortRow, kWideThreads up to kWideRow (the row's
// value keys in LDS: up to 128 KiB, one workgroup per CU).
template <bool V4, int NT>
static hipError_t launch_short(const TopkCall& c, hipStream_t stream) {
  constexpr int kMaxRow = NT == kWideThreads ? kWideRow : kShortRow;
  static PerDeviceOnce once;
  const hipError_t attr = once.run([] {
    return hipFuncSetAttribute((const void*)topk_short_kernel<V4, NT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               kMaxRow * (int)sizeof(uint32_t));
  });
  if (attr != hipSuccess) return attr;
  const size_t lds = (size_t)std::max<int64_t>(round_up(c.n_cols, 4) * 4, kMaxK * 8);
  hipLaunchKernelGGL((topk_short_kernel<V4, NT>), dim3((unsigned)c.rows), dim3(NT), lds, stream, c);
  return hipGetLastError();
}

template <bool V4>
static void launch_long(const TopkCall& c, const LongWs& ws, int64_t seg, int64_t segs, hipStream_t stream) {
  dim3 grid((unsigned)(segs * c.rows));
  hipLaunchKernelGGL(topk_hist_kernel<V4>, grid, dim3(kSegThreads), 0, stream, c, ws, seg, (int)segs);
  hipLaunchKernelGGL(topk_filter_kernel<V4>, grid, dim3(kSegThreads), 0, stream, c, ws, seg, (int)segs);
}

// Rows of up to kLinRow entries take the one-pass bucket kernel: 1024 threads per row
// when the rows fit the compute units at once, else 512 (four workgroups per CU); rows
// up to kWideRow entries too when they fit the compute units (1024 threads, 16 or 32
// entries each).
constexpr int kLinRow = 8192;

template <bool V4>
static void launch_lin(const TopkCall& c, hipStream_t stream) {
  if (c.rows > device_cu_count())
    hipLaunchKernelGGL((topk_lin_kernel<V4, 512, kLinRow / 512>), dim3((unsigned)c.rows), dim3(512), 0, stream, c);
  else if (c.n_cols <= kLinRow)
    hipLaunchKernelGGL((topk_lin_kernel<V4, 1024, kLinRow / 1024>), dim3((unsigned)c.rows), dim3(1024), 0, stream, c);
  else if (c.n_cols <= 2 * kLinRow)
    hipLaunchKernelGGL((topk_lin_kernel<V4, 1024, 2 * kLinRow / 1024>), dim3((unsigned)c.rows), dim3(1024), 0, stream,
                       c);
  else
    hipLaunchKernelGGL((topk_lin_kernel<V4, 1024, kWideRow / 1024>), dim3((unsigned)c.rows), dim3(1024), 0, stream, c);
}

const char* topk_path(int rows, int64_t n_cols) {
  if (n_cols <= kLinRow && rows > device_cu_count())
    return "short rows, one pass (one 512-thread workgroup per row, linear buckets)";
  if (n_cols <= kWideRow && rows <= device_cu_count())
    return "rows within the compute units, one pass (one 1024-thread workgroup per row, linear buckets)";
  if (n_cols <= kShortRow) return "short rows (one workgroup per row, row in LDS)";
  return "long rows (histogram, filter, finish over row segments)";
}

hipError_t launch_topk(const TopkCall& c, void* workspace, hipStream_t stream) {
  if (c.rows <= 0) return hipSuccess;
  // rows start on 16-byte boundaries: whole groups of four are read with one load
  const bool v4 = ((uintptr_t)c.logits % 16 == 0) && (c.ld % 4 == 0);
  // no more rows than compute units, up to kWideRow columns: one 1024-thread workgroup
  // per row, all rows at once (for longer rows this beats the long-row path's four
  // kernels, whose workspace, sized for it, goes unused)
  if (c.n_cols <= kLinRow || (c.n_cols <= kWideRow && c.rows <= device_cu_count())) {
    if (v4)
      launch_lin<true>(c, stream);
    else
      launch_lin<false>(c, stream);
    return hipGetLastError();
  }
  if (c.n_cols <= kShortRow)
    return v4 ? launch_short<true, kShortThreads>(c, stream) : launch_short<false, kShortThreads>(c, stream);
  const int64_t R = c.rows;
  uint8_t* p = (uint8_t*)workspace;
  LongWs ws;
  ws.hist = (uint32_t*)p;
  p += round_up(R * kHistBins * 4, 256);
  ws.counts = (uint32_t*)p;
  p += round_up(R * 2 * 4, 256);
  ws.win = (uint64_t*)p;
  p += R * kMaxK * 8;
  ws.cand = (uint64_t*)p;
  // histogram and counters start at zero (a fill kernel, not a memset node), unless the
  // score kernel before this call cleared them
  const int64_t nz = (int64_t)topk_zeroed_bytes(c.rows, c.n_cols) / 4;
  if (!c.ws_zeroed)
    hipLaunchKernelGGL(topk_zero_kernel, dim3((unsigned)std::min<int64_t>((nz + kSegThreads - 1) / kSegThreads, 1024)),
                       dim3(kSegThreads), 0, stream, (uint32_t*)workspace, nz);
  // about four segment workgroups per compute unit over all rows; segments are whole
  // passes of the segment loop
  const int cus = device_cu_count();
  int64_t segs = (4 * (int64_t)cus + R - 1) / R;
  const int64_t seg = round_up((c.n_cols + segs - 1) / segs, kSegStep);
  segs = (c.n_cols + seg - 1) / seg;
  if (v4)
    launch_long<true>(c, ws, seg, segs, stream);
  else
    launch_long<false>(c, ws, seg, segs, stream);
  hipLaunchKernelGGL(topk_finish_kernel, dim3((unsigned)R), dim3(kFinishThreads), 0, stream, c, ws);
  return hipGetLastError();
}

}  // namespace dsaidx
