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

#include <algorithm>
#include <mutex>

namespace dsaidx {

constexpr int kMaxK = 2048;
constexpr int kShortRow = kTopkShortRow;  // rows up to this width take the one-kernel path
constexpr int kWideRow = 32768;        // and up to this width too when there are at most as
                                       // many rows as compute units (1024 threads per row)
constexpr int kHistBits = 12;          // bins of the value histogram
constexpr int kHistBins = 1 << kHistBits;
constexpr int kBinShift = 32 - kHistBits;  // bin of a 32-bit value key
constexpr int kKeyBinShift = 64 - kHistBits;  // bin of a 64-bit selection key
constexpr int kCandCap = 8192;         // long rows: candidates kept per row in the workspace
constexpr int kShortCandCap = 2 * kHistBins - 512;  // short rows: candidate columns (u16) over the histogram
constexpr int kSegThreads = 256;
constexpr int kFinishThreads = 1024;
constexpr int kShortThreads = 512;
constexpr int kWideThreads = 1024;

__device__ __forceinline__ uint64_t sel_key(uint32_t vkey, int64_t col) {
  return ((uint64_t)vkey << 32) | (uint32_t)(~(uint32_t)col);
}

__device__ __forceinline__ int64_t key_col(uint64_t key) { return (int64_t)(uint32_t)(~(uint32_t)key); }

__device__ __forceinline__ int64_t row_len(const TopkCall& a, int r) {
  int64_t n = a.n_cols;
  if (a.lens) {
    n = min(n, (int64_t)max(a.lens[r], 0));
  } else if (a.len_ke) {
    n = min(n, (int64_t)max(a.len_ke[r] - a.len_ks[r], 0));
  }
  return n;
}

// Appends item[j] for every take[j] of every lane (U entries per lane) to an LDS list
// with one LDS atomic per wave; entries past cap are dropped (callers size the lists
// or detect the overflow from the count). Every lane of the wave must call it.
template <int U, class T>
__device__ __forceinline__ void wave_append(const bool (&take)[U], const T (&item)[U], T* list, uint32_t* count,
                                            uint32_t cap) {
  uint64_t m[U];
  uint32_t tot = 0;
#pragma unroll
  for (int j = 0; j < U; ++j) {
    m[j] = __ballot(take[j]);
    tot += (uint32_t)__popcll(m[j]);
  }
  if (tot == 0) return;
  uint32_t base = 0;
  if (lane_id() == 0) base = atomicAdd(count, tot);
  base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
#pragma unroll
  for (int j = 0; j < U; ++j) {
    if (take[j]) {
      const uint32_t slot = base + lanes_below(m[j]);
      if (slot < cap) list[slot] = item[j];
    }
    base += (uint32_t)__popcll(m[j]);
  }
}

// Appends item[j] for every take[j] (U per lane) to an LDS list: each lane counts its
// own entries, one wave prefix sum and one LDS atomic per wave place them, and each lane
// writes its entries in order. Cheaper than wave_append when a lane holds many entries
// and few are taken. Every lane of the wave must call it.
template <int U, class T>
__device__ __forceinline__ void lane_append(const bool (&take)[U], const T (&item)[U], T* list, uint32_t* count,
                                            uint32_t cap) {
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < U; ++j) mine += take[j] ? 1u : 0u;
  const uint32_t incl = wave_inclusive_sum(mine);
  const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
  if (tot == 0) return;
  uint32_t base = 0;
  if (lane_id() == 0) base = atomicAdd(count, tot);
  base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
  uint32_t slot = base + incl - mine;
#pragma unroll
  for (int j = 0; j < U; ++j) {
    if (take[j]) {
      if (slot < cap) list[slot] = item[j];
      ++slot;
    }
  }
}

// ------------------------------------------------------------------ radix select

struct RadixShared {
  uint64_t prefix;
  uint32_t krem, stop, total;
};

// Block-wide: among the non-zero keys get(i), i < n, whose bits at and above `top`
// equal those of `prefix`, the smallest key T such that exactly `want` of them are
// >= T. Keys are unique; needs 1 <= want <= the number of such keys. Every thread of
// the block must call it.
template <int NT, class Get>
__device__ uint64_t radix_threshold(const Get& get, int64_t n, uint32_t want, RadixShared& sh, uint32_t* rh,
                                    uint64_t prefix = 0,
                                    int top = 64) {
  const int tid = threadIdx.x;
  uint64_t mask = top >= 64 ? 0ull : ~0ull << top;
  prefix &= mask;
  uint32_t krem = want;
  while (top > 0) {
    const int shift = top > 8 ? top - 8 : 0;  // the last digit may overlap fixed bits
    for (int i = tid; i < 256; i += NT) rh[i] = 0;
    if (tid == 0) sh.stop = 0;
    __syncthreads();
    for (int64_t i = tid; i < n; i += NT) {
      const uint64_t key = get(i);
      if (key != 0 && (key & mask) == prefix) atomicAdd(&rh[(uint32_t)(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      uint32_t c[4], tot = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = rh[255 - 4 * tid - j];
        tot += c[j];
      }
      const uint32_t incl = wave_inclusive_sum(tot);
      const uint32_t excl = incl - tot;
      if (excl < krem && krem <= incl) {
        uint32_t cum = excl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (cum + c[j] >= krem) {
            sh.prefix = prefix | ((uint64_t)(255 - 4 * tid - j) << shift);
            sh.krem = krem - cum;
            if (c[j] == krem - cum) sh.stop = 1;  // the whole bin is needed
            break;
          }
          cum += c[j];
        }
      }
    }
    __syncthreads();
    prefix = sh.prefix;
    krem = sh.krem;
    const uint32_t stop = sh.stop;
    mask = ~0ull << shift;
    top = shift;
    __syncthreads();  // all threads have read the decision before the next pass resets it
    if (stop) break;
  }
  return prefix;
}

// Block-wide count of non-zero keys.
template <int NT, class Get>
__device__ uint32_t count_present(const Get& get, int64_t n, RadixShared& sh) {
  if (threadIdx.x == 0) sh.total = 0;
  __syncthreads();
  uint32_t c = 0;
  for (int64_t i = threadIdx.x; i < n; i += NT) c += get(i) != 0;
  c = wave_inclusive_sum(c);
  if (lane_id() == kWave - 1 && c) atomicAdd(&sh.total, c);
  __syncthreads();
  const uint32_t t = sh.total;
  __syncthreads();
  return t;
}

// Block-wide: appends item(i) to list (LDS, at *count) for every i < n whose key get(i)
// is non-zero and >= thr.
template <int NT, class T, class Get, class Item>
__device__ void gather_at_least(const Get& get, const Item& item, int64_t n, uint64_t thr, T* list, uint32_t* count,
                                uint32_t cap) {
  for (int64_t b = 0; b < n; b += NT) {
    const int64_t i = b + threadIdx.x;
    const uint64_t key = i < n ? get(i) : 0ull;
    const bool take[1] = {key != 0 && key >= thr};
    const T it[1] = {take[0] ? item(i) : T(0)};
    wave_append<1>(take, it, list, count, cap);
  }
  __syncthreads();
}

// ------------------------------------------------------------------ cut bin

struct CutInfo {
  int bin;          // bin of the k-th largest entry; -1: at most k entries, all selected
  uint32_t above;   // entries in higher bins
  uint32_t count;   // entries in the cut bin
  uint32_t total;   // present entries
  uint32_t sums[16];
};

// Block-wide, over a kHistBins-bin histogram h (LDS or global memory).
template <int NT>
__device__ void find_cut(const uint32_t* h, int k, CutInfo& ci) {
  constexpr int per = kHistBins / NT;
  constexpr int waves = NT / kWave;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  // thread t owns bins kHistBins-1-per*t down to kHistBins-per*(t+1), highest first;
  // they stay in registers for the search below (one round of loads, not one per step)
  uint32_t hb[per];
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < per; ++j) {
    hb[j] = h[kHistBins - 1 - per * tid - j];
    c += hb[j];
  }
  uint32_t incl = wave_inclusive_sum(c);
  if (lane_id() == kWave - 1) ci.sums[wave] = incl;
  __syncthreads();
  uint32_t off = 0, total = 0;
#pragma unroll
  for (int w = 0; w < waves; ++w) {
    const uint32_t s = ci.sums[w];
    off += w < wave ? s : 0u;
    total += s;
  }
  incl += off;
  const uint32_t excl = incl - c;
  if (tid == 0) {
    ci.total = total;
    if (total <= (uint32_t)k) {
      ci.bin = -1;
      ci.above = total;
      ci.count = 0;
    }
  }
  if (total > (uint32_t)k && excl < (uint32_t)k && (uint32_t)k <= incl) {
    uint32_t cum = excl;
    bool found = false;
#pragma unroll
    for (int j = 0; j < per; ++j) {
      if (!found && cum + hb[j] >= (uint32_t)k) {
        ci.bin = kHistBins - 1 - per * tid - j;
        ci.above = cum;
        ci.count = hb[j];
        found = true;
      }
      cum += hb[j];
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------------ sorting

// x from lane (lane ^ (1 << lb)), lb = 0..5, through DPP / permlane moves (no LDS).
// The swaps return, for both operands equal to x, the even (first) and odd (second)
// 16-lane rows or 32-lane halves duplicated, so the partner's value is the one of the
// other parity.
__device__ __forceinline__ uint32_t xor_lane(uint32_t x, int lb) {
  switch (lb) {
    case 0:  // quad_perm [1,0,3,2]
      return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);
    case 1:  // quad_perm [2,3,0,1]
      return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);
    case 2: {  // row_half_mirror (l ^ 7), then quad_perm [3,2,1,0] (l ^ 3)
      const int y = __builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false);
      return (uint32_t)__builtin_amdgcn_mov_dpp(y, 0x1B, 0xF, 0xF, false);
    }
    case 3: {  // row_mirror (l ^ 15), then row_half_mirror (l ^ 7)
      const int y = __builtin_amdgcn_mov_dpp((int)x, 0x140, 0xF, 0xF, false);
      return (uint32_t)__builtin_amdgcn_mov_dpp(y, 0x141, 0xF, 0xF, false);
    }
    case 4: {
      const auto s = __builtin_amdgcn_permlane16_swap(x, x, false, false);
      return (lane_id() & 16) ? s[0] : s[1];
    }
    default: {
      const auto s = __builtin_amdgcn_permlane32_swap(x, x, false, false);
      return (lane_id() & 32) ? s[0] : s[1];
    }
  }
}

__device__ __forceinline__ uint64_t xor_lane64(uint64_t x, int lb) {
  const uint32_t lo = xor_lane((uint32_t)x, lb), hi = xor_lane((uint32_t)(x >> 32), lb);
  return ((uint64_t)hi << 32) | lo;
}

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

// Block-wide descending bitonic sort of the NT * E keys x[e] of element tid * E + e.
// xch: LDS exchange buffer of NT * E keys (used only when NT > kWave); the first use
// is preceded by a barrier, so it may alias LDS the block was reading before the call.
template <int NT, int E>
__device__ void sort_desc(uint64_t (&x)[E], uint64_t* xch) {
  constexpr int LE = ilog2(E);
  constexpr int LP = ilog2(NT * E);
  const int tid = threadIdx.x;
#pragma unroll
  for (int m = 1; m <= LP; ++m) {  // merges of 2^m elements
#pragma unroll
    for (int b = m - 1; b >= 0; --b) {  // compare elements 2^b apart
      if (b < LE) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if (e & (1 << b)) continue;
          const int f = e | (1 << b);
          const bool desc = m < LE ? !((e >> m) & 1) : !((tid >> (m - LE)) & 1);
          const uint64_t hi = x[e] > x[f] ? x[e] : x[f];
          const uint64_t lo = x[e] > x[f] ? x[f] : x[e];
          x[e] = desc ? hi : lo;
          x[f] = desc ? lo : hi;
        }
      } else {
        const int tb = b - LE;  // the stride as a thread-index bit
        const bool take_max = (((tid >> tb) & 1) != 0) != !((tid >> (m - LE)) & 1);
        uint64_t y[E];
        if (tb < 6) {
#pragma unroll
          for (int e = 0; e < E; ++e) y[e] = xor_lane64(x[e], tb);
        } else {
          __syncthreads();
#pragma unroll
          for (int e = 0; e < E; ++e) xch[tid * E + e] = x[e];
          __syncthreads();
#pragma unroll
          for (int e = 0; e < E; ++e) y[e] = xch[(tid ^ (1 << tb)) * E + e];
        }
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = (x[e] > y[e]) == take_max ? x[e] : y[e];
      }
    }
  }
}

// ------------------------------------------------------------------ output

__device__ __forceinline__ int32_t out_index(const TopkCall& a, const int32_t* cand_row, int64_t col) {
  if (!cand_row) return (int32_t)col;
  return (int32_t)((int64_t)cand_row[col / a.block] * a.block + col % a.block);
}

// Block-wide: positions tid * E + e of row r from sorted keys (key 0: padding), and
// -1 / -inf for the positions past NT * E.
template <int NT, int E>
__device__ void write_sorted(const TopkCall& a, int r, const uint64_t (&x)[E]) {
  int32_t* oi = a.out_idx + (int64_t)r * a.out_ld;
  float* ov = a.out_val ? a.out_val + (int64_t)r * a.out_ld : nullptr;
  const int32_t* cand_row = a.cand ? a.cand + (int64_t)r * a.cand_ld : nullptr;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = threadIdx.x * E + e;
    if (i < a.k) {
      int32_t idx = -1;
      float val = -__builtin_inff();
      if (x[e]) {
        idx = out_index(a, cand_row, key_col(x[e]));
        val = key_value((uint32_t)(x[e] >> 32));
      }
      oi[i] = idx;
      if (ov) ov[i] = val;
    }
  }
  for (int i = NT * E + threadIdx.x; i < a.k; i += NT) {
    oi[i] = -1;
    if (ov) ov[i] = -__builtin_inff();
  }
}

// Block-wide: row r from the selection key(i), i < cnt, in list order (k slots, -1 / -inf
// padding).
template <int NT, class Key>
__device__ void write_list(const TopkCall& a, int r, const Key& key, int cnt) {
  int32_t* oi = a.out_idx + (int64_t)r * a.out_ld;
  float* ov = a.out_val ? a.out_val + (int64_t)r * a.out_ld : nullptr;
  const int32_t* cand_row = a.cand ? a.cand + (int64_t)r * a.cand_ld : nullptr;
  for (int i = threadIdx.x; i < a.k; i += NT) {
    int32_t idx = -1;
    float val = -__builtin_inff();
    if (i < cnt) {
      const uint64_t kk = key(i);
      idx = out_index(a, cand_row, key_col(kk));
      val = key_value((uint32_t)(kk >> 32));
    }
    oi[i] = idx;
    if (ov) ov[i] = val;
  }
}

template <int NT, int E, class Key>
__device__ void sort_write_e(const TopkCall& a, int r, const Key& key, int cnt, uint64_t* xch) {
  uint64_t x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = threadIdx.x * E + e;
    x[e] = i < cnt ? key(i) : 0ull;
  }
  sort_desc<NT, E>(x, xch);
  write_sorted<NT, E>(a, r, x);
}

// Block-wide: sorts the cnt (<= CAP) keys key(i) and writes the first k of them to row
// r; xch holds CAP keys.
template <int NT, class Key, int CAP = kMaxK>
__device__ void sort_and_write(const TopkCall& a, int r, const Key& key, int cnt, uint64_t* xch) {
  static_assert(NT * 4 >= CAP, "sort_and_write: at most four keys per thread");
  if (cnt <= NT) {
    sort_write_e<NT, 1>(a, r, key, cnt, xch);
  } else if constexpr (NT * 2 >= CAP) {
    sort_write_e<NT, 2>(a, r, key, cnt, xch);
  } else {
    if (cnt <= 2 * NT)
      sort_write_e<NT, 2>(a, r, key, cnt, xch);
    else
      sort_write_e<NT, 4>(a, r, key, cnt, xch);
  }
}

// Entries one bucket of the bucket sort may hold; a row with a fuller bucket (many
// equal or tightly clustered scores) is bitonic-sorted instead.
constexpr int kBucketCap = 64;
constexpr int kBuckets = kHistBins;

struct SortShared {
  unsigned long long kmax, kmin;
  uint32_t big;
  uint32_t sums[16];
};

// Block-wide: sorts the cnt (<= CAP) keys key(i) and writes the first k of them to row r
// in selection order. The keys are spread over kBuckets buckets linear in the score
// between the smallest and the largest key's score (a monotone map, so the buckets are in
// order); an entry's position is the number of entries in higher buckets plus the number
// of larger keys in its own bucket. counts: kBuckets words of LDS, 16-byte aligned; tmp:
// CAP keys of LDS. Neither may overlap what key(i) reads.
template <int NT, class Key, int CAP = kMaxK>
__device__ void bucket_sort_write(const TopkCall& a, int r, const Key& key, int cnt, uint32_t* counts, uint64_t* tmp,
                                  SortShared& ss) {
  constexpr int E = CAP / NT;
  constexpr int per = kBuckets / NT;
  constexpr int waves = NT / kWave;
  const int tid = threadIdx.x;
  if (cnt > 0) {
    uint64_t x[E];
    uint64_t mx = 0, mn = ~0ull;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = e * NT + tid;
      x[e] = i < cnt ? key(i) : 0ull;
      if (x[e]) {
        mx = max(mx, x[e]);
        mn = min(mn, x[e]);
      }
    }
#pragma unroll
    for (int lb = 0; lb < 6; ++lb) {
      mx = max(mx, xor_lane64(mx, lb));
      mn = min(mn, xor_lane64(mn, lb));
    }
    if (tid == 0) {
      ss.kmax = 0;
      ss.kmin = ~0ull;
      ss.big = 0;
    }
    __syncthreads();
    for (int i = tid; i < kBuckets; i += NT) counts[i] = 0;
    if (lane_id() == 0) {
      atomicMax(&ss.kmax, (unsigned long long)mx);
      atomicMin(&ss.kmin, (unsigned long long)mn);
    }
    __syncthreads();
    // bucket of a score: (v - lo) * scale, clamped; NaN (only 0 * inf) goes to 0
    const float lo = key_value((uint32_t)(ss.kmin >> 32));
    const float d = key_value((uint32_t)(ss.kmax >> 32)) - lo;
    const float scale = (d > 0.f && d <= 3.0e38f) ? (float)(kBuckets - 0.01) / d : 0.f;
    int ib[E];
    uint32_t slot[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      ib[e] = -1;
      if (x[e]) {
        const float f = (key_value((uint32_t)(x[e] >> 32)) - lo) * scale;
        const int b = f >= 1.f ? min((int)f, kBuckets - 1) : 0;
        ib[e] = kBuckets - 1 - b;  // highest bucket first
        slot[e] = atomicAdd(&counts[ib[e]], 1u);
        if (slot[e] >= (uint32_t)kBucketCap) ss.big = 1;
      }
    }
    __syncthreads();
    // exclusive scan of the bucket counts, in place (a row with a full bucket leaves
    // after the scan's first barrier: the scan only touches counts, which the bitonic
    // path does not read)
    static_assert(per % 4 == 0, "bucket counts are read four at a time");
    uint32_t c[per], sum = 0;
#pragma unroll
    for (int j = 0; j < per; j += 4) {
      const uint4 q = ((const uint4*)counts)[per / 4 * tid + j / 4];
      c[j] = q.x;
      c[j + 1] = q.y;
      c[j + 2] = q.z;
      c[j + 3] = q.w;
    }
#pragma unroll
    for (int j = 0; j < per; ++j) sum += c[j];
    uint32_t incl = wave_inclusive_sum(sum);
    if (lane_id() == kWave - 1) ss.sums[tid / kWave] = incl;
    __syncthreads();
    if (ss.big) {
      sort_and_write<NT, Key, CAP>(a, r, key, cnt, tmp);
      return;
    }
    uint32_t off = incl - sum;
#pragma unroll
    for (int w = 0; w < waves; ++w) off += w < tid / kWave ? ss.sums[w] : 0u;
#pragma unroll
    for (int j = 0; j < per; j += 4) {
      uint4 q;
      q.x = off;
      q.y = q.x + c[j];
      q.z = q.y + c[j + 1];
      q.w = q.z + c[j + 2];
      off = q.w + c[j + 3];
      ((uint4*)counts)[per / 4 * tid + j / 4] = q;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (ib[e] >= 0) tmp[counts[ib[e]] + slot[e]] = x[e];
    __syncthreads();
    // rank inside the bucket; the loads of all E entries are issued together
    uint32_t st[E], len[E], pos[E], most = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      st[e] = ib[e] >= 0 ? counts[ib[e]] : 0u;
      const uint32_t end = ib[e] < 0 ? 0u : (ib[e] == kBuckets - 1 ? (uint32_t)cnt : counts[ib[e] + 1]);
      len[e] = ib[e] >= 0 ? end - st[e] : 0u;
      pos[e] = st[e];
      most = max(most, len[e]);
    }
    for (uint32_t j = 0; j < most; j += 4) {
      uint64_t v[E][4];
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int q = 0; q < 4; ++q) v[e][q] = tmp[st[e] + min(j + q, len[e] ? len[e] - 1 : 0u)];
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int q = 0; q < 4; ++q) pos[e] += (j + q < len[e]) & (v[e][q] > x[e]);
    }
    // each key straight to its position of the row (the row's 8 KiB are written whole
    // by the block, so the scattered 4-byte stores combine in the cache), and the
    // padding past cnt
    int32_t* oi = a.out_idx + (int64_t)r * a.out_ld;
    float* ov = a.out_val ? a.out_val + (int64_t)r * a.out_ld : nullptr;
    const int32_t* cand_row = a.cand ? a.cand + (int64_t)r * a.cand_ld : nullptr;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (ib[e] >= 0 && pos[e] < (uint32_t)a.k) {
        oi[pos[e]] = out_index(a, cand_row, key_col(x[e]));
        if (ov) ov[pos[e]] = key_value((uint32_t)(x[e] >> 32));
      }
    for (int i = cnt + tid; i < a.k; i += NT) {
      oi[i] = -1;
      if (ov) ov[i] = -__builtin_inff();
    }
    return;
  }
  write_list<NT>(a, r, [&](int i) { return 0ull; }, 0);
}

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
  if (a.sorted)
    bucket_sort_write<NT>(a, r, key, (int)keff, u.hist, (uint64_t*)dyn, ss);
  else
    write_list<NT>(a, r, key, (int)keff);
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

// ------------------------------------------------------------------ one-pass selection: finish
//
// The scan's select mode leaves, for every segment (the part of a row one scan workgroup
// scored), the segment's survivors as selection keys at surv[first step * 64 ...] and
// their count at seg_info[first step]. The segments of row r are found again from the
// balanced split: workgroups w_lo..w_hi cover the row's steps [acc[r], acc[r + 1]),
// workgroup w holding steps [total w / W, total (w + 1) / W). One workgroup per row
// gathers the survivors, selects the k largest keys exactly and writes the row.

struct SelFinishArgs {
  const int64_t* acc;
  const uint32_t* seg_info;
  const uint64_t* surv;
  int64_t waves;
};

// Survivors up to this count are sorted whole (the first k written) instead of selected.
constexpr int kFinishSortCap = 4096;

__global__ __launch_bounds__(kFinishThreads) void select_finish_kernel(TopkCall a, SelFinishArgs f) {
  constexpr int NT = kFinishThreads;
  constexpr int PER = kSelMaxBlocks / NT;
  static_assert(kSelMaxBlocks % NT == 0, "segments per thread");
  static_assert(kMaxK * 2 >= kBuckets && 2 * kFinishSortCap <= kCandCap, "sort scratch in sel and cand");
  __shared__ __align__(16) uint64_t sel[kMaxK];  // the selected keys, or the sort's bucket counts
  __shared__ __align__(16) uint64_t cand[kCandCap];  // survivors, then the sort's scratch
  __shared__ uint32_t soff[kSelMaxBlocks + 1];          // survivors before each segment
  __shared__ RadixShared sh;
  __shared__ uint32_t rh[256];
  __shared__ SortShared ss;
  __shared__ uint32_t count;
  __shared__ uint32_t wsum[NT / kWave];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int r = blockIdx.x;
  const uint64_t total = (uint64_t)f.acc[a.rows];
  const uint64_t s0 = (uint64_t)f.acc[r], s1 = (uint64_t)f.acc[r + 1];
  if (s1 <= s0) {
    write_list<NT>(a, r, [](int) { return 0ull; }, 0);
    return;
  }
  const uint64_t W = (uint64_t)f.waves;
  const int64_t w_lo = (int64_t)(((s0 + 1) * W - 1) / total);
  const int64_t w_hi = (int64_t)((s1 * W - 1) / total);  // the wave of step s1 - 1
  const int nseg = (int)min(w_hi - w_lo + 1, (int64_t)kSelMaxBlocks);
  auto seg_lo = [&](int i) -> uint64_t { return max(total * (uint64_t)(w_lo + i) / W, s0); };
  auto seg_hi = [&](int i) -> uint64_t { return min(total * (uint64_t)(w_lo + i + 1) / W, s1); };

  // survivors of each segment (workgroups without steps have none) and their exclusive prefix
  uint32_t c[PER], t = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid * PER + j;
    c[j] = 0;
    if (i < nseg) {
      const uint64_t lo = seg_lo(i);
      if (lo < seg_hi(i)) c[j] = f.seg_info[lo] & 0x7FFFFFFFu;
    }
    t += c[j];
  }
  const uint32_t incl = wave_inclusive_sum(t);
  if (lane == kWave - 1) wsum[tid / kWave] = incl;
  __syncthreads();
  uint32_t off = incl - t, S = 0;
#pragma unroll
  for (int wv = 0; wv < NT / kWave; ++wv) {
    const uint32_t v = wsum[wv];
    off += wv < tid / kWave ? v : 0u;
    S += v;
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    soff[tid * PER + j] = off;
    off += c[j];
  }
  if (tid == 0) {
    soff[kSelMaxBlocks] = S;
    count = 0;
  }
  __syncthreads();

  // survivor i of the row: entry i - soff[j] of the segment j with soff[j] <= i < soff[j + 1]
  auto surv_at = [&](int64_t i) -> uint64_t {
    int lo = 0, hi = nseg;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (soff[mid] <= (uint32_t)i) lo = mid;
      else hi = mid;
    }
    return f.surv[seg_lo(lo) * kTileTokens + (i - soff[lo])];
  };
  int cnt;
  if (a.sorted && S <= (uint32_t)kFinishSortCap) {
    // few enough to sort them all and keep the first k: no selection pass
    constexpr int kPer = kFinishSortCap / NT;
    uint64_t v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t i = (uint32_t)(j * NT + tid);
      v[j] = i < S ? surv_at(i) : 0ull;
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t i = (uint32_t)(j * NT + tid);
      if (i < S) cand[i] = v[j];
    }
    __syncthreads();
    auto keyc = [&](int i) -> uint64_t { return cand[i]; };
    bucket_sort_write<NT, decltype(keyc), kFinishSortCap>(a, r, keyc, (int)S, (uint32_t*)sel, cand + kFinishSortCap,
                                                          ss);
    return;
  }
  if (S <= (uint32_t)kCandCap) {
    // into LDS, all threads at once (the loads of a thread are independent)
    constexpr int kPer = kCandCap / NT;
    uint64_t v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t i = (uint32_t)(j * NT + tid);
      v[j] = i < S ? surv_at(i) : 0ull;
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t i = (uint32_t)(j * NT + tid);
      if (i < S) cand[i] = v[j];
    }
    __syncthreads();
    if (S <= (uint32_t)a.k) {
      for (uint32_t i = tid; i < S; i += NT) sel[i] = cand[i];
      cnt = (int)S;
    } else {
      auto get = [&](int64_t i) -> uint64_t { return cand[i]; };
      const uint64_t thr = radix_threshold<NT>(get, S, (uint32_t)a.k, sh, rh);
      gather_at_least<NT, uint64_t>(get, get, S, thr, sel, &count, (uint32_t)kMaxK);
      cnt = a.k;
    }
  } else {
    // more survivors than LDS holds (e.g. many equal scores): select from the regions
    auto get = [&](int64_t i) -> uint64_t { return surv_at(i); };
    const uint64_t thr = radix_threshold<NT>(get, S, (uint32_t)a.k, sh, rh);
    gather_at_least<NT, uint64_t>(get, get, S, thr, sel, &count, (uint32_t)kMaxK);
    cnt = a.k;
  }
  __syncthreads();
  auto key = [&](int i) -> uint64_t { return sel[i]; };
  if (a.sorted)
    bucket_sort_write<NT>(a, r, key, cnt, (uint32_t*)cand, cand + kBuckets / 2, ss);
  else
    write_list<NT>(a, r, key, cnt);
}

hipError_t launch_select_finish(const TopkCall& t, const SelectState& s, int64_t blocks, hipStream_t stream) {
  if (t.rows <= 0) return hipSuccess;
  SelFinishArgs f{s.acc, s.seg_info, s.surv, blocks};
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
  if (rows <= 0 || n_cols <= kShortRow) return 0;
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

const char* topk_path(int rows, int64_t n_cols) {
  if (n_cols <= kShortRow) return "short rows (one workgroup per row, row in LDS)";
  if (n_cols <= kWideRow && rows <= device_cu_count()) return "wide rows (one workgroup per row, row in LDS)";
  return "long rows (histogram, filter, finish over row segments)";
}

hipError_t launch_topk(const TopkCall& c, void* workspace, hipStream_t stream) {
  if (c.rows <= 0) return hipSuccess;
  // rows start on 16-byte boundaries: whole groups of four are read with one load
  const bool v4 = ((uintptr_t)c.logits % 16 == 0) && (c.ld % 4 == 0);
  if (c.n_cols <= kShortRow)
    return v4 ? launch_short<true, kShortThreads>(c, stream) : launch_short<false, kShortThreads>(c, stream);
  // a few rows of up to kWideRow: one pass over each row, all rows at once, beats the
  // long-row path's four kernels (its workspace, sized for the long path, goes unused)
  if (c.n_cols <= kWideRow && c.rows <= device_cu_count())
    return v4 ? launch_short<true, kWideThreads>(c, stream) : launch_short<false, kWideThreads>(c, stream);
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
