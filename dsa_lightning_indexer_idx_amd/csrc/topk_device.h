// Device-side building blocks of the exact top-k (selection keys, radix threshold,
// compaction, sorts and row writes) and the one-pass selection's per-row finish. Selection
// key: the order-preserving image of an entry's fp32 score in
// the high word and the complement of its column in the low word, so "larger key" means
// "higher score, then lower column" and no two entries tie.
#pragma once

#include "device.h"
#include "launch.h"

namespace dsaidx {

constexpr int kMaxK = 2048;
constexpr int kShortRow = kTopkShortRow;  // rows up to this width take the one-kernel path
constexpr int kWideRow = kTopkWideRow;  // and up to this width too when there are at most as
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
  int top;          // highest bin holding an entry (-1: none)
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
    if (total == 0u) ci.top = -1;
    if (total <= (uint32_t)k) {
      ci.bin = -1;
      ci.above = total;
      ci.count = 0;
    }
  }
  if (excl == 0u && c != 0u) {  // the thread holding the highest entries
    bool found = false;
#pragma unroll
    for (int j = 0; j < per; ++j) {
      if (!found && hb[j] != 0u) {
        ci.top = kHistBins - 1 - per * tid - j;
        found = true;
      }
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

// Order-key bounds of the entries in bins lo_bin .. hi_bin (for bucket_sort_write): the
// lower edge of lo_bin (at least 1) and the upper edge of hi_bin, no higher than +inf's key.
__device__ __forceinline__ void bin_bounds(int lo_bin, int hi_bin, uint32_t& lo_key, uint32_t& hi_key) {
  lo_key = max((uint32_t)lo_bin << kBinShift, 1u);
  const uint64_t hi = (((uint64_t)hi_bin + 1) << kBinShift) - 1;
  hi_key = (uint32_t)min(hi, (uint64_t)0xFF800000u);
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
  uint32_t wmax[16], wmin[16];
  uint32_t big;
  uint32_t sums[16];
};

// Block-wide: sorts the cnt (<= CAP) keys key(i) and writes the first k of them to row r
// in selection order. The keys are spread over kBuckets buckets linear in the score
// between a lower and an upper bound (a monotone map, so the buckets are in order; keys
// outside the bounds go to the end buckets, so any bounds give the same result, close ones
// fewer keys per bucket); an entry's position is the number of entries in higher buckets
// plus the number of larger keys in its own bucket. The bounds are the order keys lo_key
// and hi_key when the caller knows them (lo_key != 0), else the smallest and largest
// key's. counts: kBuckets words of LDS, 16-byte aligned; tmp: CAP keys of LDS. Neither
// may overlap what key(i) reads.
template <int NT, class Key, int CAP = kMaxK>
__device__ void bucket_sort_write(const TopkCall& a, int r, const Key& key, int cnt, uint32_t* counts, uint64_t* tmp,
                                  SortShared& ss, uint32_t lo_key = 0, uint32_t hi_key = 0) {
  constexpr int E = CAP / NT;
  constexpr int per = kBuckets / NT;
  constexpr int waves = NT / kWave;
  const int tid = threadIdx.x;
  if (cnt > 0) {
    uint64_t x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = e * NT + tid;
      x[e] = i < cnt ? key(i) : 0ull;
    }
    for (int i = tid; i < kBuckets; i += NT) counts[i] = 0;
    if (tid == 0) ss.big = 0;
    if (lo_key == 0) {
      // the smallest and largest value key: per wave by lane swaps, then over the waves
      uint32_t mx = 0, mn = ~0u;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (x[e]) {
          mx = max(mx, (uint32_t)(x[e] >> 32));
          mn = min(mn, (uint32_t)(x[e] >> 32));
        }
      }
#pragma unroll
      for (int lb = 0; lb < 6; ++lb) {
        mx = max(mx, xor_lane(mx, lb));
        mn = min(mn, xor_lane(mn, lb));
      }
      if (lane_id() == 0) {
        ss.wmax[tid / kWave] = mx;
        ss.wmin[tid / kWave] = mn;
      }
      __syncthreads();
      lo_key = ~0u;
      hi_key = 0u;
#pragma unroll
      for (int w = 0; w < waves; ++w) {
        lo_key = min(lo_key, ss.wmin[w]);
        hi_key = max(hi_key, ss.wmax[w]);
      }
    } else {
      __syncthreads();
    }
    // bucket of a score: (v - lo) * scale, clamped; NaN (only 0 * inf) goes to 0
    const float lo = key_value(lo_key);
    const float d = key_value(hi_key) - lo;
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

// ------------------------------------------------------------------ one-pass selection: finish
//
// The select-mode scan leaves, for every segment (the part of a row one scan workgroup
// scored), the segment's survivors as selection keys at surv[first step * 64 ...] and, at
// seg[first step], their count, the cut they reach and the largest of them. The segments
// of a row are found again from the balanced split: workgroups w_lo..w_hi cover the row's
// steps [s0, s1), workgroup w holding steps [total w / W, total (w + 1) / W). One workgroup
// per row gathers the row's survivors, selects the k largest keys exactly and writes the
// row.

// Survivors up to this count are sorted whole (the first k written) instead of selected.
constexpr int kFinishSortCap = 4096;

// LDS of one row's finish by NT threads.
template <int NT>
struct alignas(16) FinishLds {
  uint64_t sel[kMaxK];               // the selected keys, or the sort's bucket counts
  uint64_t cand[kCandCap];           // the survivors, then the sort's scratch
  uint64_t sbeg[kSelMaxBlocks];      // first step of each segment
  uint32_t soff[kSelMaxBlocks + 1];  // survivors before each segment
  uint32_t rh[256];
  RadixShared sh;
  SortShared ss;
  uint32_t count;
  uint32_t wsum[NT / kWave], wlo[NT / kWave], whi[NT / kWave], wcut[NT / kWave];
  uint64_t ltmp[kMaxK + kBucketCap];  // finish_lin: the keys at or above the cut bucket
  uint32_t lcut, lfill, lbig;
};

// Block-wide: row r from the exact top k of the S (<= kCandCap) keys in L.cand, whose
// order keys lie in [lo_key, hi_key] (lo_key > 0), in one pass as the one-pass short-row
// kernel does it: counts in kBuckets buckets linear in the score, an exclusive scan from
// the highest down for each bucket's first position and the cut bucket, the keys at or
// above it to their buckets' positions, and each key's place from the larger keys of its
// bucket. false, with nothing written, when a bucket at or above the cut holds more than
// kBucketCap keys.
template <int NT>
__device__ bool finish_lin(const TopkCall& a, int r, int S, uint32_t lo_key, uint32_t hi_key, FinishLds<NT>& L) {
  constexpr int E = kCandCap / NT;
  constexpr int per = kBuckets / NT;
  static_assert(per % 4 == 0 || per == 4, "four counts per read");
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wv = tid / kWave;
  uint32_t* cnt = (uint32_t*)L.sel;  // kBuckets counts, then first positions
  uint64_t* tmp = L.ltmp;
  uint64_t x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = e * NT + tid;
    x[e] = i < S ? L.cand[i] : 0ull;
  }
  for (int i = tid; i < kBuckets / 4; i += NT) ((uint4*)cnt)[i] = make_uint4(0u, 0u, 0u, 0u);
  if (tid == 0) L.lbig = 0u;
  __syncthreads();
  const float lo = key_value(lo_key);
  const float d = key_value(hi_key) - lo;
  const float scale = (d > 0.f && d <= 3.0e38f) ? (float)(kBuckets - 0.01) / d : 0.f;
  auto bucket = [&](uint32_t k) -> uint32_t {
    const float f = (key_value(k) - lo) * scale;
    const int b = f >= 1.f ? min((int)f, kBuckets - 1) : 0;
    return (uint32_t)(kBuckets - 1 - b);
  };
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (x[e]) atomicAdd(&cnt[bucket((uint32_t)(x[e] >> 32))], 1u);
  __syncthreads();
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
  if (lane == kWave - 1) L.wsum[wv] = incl;
  __syncthreads();
  uint32_t off = incl - sum, total = 0u;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    off += w < wv ? L.wsum[w] : 0u;
    total += L.wsum[w];
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
      L.lcut = (uint32_t)per * tid + jc;
      L.lfill = fc;
    }
    if (big) L.lbig = 1u;
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
  if (L.lbig || keff == 0u) return false;
  const uint32_t cut = L.lcut, fill = L.lfill;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (!x[e]) continue;
    const uint32_t b = bucket((uint32_t)(x[e] >> 32));
    if (b <= cut) tmp[atomicAdd(&cnt[b], 1u)] = x[e];
  }
  __syncthreads();
  int32_t* oi = a.out_idx + (int64_t)r * a.out_ld;
  float* ov = a.out_val ? a.out_val + (int64_t)r * a.out_ld : nullptr;
  const int32_t* cand_row = a.cand ? a.cand + (int64_t)r * a.cand_ld : nullptr;
  for (uint32_t i = tid; i < fill; i += NT) {
    const uint64_t y = tmp[i];
    const uint32_t b = bucket((uint32_t)(y >> 32));
    const uint32_t st = b > 0 ? cnt[b - 1] : 0u;
    const uint32_t len = cnt[b] - st;
    uint32_t pos = st;
    for (uint32_t j = 0; j < len; j += 4) {
      uint64_t v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = tmp[st + min(j + q, len - 1)];
#pragma unroll
      for (int q = 0; q < 4; ++q) pos += (j + q < len) & (v[q] > y);
    }
    if (pos < keff) {
      oi[pos] = out_index(a, cand_row, key_col(y));
      if (ov) ov[pos] = key_value((uint32_t)(y >> 32));
    }
  }
  for (int i = (int)keff + tid; i < a.k; i += NT) {
    oi[i] = -1;
    if (ov) ov[i] = -__builtin_inff();
  }
  return true;
}

// Block-wide: row r from the exact top k of the S keys in L.cand (lo_key / hi_key: order
// keys at or below and at or above all of them, 0 if not known).
template <int NT>
__device__ __forceinline__ void finish_cand(const TopkCall& a, int r, int S, uint32_t lo_key, uint32_t hi_key,
                                            FinishLds<NT>& L) {
  static_assert(kMaxK * 2 >= kBuckets && 2 * kFinishSortCap <= kCandCap, "sort scratch in sel and cand");
  const int tid = threadIdx.x;
  auto keyc = [&](int64_t i) -> uint64_t { return L.cand[i]; };
  if (a.sorted && S <= kFinishSortCap) {
    // few enough to sort them all and keep the first k: no selection pass
    bucket_sort_write<NT, decltype(keyc), kFinishSortCap>(a, r, keyc, S, (uint32_t*)L.sel, L.cand + kFinishSortCap,
                                                          L.ss, lo_key, hi_key);
    return;
  }
  // more: one pass over linear buckets when the bounds are known and no bucket at or
  // above the cut is too full, else a radix threshold, then the sort of the k
  if (a.sorted && lo_key > 0u && S <= kCandCap && finish_lin<NT>(a, r, S, lo_key, hi_key, L)) return;
  if (tid == 0) L.count = 0;
  __syncthreads();
  int cnt;
  if (S <= a.k) {
    for (int i = tid; i < S; i += NT) L.sel[i] = L.cand[i];
    cnt = S;
  } else {
    const uint64_t thr = radix_threshold<NT>(keyc, S, (uint32_t)a.k, L.sh, L.rh);
    gather_at_least<NT, uint64_t>(keyc, keyc, S, thr, L.sel, &L.count, (uint32_t)kMaxK);
    cnt = a.k;
  }
  __syncthreads();
  auto key = [&](int i) -> uint64_t { return L.sel[i]; };
  if (a.sorted)
    bucket_sort_write<NT>(a, r, key, cnt, (uint32_t*)L.cand, L.cand + kBuckets / 2, L.ss);
  else
    write_list<NT>(a, r, key, cnt);
}

// Block-wide: row r (steps [s0, s1) of total, s0 < s1, over the W workgroups of the
// scan) from its segments' survivors. A segment may hold survivors below the row's cut
// (it was filtered at a lower cut of its own): those are dropped as the survivors come
// into LDS. The bounds of the final sort come from the segment records: the row's cut,
// or else the lowest cut (when every segment had one), and the largest survivor.
template <int NT>
__device__ __forceinline__ void finish_survivors(const TopkCall& a, int r, uint64_t total, uint64_t s0, uint64_t s1,
                                                 uint64_t W, const uint4* seg, const uint64_t* surv,
                                                 FinishLds<NT>& L) {
  constexpr int PER = kSelMaxBlocks / NT;
  static_assert(kSelMaxBlocks % NT == 0, "segments per thread");
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wv = tid / kWave;
  const int64_t w_lo = (int64_t)(((s0 + 1) * W - 1) / total);
  const int64_t w_hi = (int64_t)((s1 * W - 1) / total);  // the workgroup of step s1 - 1
  const int nseg = (int)min(w_hi - w_lo + 1, (int64_t)kSelMaxBlocks);

  // segment i: steps [max(total (w_lo + i) / W, s0), min(total (w_lo + i + 1) / W, s1))
  // (workgroups without steps have none); its survivors and their exclusive prefix; the
  // lowest cut (0: a segment kept every entry) and the largest survivor
  uint32_t c[PER], t = 0, lo = ~0u, hi = 0u, cut = 0u;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid * PER + j;
    c[j] = 0;
    if (i < nseg) {
      const uint64_t sl = max(total * (uint64_t)(w_lo + i) / W, s0);
      L.sbeg[i] = sl;
      if (sl < min(total * (uint64_t)(w_lo + i + 1) / W, s1)) {
        const uint4 g = seg[sl];
        c[j] = g.x & ~kSegNoCut;
        cut = max(cut, g.w);
        if (c[j]) {
          lo = min(lo, (g.x & kSegNoCut) ? 0u : g.y);
          hi = max(hi, g.z);
        }
      }
    }
    t += c[j];
  }
  const uint32_t incl = wave_inclusive_sum(t);
#pragma unroll
  for (int lb = 0; lb < 6; ++lb) {
    lo = min(lo, xor_lane(lo, lb));
    hi = max(hi, xor_lane(hi, lb));
    cut = max(cut, xor_lane(cut, lb));
  }
  if (lane == kWave - 1) L.wsum[wv] = incl;
  if (lane == 0) {
    L.wlo[wv] = lo;
    L.whi[wv] = hi;
    L.wcut[wv] = cut;
  }
  __syncthreads();
  uint32_t off = incl - t, S = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    const uint32_t v = L.wsum[w];
    off += w < wv ? v : 0u;
    S += v;
    lo = min(lo, L.wlo[w]);
    hi = max(hi, L.whi[w]);
    cut = max(cut, L.wcut[w]);
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    L.soff[tid * PER + j] = off;
    off += c[j];
  }
  if (tid == 0) L.soff[kSelMaxBlocks] = S;
  __syncthreads();

  // survivor i of the row: entry i - soff[j] of the segment j with soff[j] <= i < soff[j + 1]
  auto surv_at = [&](int64_t i) -> uint64_t {
    int lo_s = 0, hi_s = nseg;
    while (hi_s - lo_s > 1) {
      const int mid = (lo_s + hi_s) >> 1;
      if (L.soff[mid] <= (uint32_t)i) lo_s = mid;
      else hi_s = mid;
    }
    return surv[L.sbeg[lo_s] * kTileTokens + (i - L.soff[lo_s])];
  };
  if (S <= (uint32_t)kCandCap) {
    // into LDS, all threads at once (the loads of a thread are independent)
    constexpr int kPer = kCandCap / NT;
    uint64_t v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int64_t i = (int64_t)j * NT + tid;
      v[j] = i < (int64_t)S ? surv_at(i) : 0ull;
    }
    int S2 = (int)S;
    if (cut > 1u && lo < cut) {
      // those at or above the row's cut, packed in thread order
      uint32_t keep = 0;
#pragma unroll
      for (int j = 0; j < kPer; ++j) keep |= (v[j] != 0ull && (uint32_t)(v[j] >> 32) >= cut ? 1u : 0u) << j;
      const uint32_t mine = (uint32_t)__popc(keep);
      const uint32_t inc = wave_inclusive_sum(mine);
      if (lane == kWave - 1) L.wsum[wv] = inc;
      __syncthreads();
      uint32_t at = inc - mine, all = 0;
#pragma unroll
      for (int w = 0; w < NT / kWave; ++w) {
        const uint32_t n = L.wsum[w];
        at += w < wv ? n : 0u;
        all += n;
      }
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if ((keep >> j) & 1u) L.cand[at++] = v[j];
      S2 = (int)all;
      lo = cut;
    } else {
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int64_t i = (int64_t)j * NT + tid;
        if (i < (int64_t)S) L.cand[i] = v[j];
      }
    }
    __syncthreads();
    const bool bounded = lo > 1u && lo != ~0u && hi >= lo;  // a cut of 1 is no bound
    finish_cand<NT>(a, r, S2, bounded ? lo : 0u, bounded ? hi : 0u, L);
    return;
  }
  // more than LDS holds (e.g. many equal scores): select from the survivors in place
  if (tid == 0) L.count = 0;
  __syncthreads();
  const uint64_t thr = radix_threshold<NT>(surv_at, (int64_t)S, (uint32_t)a.k, L.sh, L.rh);
  gather_at_least<NT, uint64_t>(surv_at, surv_at, (int64_t)S, thr, L.sel, &L.count, (uint32_t)kMaxK);
  __syncthreads();
  auto key = [&](int i) -> uint64_t { return L.sel[i]; };
  if (a.sorted)
    bucket_sort_write<NT>(a, r, key, a.k, (uint32_t*)L.cand, L.cand + kBuckets / 2, L.ss);
  else
    write_list<NT>(a, r, key, a.k);
}

}  // namespace dsaidx
