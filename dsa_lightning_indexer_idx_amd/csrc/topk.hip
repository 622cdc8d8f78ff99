// Exact top-k per row (the fine-grained token selection of the DeepSeek-V3.2
// architecture section).
//
// Selection key. Every entry gets a 64-bit key: the order-preserving image of its
// fp32 score in the high word and the bitwise complement of its column in the low
// word, so "larger key" means "higher score, then lower column" and no two entries
// tie. The k winners are exactly the keys >= the k-th largest key T, found by
// MSB-first radix select with 8-bit digits (LDS histograms); the passes over the
// column word run only when score ties straddle the cut. The winners are then
// bitonic-sorted into selection order.
//
// Short rows (n_cols <= kShortRow) take one workgroup per row with the row's value
// keys cached in LDS, so the row is read from memory once.
//
// Long rows use the whole chip. The cutoff is estimated from the scores themselves
// (the sampled-filtering idea of the persistent top-k on the pages, here with an
// exact histogram instead of a sample, so the estimate is never wrong):
//   1. hist:   segments of every row build 12-bit histograms of their value keys
//              in LDS and add the non-empty bins into the row's histogram;
//   2. filter: every segment reads the row histogram, finds the bin holding the
//              k-th largest value, and streams out the entries above that bin
//              (certain winners) and the entries in it (candidates), with one
//              atomic per wave for each list;
//   3. finish: one workgroup per row loads the candidates into LDS, radix-selects
//              the missing winners among them, sorts and writes the row. If the
//              cut bin held more candidates than the workspace keeps (e.g. a row
//              of equal scores) the row is selected from memory instead.
#include "device.h"
#include "launch.h"

#include <algorithm>
#include <mutex>

namespace dsaidx {

constexpr int kMaxK = 2048;
constexpr int kShortRow = 16384;       // rows up to this width take the one-kernel path
constexpr int kHistBits = 12;          // bins of the long-row histogram
constexpr int kHistBins = 1 << kHistBits;
constexpr int kCandCap = 8192;         // candidates kept per row in the workspace
constexpr int kSegThreads = 256;
constexpr int kFinishThreads = 1024;
constexpr int kShortThreads = 512;

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

struct RadixShared {
  uint32_t hist[256];
  uint64_t prefix;
  uint32_t krem, stop, total;
};

// Block-wide: the smallest threshold T such that exactly ``want`` of the (unique,
// non-zero) keys produced by get(i), i < n, are >= T. Needs 1 <= want <= number of
// non-zero keys. Every thread of the block must call it.
template <int NT, class Get>
__device__ uint64_t radix_threshold(const Get& get, int64_t n, uint32_t want, RadixShared& sh) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0, mask = 0;
  uint32_t krem = want;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    for (int i = tid; i < 256; i += NT) sh.hist[i] = 0;
    if (tid == 0) sh.stop = 0;
    __syncthreads();
    for (int64_t i = tid; i < n; i += NT) {
      const uint64_t key = get(i);
      if (key != 0 && (key & mask) == prefix) atomicAdd(&sh.hist[(uint32_t)(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      uint32_t c[4], tot = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = sh.hist[255 - 4 * tid - j];
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
    mask |= (uint64_t)255u << shift;
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

// Block-wide descending bitonic sort of sel[0, cnt) (cnt <= kMaxK).
template <int NT>
__device__ void sort_desc(uint64_t* sel, int cnt) {
  int P = 1;
  while (P < cnt) P <<= 1;
  if (cnt <= 1) return;
  for (int i = cnt + threadIdx.x; i < P; i += NT) sel[i] = 0ull;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < (P >> 1); t += NT) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint64_t x = sel[lo], y = sel[hi];
        if ((x < y) == desc) {
          sel[lo] = y;
          sel[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

// Block-wide: write row r's output from sel[0, cnt) (k slots, -1 / -inf padding).
template <int NT>
__device__ void write_row(const TopkCall& a, int r, const uint64_t* sel, int cnt) {
  int32_t* oi = a.out_idx + (int64_t)r * a.out_ld;
  float* ov = a.out_val ? a.out_val + (int64_t)r * a.out_ld : nullptr;
  const int32_t* cand_row = a.cand ? a.cand + (int64_t)r * a.cand_ld : nullptr;
  for (int i = threadIdx.x; i < a.k; i += NT) {
    int32_t idx = -1;
    float val = -__builtin_inff();
    if (i < cnt) {
      const uint64_t key = sel[i];
      const int64_t col = key_col(key);
      val = key_value((uint32_t)(key >> 32));
      idx = (int32_t)col;
      if (cand_row) idx = (int32_t)((int64_t)cand_row[col / a.block] * a.block + col % a.block);
    }
    oi[i] = idx;
    if (ov) ov[i] = val;
  }
}

// Block-wide: append every key >= thr produced by get(i), i < n, to sel starting at
// *count (an LDS counter).
template <int NT, class Get>
__device__ void gather_at_least(const Get& get, int64_t n, uint64_t thr, uint64_t* sel, uint32_t* count) {
  for (int64_t i = threadIdx.x; i < n; i += NT) {
    const uint64_t key = get(i);
    if (key != 0 && key >= thr) {
      const uint32_t slot = atomicAdd(count, 1u);
      if (slot < (uint32_t)kMaxK) sel[slot] = key;
    }
  }
  __syncthreads();
}

// Full selection of one row read from memory (the short-row kernel without its LDS
// cache, and the long-row fallback).
template <int NT, class Get>
__device__ int select_row(const Get& get, int64_t n, int k, uint64_t* sel, RadixShared& sh, uint32_t* count) {
  const uint32_t total = count_present<NT>(get, n, sh);
  const uint32_t keff = min((uint32_t)k, total);
  const uint64_t thr = keff == 0 ? ~0ull : (keff == total ? 1ull : radix_threshold<NT>(get, n, keff, sh));
  if (threadIdx.x == 0) *count = 0;
  __syncthreads();
  gather_at_least<NT>(get, n, thr, sel, count);
  return (int)keff;
}

// ------------------------------------------------------------------ short rows

__global__ __launch_bounds__(kShortThreads) void topk_short_kernel(TopkCall a) {
  extern __shared__ uint32_t vkeys[];  // n_cols value keys
  __shared__ uint64_t sel[kMaxK];
  __shared__ RadixShared sh;
  __shared__ uint32_t count;
  const int r = blockIdx.x;
  const int64_t n = row_len(a, r);
  const float* row = a.logits + (int64_t)r * a.ld;
  for (int64_t i = threadIdx.x; i < n; i += kShortThreads) vkeys[i] = order_key(row[i]);
  __syncthreads();
  auto get = [&](int64_t i) -> uint64_t {
    const uint32_t v = vkeys[i];
    return v ? sel_key(v, i) : 0ull;
  };
  const int cnt = select_row<kShortThreads>(get, n, a.k, sel, sh, &count);
  if (a.sorted) sort_desc<kShortThreads>(sel, cnt);
  write_row<kShortThreads>(a, r, sel, cnt);
}

// ------------------------------------------------------------------ long rows

struct LongWs {
  uint32_t* hist;    // [rows, kHistBins]
  uint32_t* counts;  // [rows, 2]: certain winners, candidates
  uint64_t* win;     // [rows, kMaxK]
  uint64_t* cand;    // [rows, kCandCap]
};

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__global__ __launch_bounds__(kSegThreads) void topk_zero_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kSegThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kSegThreads)
    p[i] = 0u;
}

// Values per thread per pass of the segment loops: independent loads issued together
// so the loop is not bound by one memory latency per element.
constexpr int kUnroll = 16;

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
  for (int64_t b = s0; b < s1; b += kSegThreads * kUnroll) {
    float x[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t i = b + j * kSegThreads + threadIdx.x;
      x[j] = i < s1 ? row[i] : -__builtin_inff();
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const uint32_t v = order_key(x[j]);
      if (v) atomicAdd(&hist[v >> (32 - kHistBits)], 1u);
    }
  }
  __syncthreads();
  uint32_t* g = ws.hist + (int64_t)r * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += kSegThreads)
    if (hist[i]) atomicAdd(&g[i], hist[i]);
}

// The bin holding the k-th largest value of row r and the number of entries above it;
// bin -1 means "take every entry".
__device__ void find_cut(const uint32_t* ghist, int k, int* s_bin, uint32_t* s_above, uint32_t* sums) {
  constexpr int per = kHistBins / kSegThreads;
  const int tid = threadIdx.x;
  // thread t owns bins from the top: kHistBins-1-per*t .. kHistBins-per*(t+1)
  uint32_t c = 0;
  for (int j = 0; j < per; ++j) c += ghist[kHistBins - 1 - per * tid - j];
  // block inclusive scan in thread order (highest bins first)
  uint32_t incl = wave_inclusive_sum(c);
  const int wave = tid / kWave;
  if (lane_id() == kWave - 1) sums[wave] = incl;
  __syncthreads();
  uint32_t off = 0;
  for (int w = 0; w < wave; ++w) off += sums[w];
  incl += off;
  const uint32_t excl = incl - c;
  uint32_t total = 0;
  for (int w = 0; w < kSegThreads / kWave; ++w) total += sums[w];
  if (tid == 0 && total <= (uint32_t)k) {
    *s_bin = -1;
    *s_above = 0;
  }
  if (total > (uint32_t)k && excl < (uint32_t)k && (uint32_t)k <= incl) {
    uint32_t cum = excl;
    for (int j = 0; j < per; ++j) {
      const int b = kHistBins - 1 - per * tid - j;
      const uint32_t h = ghist[b];
      if (cum + h >= (uint32_t)k) {
        *s_bin = b;
        *s_above = cum;
        break;
      }
      cum += h;
    }
  }
  __syncthreads();
}

// Candidates one filter workgroup stages in LDS; a segment with more forces its row
// onto the full-row fallback (the candidate count is pushed past kCandCap).
constexpr int kSegCandCap = 4096;

// Appends key to an LDS list through one LDS atomic per wave; returns nothing, drops
// entries past cap (the caller detects the overflow from the final count).
__device__ __forceinline__ void wave_append(bool take, uint64_t key, uint64_t* list, uint32_t* count,
                                            uint32_t cap) {
  const uint64_t m = __ballot(take);
  if (!m) return;
  const int leader = __builtin_ctzll(m);
  uint32_t base = 0;
  if (lane_id() == leader) base = atomicAdd(count, (uint32_t)__popcll(m));
  base = __shfl(base, leader, kWave);
  if (take) {
    const uint32_t slot = base + lanes_below(m);
    if (slot < cap) list[slot] = key;
  }
}

__global__ __launch_bounds__(kSegThreads) void topk_filter_kernel(TopkCall a, LongWs ws, int64_t seg, int segs) {
  __shared__ uint32_t sums[kSegThreads / kWave];
  __shared__ int s_bin;
  __shared__ uint32_t s_above;
  __shared__ uint64_t lwin[kMaxK];
  __shared__ uint64_t lcand[kSegCandCap];
  __shared__ uint32_t n_lwin, n_lcand, base_win, base_cand;
  const int r = (int)(blockIdx.x / (unsigned)segs);
  const int64_t n = row_len(a, r);
  const int64_t s0 = (int64_t)(blockIdx.x % (unsigned)segs) * seg;
  const int64_t s1 = min(s0 + seg, n);
  if (s0 >= s1) return;
  if (threadIdx.x == 0) {
    n_lwin = 0;
    n_lcand = 0;
  }
  find_cut(ws.hist + (int64_t)r * kHistBins, a.k, &s_bin, &s_above, sums);
  const int cut = s_bin;
  const float* row = a.logits + (int64_t)r * a.ld;
  // every thread runs the same number of iterations so whole waves vote together
  for (int64_t b = s0; b < s1; b += kSegThreads * kUnroll) {
    float x[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t i = b + j * kSegThreads + threadIdx.x;
      x[j] = i < s1 ? row[i] : -__builtin_inff();
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t i = b + j * kSegThreads + threadIdx.x;
      const uint32_t v = order_key(x[j]);
      const int bin = v ? (int)(v >> (32 - kHistBits)) : -2;
      const uint64_t key = sel_key(v, i);
      wave_append(v && bin > cut, key, lwin, &n_lwin, kMaxK);
      wave_append(v && bin == cut, key, lcand, &n_lcand, kSegCandCap);
    }
  }
  __syncthreads();
  uint32_t* cnt = ws.counts + 2 * (int64_t)r;
  const uint32_t nw = min(n_lwin, (uint32_t)kMaxK);
  const uint32_t nc = n_lcand;
  if (threadIdx.x == 0) {
    base_win = nw ? atomicAdd(&cnt[0], nw) : 0u;
    // an overflowing segment pushes the row's count past the cap: full-row fallback
    base_cand = nc ? atomicAdd(&cnt[1], nc > (uint32_t)kSegCandCap ? (uint32_t)kCandCap + 1u : nc) : 0u;
  }
  __syncthreads();
  uint64_t* win = ws.win + (int64_t)r * kMaxK;
  uint64_t* cand = ws.cand + (int64_t)r * kCandCap;
  for (uint32_t i = threadIdx.x; i < nw; i += kSegThreads)
    if (base_win + i < (uint32_t)kMaxK) win[base_win + i] = lwin[i];
  if (nc <= (uint32_t)kSegCandCap)
    for (uint32_t i = threadIdx.x; i < nc; i += kSegThreads)
      if (base_cand + i < (uint32_t)kCandCap) cand[base_cand + i] = lcand[i];
}

__global__ __launch_bounds__(kFinishThreads) void topk_finish_kernel(TopkCall a, LongWs ws) {
  __shared__ uint64_t sel[kMaxK];
  __shared__ uint64_t cand[kCandCap];
  __shared__ RadixShared sh;
  __shared__ uint32_t count;
  const int r = blockIdx.x;
  const int64_t n = row_len(a, r);
  const uint32_t n_win = min(ws.counts[2 * (int64_t)r], (uint32_t)kMaxK);
  const uint32_t n_cand = ws.counts[2 * (int64_t)r + 1];
  int cnt;
  if (n_cand <= (uint32_t)kCandCap) {
    const uint64_t* gw = ws.win + (int64_t)r * kMaxK;
    const uint64_t* gc = ws.cand + (int64_t)r * kCandCap;
    for (uint32_t i = threadIdx.x; i < n_win; i += kFinishThreads) sel[i] = gw[i];
    for (uint32_t i = threadIdx.x; i < n_cand; i += kFinishThreads) cand[i] = gc[i];
    if (threadIdx.x == 0) count = n_win;
    __syncthreads();
    // every present entry is a winner or a candidate, so the winners still missing are
    // min(k, total) - n_win and they all come from the candidates
    const uint32_t need = min((uint32_t)a.k - n_win, n_cand);
    auto get = [&](int64_t i) -> uint64_t { return cand[i]; };
    if (need > 0) {
      const uint64_t thr = need == n_cand ? 1ull : radix_threshold<kFinishThreads>(get, n_cand, need, sh);
      gather_at_least<kFinishThreads>(get, n_cand, thr, sel, &count);
    }
    cnt = (int)(n_win + need);
  } else {
    const float* row = a.logits + (int64_t)r * a.ld;
    auto get = [&](int64_t i) -> uint64_t {
      const uint32_t v = order_key(row[i]);
      return v ? sel_key(v, i) : 0ull;
    };
    cnt = select_row<kFinishThreads>(get, n, a.k, sel, sh, &count);
  }
  if (a.sorted) sort_desc<kFinishThreads>(sel, cnt);
  write_row<kFinishThreads>(a, r, sel, cnt);
}

// ------------------------------------------------------------------ host side

static int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

size_t topk_workspace_bytes(int rows, int64_t n_cols) {
  if (rows <= 0 || n_cols <= kShortRow) return 0;
  const int64_t R = rows;
  return (size_t)(round_up(R * kHistBins * 4, 256) + round_up(R * 2 * 4, 256) + R * kMaxK * 8 +
                  R * kCandCap * 8);
}

hipError_t launch_topk(const TopkCall& c, void* workspace, hipStream_t stream) {
  if (c.rows <= 0) return hipSuccess;
  if (c.n_cols <= kShortRow) {
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
      attr = hipFuncSetAttribute((const void*)topk_short_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 kShortRow * (int)sizeof(uint32_t));
    });
    if (attr != hipSuccess) return attr;
    const size_t lds = (size_t)(c.n_cols > 0 ? c.n_cols : 1) * sizeof(uint32_t);
    hipLaunchKernelGGL(topk_short_kernel, dim3((unsigned)c.rows), dim3(kShortThreads), lds, stream, c);
    return hipGetLastError();
  }
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
  // histogram and counters start at zero (a fill kernel, not a memset node)
  const int64_t nz = (int64_t)((uint8_t*)ws.win - (uint8_t*)workspace) / 4;
  hipLaunchKernelGGL(topk_zero_kernel, dim3((unsigned)std::min<int64_t>((nz + kSegThreads - 1) / kSegThreads, 1024)),
                     dim3(kSegThreads), 0, stream, (uint32_t*)workspace, nz);
  // about four segment workgroups per compute unit over all rows
  const int cus = device_cu_count();
  int64_t segs = (4 * (int64_t)cus + R - 1) / R;
  int64_t seg = round_up((c.n_cols + segs - 1) / segs, 1024);
  segs = (c.n_cols + seg - 1) / seg;
  dim3 grid((unsigned)(segs * R));
  hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(kSegThreads), 0, stream, c, ws, seg, (int)segs);
  hipLaunchKernelGGL(topk_filter_kernel, grid, dim3(kSegThreads), 0, stream, c, ws, seg, (int)segs);
  hipLaunchKernelGGL(topk_finish_kernel, dim3((unsigned)R), dim3(kFinishThreads), 0, stream, c, ws);
  return hipGetLastError();
}

}  // namespace dsaidx
