// Exact top-k per row (the fine-grained token selection of the DeepSeek-V3.2
// architecture section), one workgroup per row.
//
// Every entry gets a 64-bit selection key: the order-preserving image of its
// fp32 score in the high word and the bitwise complement of its column in the
// low word, so "larger key" means "higher score, then lower column" and no two
// entries tie. The k-th largest key is found by MSB-first radix select with
// 8-bit digits (an LDS histogram per pass; the passes over the column word run
// only when score ties straddle the cut). One more pass compacts the k winners
// into LDS through an LDS counter, and a bitonic sort puts them in selection
// order.
#include "device.h"
#include "launch.h"

namespace dsaidx {

constexpr int kTopkThreads = 1024;
constexpr int kMaxK = 2048;

__device__ __forceinline__ uint64_t sel_key(uint32_t vkey, int64_t col) {
  return ((uint64_t)vkey << 32) | (uint32_t)(~(uint32_t)col);
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkCall a) {
  __shared__ uint32_t hist[256];
  __shared__ uint64_t sel[kMaxK];
  __shared__ uint64_t s_prefix;
  __shared__ uint32_t s_krem, s_keff, s_stop, s_count;

  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const float* row = a.logits + (int64_t)r * a.ld;
  int64_t n = a.n_cols;
  if (a.lens) {
    n = min(n, (int64_t)max(a.lens[r], 0));
  } else if (a.len_ke) {
    n = min(n, (int64_t)max(a.len_ke[r] - a.len_ks[r], 0));
  }

  // ---- radix select of the k-th largest selection key
  uint64_t prefix = 0, mask = 0;
  uint32_t krem = (uint32_t)a.k;
  uint32_t keff = (uint32_t)a.k;
  bool take_all = false;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0;
    if (tid == 0) s_stop = 0;
    __syncthreads();
    for (int64_t i = tid; i < n; i += kTopkThreads) {
      const uint32_t vk = order_key(row[i]);
      if (vk == 0) continue;
      const uint64_t key = sel_key(vk, i);
      if ((key & mask) == prefix) atomicAdd(&hist[(uint32_t)(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      // lane L owns bins 255-4L .. 252-4L (highest digits first)
      uint32_t c[4], tot = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hist[255 - 4 * tid - j];
        tot += c[j];
      }
      const uint32_t incl = wave_inclusive_sum(tot);
      const uint32_t excl = incl - tot;
      const uint32_t total = __shfl(incl, kWave - 1, kWave);
      if (pass == 0 && total <= krem) {
        if (tid == 0) {
          s_keff = total;
          s_krem = 0;
          s_prefix = 0;
          s_stop = 2;
        }
      } else if (excl < krem && krem <= incl) {
        uint32_t cum = excl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (cum + c[j] >= krem) {
            const uint64_t d = (uint64_t)(255 - 4 * tid - j);
            s_prefix = prefix | (d << shift);
            s_krem = krem - cum;
            // the whole bin is needed: every key >= its lowest value is selected
            if (c[j] == krem - cum) s_stop = 1;
            break;
          }
          cum += c[j];
        }
        if (pass == 0) s_keff = krem;
      }
    }
    __syncthreads();
    const uint32_t stop = s_stop;
    prefix = s_prefix;
    krem = s_krem;
    if (pass == 0) keff = s_keff;
    mask |= (uint64_t)255u << shift;
    if (stop == 2) take_all = true;
    __syncthreads();  // every thread has read this pass's decision before the next resets it
    if (stop) break;
  }
  // threshold: select every key >= thr (exactly keff keys)
  const uint64_t thr = take_all ? 1ull : prefix;

  // ---- compaction of the winners into LDS
  if (tid == 0) s_count = 0;
  __syncthreads();
  for (int64_t i = tid; i < n; i += kTopkThreads) {
    const uint32_t vk = order_key(row[i]);
    if (vk == 0) continue;
    const uint64_t key = sel_key(vk, i);
    if (key >= thr) {
      const uint32_t slot = atomicAdd(&s_count, 1u);
      if (slot < (uint32_t)kMaxK) sel[slot] = key;
    }
  }
  __syncthreads();
  const int cnt = (int)min(min(s_count, keff), (uint32_t)kMaxK);

  // ---- bitonic sort (descending) of the winners
  int P = 1;
  while (P < cnt) P <<= 1;
  if (a.sorted && cnt > 1) {
    for (int i = cnt + tid; i < P; i += kTopkThreads) sel[i] = 0ull;
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int t = tid; t < (P >> 1); t += kTopkThreads) {
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

  // ---- output
  int32_t* oi = a.out_idx + (int64_t)r * a.out_ld;
  float* ov = a.out_val ? a.out_val + (int64_t)r * a.out_ld : nullptr;
  const int32_t* cand_row = a.cand ? a.cand + (int64_t)r * a.cand_ld : nullptr;
  for (int i = tid; i < a.k; i += kTopkThreads) {
    int32_t idx = -1;
    float val = -__builtin_inff();
    if (i < cnt) {
      const uint64_t key = sel[i];
      const int64_t col = (int64_t)(uint32_t)(~(uint32_t)key);
      val = key_value((uint32_t)(key >> 32));
      idx = (int32_t)col;
      if (cand_row) idx = (int32_t)((int64_t)cand_row[col / a.block] * a.block + col % a.block);
    }
    oi[i] = idx;
    if (ov) ov[i] = val;
  }
}

hipError_t launch_topk(const TopkCall& c, hipStream_t stream) {
  if (c.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)c.rows), dim3(kTopkThreads), 0, stream, c);
  return hipGetLastError();
}

}  // namespace dsaidx
