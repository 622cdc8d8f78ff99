// Indexer key-cache writer: new keys (128 bf16 values each) quantised into the cache
// format and stored at their slots, the step before the scan (the extra key per token
// and layer of the DeepSeek-V3.2 architecture section; the fp8 and MXFP4 cache formats
// of the vLLM sparse_indexer page). Readings of the quantisation (the pages give none):
//   * fp8: scale = amax / 448, code = e4m3fn nearest-even of value * (448 / amax), both
//     quotients and the product in float32; amax = 0 gives scale 0 and zero codes;
//   * MXFP4 (OCP MX v1.0 conversion): per group of 32, shared exponent
//     X = floor(log2(amax)) - 2 stored as UE8M0 X + 127 clamped to [0, 254]; each
//     value / 2^X to the nearest e2m1 value, ties to even, magnitudes above 6 to 6.
//
// A wave writes four keys per pass: 16 lanes per key, eight elements per lane (one
// 16-byte load). The fp8 amax is a 16-lane reduction, an MXFP4 group's a 4-lane one.
// Bandwidth-bound and tiny: 256 bytes in and 132 (fp8) or 68 (MXFP4) bytes out per key.
#include "device.h"
#include "launch.h"

#include <algorithm>

namespace dsaidx {

constexpr int kWriterThreads = 256;

struct KcacheArgs {
  const uint16_t* k_new;
  const int64_t* slots;
  int64_t n_new;
  uint8_t* cache;
  void* scale;
  int64_t n_slots;
  unsigned* err;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

// Largest value over the lanes (lane ^ m) for m = 1 .. span / 2 (span a power of two <= 32).
template <int SPAN>
__device__ __forceinline__ float max_over_lanes(float v) {
#pragma unroll
  for (int m = 1; m < SPAN; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

// e2m1 code of a finite value: the grid steps are 0.5 below 2, 1 in [2, 4) and 2 in
// [4, 6], so round-half-even of the magnitude in units of its step gives the nearest
// code with ties to the even one; magnitudes above 6 saturate.
__device__ __forceinline__ uint32_t e2m1_code(float s) {
  const float mag = fminf(fabsf(s), 6.0f);
  float c;
  if (mag < 2.0f)
    c = rintf(mag * 2.0f);
  else if (mag < 4.0f)
    c = rintf(mag) + 2.0f;
  else
    c = rintf(mag * 0.5f) + 4.0f;
  return (uint32_t)c | (__float_as_uint(s) >> 31 << 3);
}

template <int F>
__global__ __launch_bounds__(kWriterThreads) void kcache_write_kernel(KcacheArgs a) {
  const int lane = lane_id();
  const int quarter = lane >> 4, l16 = lane & 15;
  const int64_t wave = ((int64_t)blockIdx.x * kWriterThreads + threadIdx.x) / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * (kWriterThreads / kWave);
  for (int64_t base = 4 * wave; base < a.n_new; base += 4 * nwaves) {
    const int64_t t = base + quarter;
    const bool valid = t < a.n_new;
    int64_t slot = valid ? a.slots[t] : -1;
    if (slot >= a.n_slots) {
      if (l16 == 0) flag_error(a.err, kErrSlot);
      slot = -1;
    }
    uint4 raw = make_uint4(0u, 0u, 0u, 0u);
    if (valid) raw = *(const uint4*)(a.k_new + t * kDim + 8 * l16);
    const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_to_f32(wds[i] & 0xFFFFu);
      x[2 * i + 1] = bf16_to_f32(wds[i] >> 16);
    }
    float m8 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m8 = fmaxf(m8, fabsf(x[i]));
    if constexpr (F == FMT_FP8) {
      const float amax = max_over_lanes<16>(m8);
      float y[8];
      const float inv = amax > 0.f ? 448.0f / amax : 1.0f;  // amax = 0: every value is +-0
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = x[i] * inv;
      int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
      int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
      w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
      if (slot >= 0) {
        *(uint2*)(a.cache + slot * kDim + 8 * l16) = make_uint2((uint32_t)w0, (uint32_t)w1);
        if (l16 == 0) ((float*)a.scale)[slot] = amax > 0.f ? amax / 448.0f : 0.f;
      }
    } else {
      const float amax = max_over_lanes<4>(m8);  // the lane's group of 32 elements
      int biased = 0;
      if (amax > 0.f) {
        int e = 0;
        frexpf(amax, &e);  // amax = m 2^e, m in [0.5, 1)
        biased = min(max((e - 1) - 2 + 127, 0), 254);
      }
      uint32_t code = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) code |= e2m1_code(ldexpf(x[i], 127 - biased)) << (4 * i);
      if (slot >= 0) {
        *(uint32_t*)(a.cache + slot * (kDim / 2) + 4 * l16) = code;
        if ((l16 & 3) == 0) ((uint8_t*)a.scale)[slot * 4 + (l16 >> 2)] = (uint8_t)biased;
      }
    }
  }
}

hipError_t launch_kcache_write(const KcacheCall& c, hipStream_t stream) {
  if (c.n_new <= 0) return hipSuccess;
  KcacheArgs a{(const uint16_t*)c.k_new, c.slots, c.n_new, c.cache, c.scale, c.n_slots, c.err};
  const int64_t waves = (c.n_new + 3) / 4;
  const int64_t blocks = std::min<int64_t>((waves + 3) / 4, 16 * (int64_t)device_cu_count());
  if (c.fmt == FMT_FP8)
    hipLaunchKernelGGL(kcache_write_kernel<FMT_FP8>, dim3((unsigned)blocks), dim3(kWriterThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(kcache_write_kernel<FMT_MXFP4>, dim3((unsigned)blocks), dim3(kWriterThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsaidx
