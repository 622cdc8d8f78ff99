// Device helpers shared by the dsaidx kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace dsaidx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));

constexpr int kHeads = 64;
constexpr int kDim = 128;
constexpr int kWave = 64;
constexpr int kTileTokens = 64;  // tokens one wave scores per step: four 16-token MFMA columns

// Device argument-error bits (mirrors the IDX_DEVERR_* values of the C ABI).
constexpr unsigned kErrRange = 1u;
constexpr unsigned kErrPage = 2u;
constexpr unsigned kErrBlock = 4u;
constexpr unsigned kErrSlot = 8u;
constexpr unsigned kErrOrder = 16u;

__device__ __forceinline__ void flag_error(unsigned* err, unsigned bits) {
  if (err) atomicOr(err, bits);
}

// ---------------------------------------------------------------- global -> LDS loads
//
// One 64-lane load from global memory straight into LDS: lane l's 16 (4) bytes land at
// m0 + 16 l (4 l), in lane order. Issued as inline assembly so the compiler adds no wait
// for them before later LDS reads (without alias information it would make every LDS
// read wait for all such loads in flight): the caller waits for them itself (vmcnt) and
// orders the waves with barriers, whose fence also completes earlier LDS reads of the
// target. The no-op covers the one wait state the load needs after m0 is written.
__device__ __forceinline__ void lds_load16(const void* src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void lds_load4(const void* src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}
// LDS byte address of a pointer into a __shared__ array
template <class T>
__device__ __forceinline__ uint32_t lds_addr(const T* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) T*)p;
}
// s_waitcnt operand: vmcnt(n) (6 bits, split over [3:0] and [15:14]), expcnt and lgkmcnt
// at their maxima (no wait)
constexpr int vmcnt_enc(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// ---------------------------------------------------------------- MFMA wrappers
//
// v_mfma_scale_f32_16x16x128_f8f6f4: D[16 x 16] += A[16 x 128] * B[128 x 16].
// Operand lane l holds row (A) / column (B) l % 16; with g = l / 16, an 8-bit
// operand carries K = 16g .. 16g+15 in bytes 0..15 and K = 64+16g .. 64+16g+15 in
// bytes 16..31, an fp4 operand K = 32g .. 32g+31 in 16 bytes (low nibble first).
// The accumulator lane l holds D[4 * g + i][l % 16], i = 0..3. Each lane also
// supplies the UE8M0 scale of its row or column for K-block g (127 is 2^0).
// Format codes: 0 = fp8 e4m3, 4 = fp4 e2m1. When both operands are 8-bit, any
// permutation of K applied to both gives the same product.

__device__ __forceinline__ v4f mfma_fp8_fp8(const v8i& a, const v8i& b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ v4f mfma_fp8_fp4(const v8i& a, const v8i& b, int b_scale, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, 127, 0, b_scale);
}

// v_mfma_f32_16x16x32_bf16: the same D layout; A/B lane l holds row/column l % 16
// and 8 consecutive K-elements of block l / 16.
__device__ __forceinline__ v4f mfma_bf16(const v8bf& a, const v8bf& b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ReLU as one integer max: a float with its sign bit set is a negative int, so
// max(bits, 0) keeps positive values and turns negatives and -0.0 into +0.0.
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// ---------------------------------------------------------------- cross-lane sums
//
// Lane l holds four partial sums p[j], one per 16-token tile j, each covering the
// heads of lane group l / 16. Returns, in lane l, the sum over the four lane groups
// of p[l / 16] for column l % 16, i.e. the value for token 16 * (l / 16) + l % 16 = l.
// v_permlane32_swap exchanges lanes 32..63 of its first operand with lanes 0..31 of
// its second; v_permlane16_swap does the same for odd / even 16-lane rows.
__device__ __forceinline__ float sum_lane_groups(float p0, float p1, float p2, float p3) {
  auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p2), false, false);
  auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p1), __float_as_uint(p3), false, false);
  float a = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
  float b = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
  auto sab = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(sab[0]) + __uint_as_float(sab[1]);
}

// ---------------------------------------------------------------- selection keys
//
// Order-preserving map from fp32 to uint32 for "higher value first": -0.0 is
// folded onto +0.0 so the two tie; -inf and NaN map to 0, the key of an entry that
// does not exist. Every finite value and +inf maps to a key >= 0x00800000.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0u) u = 0u;
  uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  bool absent = (x != x) || (u == 0xFF800000u);
  return absent ? 0u : k;
}

__device__ __forceinline__ float key_value(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Workgroup barrier that orders LDS accesses only: global stores issued before it need not
// have completed (__syncthreads also waits for those).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Set bits of a 64-lane mask below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Wave-wide inclusive prefix sum (lane order): a scan inside each 16-lane row with
// DPP row shifts (lanes without a source add 0), then the row totals, read from lanes
// 15, 31 and 47, added to the rows above them.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  const uint32_t t0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  const uint32_t t1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t t2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  const int row = lane_id() >> 4;
  v += (row >= 1 ? t0 : 0u) + (row >= 2 ? t1 : 0u) + (row >= 3 ? t2 : 0u);
  return v;
}

}  // namespace dsaidx
