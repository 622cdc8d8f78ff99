// Streaming-read probe: reads a device buffer once with wide non-temporal loads and
// discards the data. It is the measuring stick for the scan's HBM fraction (what this
// machine actually delivers to a plain read), not part of the indexer path.
#include "device.h"
#include "launch.h"

#include <algorithm>

namespace dsaidx {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const v4i* __restrict__ p, int64_t n, uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  v4i acc = {0, 0, 0, 0};
  for (; i + (kProbeUnroll - 1) * stride < n; i += kProbeUnroll * stride) {
    v4i v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  for (; i < n; i += stride) acc ^= p[i];
  // never true for the probe's buffers in practice; keeps the loads
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x7A5A5A5A) sink[0] = 1u;
}

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>(32 * (int64_t)device_cu_count(), (n + kProbeThreads - 1) / kProbeThreads);
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, stream, (const v4i*)buf, n,
                     sink);
  return hipGetLastError();
}

}  // namespace dsaidx
