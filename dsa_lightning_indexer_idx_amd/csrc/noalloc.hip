// idx_select_noalloc: idx_select on a workspace the library holds in device memory for the
// whole process, for callers that cannot allocate (code under stream capture, serving loops,
// hosts that forbid allocation). The workspace is one file-scope device array; each device
// has its own copy, whose address is looked up once per device and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "api_internal.h"
#include "dsaidx.h"
#include "launch.h"

// The shared workspace of idx_select_noalloc. In host code this name is only a handle for
// the symbol lookup; kernels get the per-device address found below.
static __device__ __align__(256) unsigned char scratch[IDX_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_mu;
void* g_scratch[dsaidx::kMaxDevices];

// The current device's scratch address (looked up on the device's first call); null and
// an error message on failure.
void* device_scratch(const char* fn, idx_status* st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= dsaidx::kMaxDevices) {
    *st = dsaidx::api_fail(IDX_ERR_HIP, "%s: no usable current device (%s)", fn,
                           e == hipSuccess ? "device id out of range" : hipGetErrorString(e));
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *st = dsaidx::api_fail(IDX_ERR_HIP, "%s: scratch address lookup on device %d failed: %s", fn, dev,
                             hipGetErrorString(e));
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" idx_status idx_select_noalloc(const idx_problem* p, int k, int32_t* out_idx, float* out_val,
                                         int64_t out_ld, uint32_t flags, idx_stream_t stream) {
  const char* fn = "idx_select_noalloc";
  if (!p) return dsaidx::api_fail(IDX_ERR_ARG, "%s: problem is null", fn);
  const size_t need = idx_select_workspace(p, k);
  if (need > (size_t)IDX_NOALLOC_SCRATCH_BYTES)
    return dsaidx::api_fail(IDX_ERR_WORKSPACE,
                            "%s: the call needs %zu bytes of workspace, more than the %zu of the static scratch "
                            "(use idx_select with a workspace)",
                            fn, need, (size_t)IDX_NOALLOC_SCRATCH_BYTES);
  if (p->rows <= 0) return dsaidx::select_call(fn, p, k, out_idx, out_val, out_ld, flags, nullptr, 0, (hipStream_t)stream);
  idx_status st = IDX_OK;
  void* ws = device_scratch(fn, &st);
  if (!ws) return st;
  return dsaidx::select_call(fn, p, k, out_idx, out_val, out_ld, flags, ws, (size_t)IDX_NOALLOC_SCRATCH_BYTES,
                             (hipStream_t)stream);
}
