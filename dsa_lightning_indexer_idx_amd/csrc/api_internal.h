// C-ABI layer internals shared by the entry points' source files.
#pragma once

#include <hip/hip_runtime.h>

#include "dsaidx.h"

namespace dsaidx {

// Records the calling thread's last error message; returns s.
idx_status api_fail(idx_status s, const char* fmt, ...);

// idx_select on the given workspace; fn names the entry point in error messages.
idx_status select_call(const char* fn, const idx_problem* p, int k, int32_t* out_idx, float* out_val,
                       int64_t out_ld, uint32_t flags, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

}  // namespace dsaidx
