// Host-side declarations of the library's entry points that are not one of the
// scan's own kernel pipelines: the fixed scratch of the allocation-free scan
// entry point and the benchmark's diagnostic kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "ssm_scan.h"

namespace ssm {

// ssm_scan_fwd_noalloc: the workspace lives in a fixed device array of this many
// bytes per GPU (scan_noalloc.hip); *out = its device address on `device`.
constexpr size_t kNoallocScratchBytes = SSM_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(int device, void** out);

// diagnostics (diag.hip)
hipError_t launch_valu_rate(int mode, int blocks, int iters, float* out, hipStream_t st);
hipError_t launch_stream_scale(float* p, size_t n, float s, hipStream_t st);
hipError_t launch_copy(const float* src, float* dst, size_t n, hipStream_t st);

}  // namespace ssm
