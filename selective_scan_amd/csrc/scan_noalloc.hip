// Fixed device scratch for ssm_scan_fwd_noalloc: the scan's carry workspace in a
// file-scope device array instead of caller-provided memory, for callers that
// cannot allocate. Each GPU the library runs on holds its own copy of the array
// (kNoallocScratchBytes) from module load until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its device
// address is looked up once per device with hipGetSymbolAddress (with that device
// current) and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "extras.h"

namespace ssm {

namespace {
__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(int device, void** out) {
    *out = nullptr;
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ptr[device] == nullptr) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != device) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        g_ptr[device] = p;
    }
    *out = g_ptr[device];
    return hipSuccess;
}

}  // namespace ssm
