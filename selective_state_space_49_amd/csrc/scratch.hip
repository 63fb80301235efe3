// scratch.hip -- device scratch for the prefill entry point that allocates nothing.
//
// ssm_scan_fwd_noalloc keeps the prefill's chunk summaries (the per-chunk decay and end
// state, and after the carry scan the state entering each chunk) in this file-scope
// array instead of a caller workspace. Every GPU the library runs on holds its own copy
// of SSM_NOALLOC_SCRATCH_BYTES bytes from the first use of the library's code on that
// GPU until the process ends.
//
// In host code the name `scratch` is only a stand-in for the device variable, not a
// device address: it is never passed to a kernel or a copy. Its address on a device is
// taken once per device with hipGetSymbolAddress, with that device current, and cached;
// every later use goes through the cached pointer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ssm_internal.h"
#include "ssm_scan.h"

static __device__ __align__(256) unsigned char scratch[SSM_NOALLOC_SCRATCH_BYTES];

namespace ssm {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once known

}  // namespace

hipError_t scratch_buffer(void **ptr, size_t *bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    *bytes = SSM_NOALLOC_SCRATCH_BYTES;
    return hipSuccess;
}

}  // namespace ssm
