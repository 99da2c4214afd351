// Fixed device array holding the chunk states of sink_attn_decode_noalloc, for
// callers that cannot allocate.  Each GPU the library runs on holds its own copy
// of the array until the process ends; every call on that GPU shares it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace sa {

namespace {

constexpr size_t kScratchFloats = kDecodeScratchBytes / sizeof(float);

// The array itself.  In host code its name stands for the host-side shadow, not a
// device address: host code uses only the per-device address below.
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
float* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t decode_scratch(float** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> guard(g_lock);
    if (g_ptr[dev] == nullptr) {
        // once per device, with that device current
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_ptr[dev] = static_cast<float*>(p);
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace sa
