// Host-only stand-ins for the sanitizer build of the C ABI (tests/test_sanitizers.py):
// the kernel launchers and the HIP runtime calls the validation code makes.  The
// runtime reports that no device is present, so every call that passes validation
// stops at the device check and nothing here is ever asked to launch.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace {
hipError_t none() { return hipErrorNoDevice; }
}  // namespace

namespace sa {
hipError_t launch_generic_prefill(bool, const void*, const void*, const void*, const float*,
                                  const int32_t*, const int32_t*, int, int, int, int, float, int,
                                  void*, float*, hipStream_t) { return none(); }
hipError_t launch_generic_prefill_split(bool, const void*, const void*, const void*, const float*,
                                        const int32_t*, const int32_t*, int, int, int, int,
                                        const StateSlots&, float, int, float*, float*, float*,
                                        hipStream_t) { return none(); }
hipError_t launch_generic_decode_split(bool, const void*, const void*, const void*, const float*,
                                       const int32_t*, int, int, int, int, int, float, float*,
                                       float*, float*, hipStream_t) { return none(); }
hipError_t launch_mfma_decode_plan(const void*, const void*, const void*, const float*,
                                   const int32_t*, int, int, int, const DecodePlan&, float, float*,
                                   float*, float*, hipStream_t) { return none(); }
hipError_t launch_mfma_decode_split(const void*, const void*, const void*, const float*,
                                    const int32_t*, int, int, int, int, int, float, float*, float*,
                                    float*, hipStream_t) { return none(); }
hipError_t launch_mfma_prefill_split(const void*, const void*, const void*, const float*,
                                     const int32_t*, const int32_t*, int, int, int, int, int,
                                     const StateSlots&, float, int, float*, float*, float*,
                                     hipStream_t) { return none(); }
hipError_t launch_mfma_prefill(const void*, const void*, const void*, const float*, const int32_t*,
                               const int32_t*, int, int, int, int, int, float, int, void*, float*,
                               hipStream_t) { return none(); }
hipError_t launch_topk_softmax(const void*, int64_t, int, int, int32_t*, void*, hipStream_t) {
    return none();
}
hipError_t launch_qkv_rope(const void*, const void*, const int32_t*, const float*, int64_t, int, int,
                           int, void*, void*, void*, hipStream_t) { return none(); }
hipError_t launch_merge(bool, const float*, const float*, const float*, const int32_t*, int, int,
                        int, int, void*, float*, hipStream_t) { return none(); }
hipError_t launch_merge_plan(bool, const float*, const float*, const float*, const int32_t*,
                             const DecodePlan&, int, int, void*, float*, hipStream_t) {
    return none();
}
hipError_t launch_read_probe(const void*, int64_t, int, uint32_t*, hipStream_t) { return none(); }
hipError_t decode_scratch(float**) { return none(); }
}  // namespace sa

extern "C" {
hipError_t hipGetDevice(int*) { return hipErrorNoDevice; }
hipError_t hipGetLastError(void) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "no device (host-only build)"; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipErrorNoDevice; }
hipError_t hipMemcpy(void*, const void*, size_t, hipMemcpyKind) { return hipErrorNoDevice; }
hipError_t hipDeviceGetAttribute(int*, hipDeviceAttribute_t, int) { return hipErrorNoDevice; }
}
