// Which shapes the matrix-core kernels take, and how the decode launch groups its
// waves.  Host code only: it has no device code, so the C ABI's validation can be
// built and checked on its own (the sanitizer build of the tests).
#include "kernels.h"

namespace sa {

bool mfma_decode_supported(int group) { return group >= 1 && group <= 64; }

bool mfma_prefill_supported(int group) { return group >= 1 && group <= 64; }

// One wave per KV head, or above 16 query heads per KV head one wave per slice of
// the largest power of two (at most 16) that divides the group; eight waves per
// workgroup.  decode.hip's launch picks the same slices.
int mfma_decode_head_blocks(int hq, int hkv) {
    const int group = hq / hkv;
    int slice = group;  // query heads per wave
    if (group > 16)
        slice = group % 16 == 0 ? 16 : group % 8 == 0 ? 8 : group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
    const int waves = hkv * (group / slice);
    return waves / 8 + (waves % 8 != 0);
}

bool topk_softmax_supported(int num_experts) {
    return num_experts == 8 || num_experts == 16 || num_experts == 32 || num_experts == 64 ||
           num_experts == 128 || num_experts == 256 || num_experts == 512;
}

}  // namespace sa
