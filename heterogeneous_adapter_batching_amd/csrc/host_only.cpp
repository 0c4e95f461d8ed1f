// Kernel launchers for a build of the host library without device code: each
// reports hipErrorInvalidValue.  Such a build (host_sanitized() in build.py)
// exercises the pool, plan, validation and exchange bookkeeping under the
// address and undefined-behaviour sanitizers on a machine without a GPU; no
// call that launches a kernel can succeed in it.
#include "sgmv_internal.h"

namespace lora {
hipError_t launch_shrink(int, int, bool, const ShrinkArgs &, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_pack_a(int, const void *, int, int, void *, int, int, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_pack_b(int, const void *, int, int, void *, int, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_reduce(int, const ReduceArgs &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_prefill(int, int, int, int, int, const PrefillArgs &, int, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_expand_decode(int, int, const ExpandArgs &, int, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_expand_merge(int, int, int, const MergeArgs &, int, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t static_scratch(void **, uint64_t *) { return hipErrorInvalidValue; }
bool debug_build() { return false; }
hipError_t debug_errors(uint32_t *, bool) { return hipErrorInvalidValue; }
}  // namespace lora
