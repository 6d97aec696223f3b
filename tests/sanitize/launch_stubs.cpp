// launch_stubs.cpp -- host-only stand-ins for the kernel launchers of
// libkda.so, for the sanitizer build of the C ABI's validation layer
// (kda_api.cpp).  Every launcher reports a failed launch, so an argument
// set that passes validation returns KDA_ERR_DEVICE and no pointer is ever
// dereferenced.  Test infrastructure only.
#include "../../gated_delta_rule_27_amd/csrc/kda_launch.h"

namespace kda {

hipError_t launch_chunk(const ChunkArgs&, int, int, int, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_decode(const DecodeArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_decode_multi(const DecodeMultiArgs&, int, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_segment_scan(const float*, const float*, const float*, int32_t, int32_t,
                               float*, float*, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_prologue(const PrologueArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_epilogue(const EpilogueArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_bwd(const BwdArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_bwd_rev(const BwdArgs&, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_bwd_grad(const BwdArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_bwd_dh_ws(const BwdArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipStream_t bwd_fork(hipStream_t) { return nullptr; }
hipError_t bwd_join(hipStream_t) { return hipErrorInvalidValue; }
hipError_t noalloc_scratch(void** ptr) {
    *ptr = nullptr;
    return hipErrorInvalidValue;
}

}  // namespace kda
