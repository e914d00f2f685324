// Launcher stand-ins for the sanitizer build of the ABI layer (tests only).  The host-validation
// tests never reach a launch: every invalid call returns before one.  If a call did get this far,
// these report a HIP error instead of running anything.
#include "launch.hpp"

namespace da {

hipError_t launch_v1_f32(const PrefillParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_v1_bf16(const PrefillParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_v1(const BwdParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_v2_bf16(const PrefillParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_decode_v2(const DecodeParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_decode_v2_paged(const DecodeParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_decode_v1(const DecodeV1Params&, hipStream_t) { return hipErrorNotSupported; }
void* noalloc_scratch() { return nullptr; }

}  // namespace da
