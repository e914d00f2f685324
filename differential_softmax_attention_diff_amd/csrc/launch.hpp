// Host-side launchers, one per kernel family (defined in the .hip translation units).
#pragma once
#include <hip/hip_runtime.h>

#include "params.hpp"

namespace da {

hipError_t launch_v1_f32(const PrefillParams& p, hipStream_t stream);
hipError_t launch_v1_bf16(const PrefillParams& p, hipStream_t stream);
hipError_t launch_bwd_v1(const BwdParams& p, hipStream_t stream);
hipError_t launch_v2_bf16(const PrefillParams& p, hipStream_t stream);
hipError_t launch_decode_v2(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_v2_paged(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_v1(const DecodeV1Params& p, hipStream_t stream);

}  // namespace da
