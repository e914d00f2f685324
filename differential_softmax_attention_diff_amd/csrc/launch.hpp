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

// The allocation-free decode's scratch: a fixed device array of kNoAllocScratchBytes per GPU.
// Returns its device address on the current device (looked up on first use per device), or
// nullptr if the lookup fails.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
void* noalloc_scratch();

}  // namespace da
