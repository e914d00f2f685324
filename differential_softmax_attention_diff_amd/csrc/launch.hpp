// Host-side launchers, one per kernel family (defined in the .hip translation units).
#pragma once
#include <hip/hip_runtime.h>

#include "params.hpp"

namespace da {

// Heads per chunk of the workgroup order (see chunked_block): the heads' streamed tiles,
// bytes_per_head each, split into chunks of about a quarter of the 256 MB last-level cache (the
// nearest whole number of chunks, at least one), the chunks of equal size in multiples of 8 (one
// head per XCD); all heads if that is more than there are.
inline int head_chunk(int64_t heads, int64_t bytes_per_head) {
  constexpr int64_t kChunkBytes = int64_t(64) << 20;
  int64_t n = (heads * bytes_per_head + kChunkBytes / 2) / kChunkBytes;
  if (n < 1) n = 1;
  int64_t c = (heads + n - 1) / n;
  c = (c + 7) / 8 * 8;
  return (int)(c < heads ? c : heads);
}

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
