// Device-side helpers shared by the gfx950 kernels: vector types, 64-lane wavefront
// reductions, and the per-head lambda prologue.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "params.hpp"

namespace da {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// fp32 values of the low / high bf16 halves of a 32-bit word (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

// lambda = exp(<lq1, lk1>) - exp(<lq2, lk2>) + lambda_init for head (or pair) `idx`
// (ai-engineering.academy "Atención Diferencial (V2)", section "La idea diferencial": one
// learnable scalar per head built from four vectors).  Every lane of the calling wavefront
// returns the same value.  `lane` is the caller's lane index (0..63).
__device__ __forceinline__ float head_lambda(const LambdaArgs& L, int idx, int lane) {
  if (L.override_ != nullptr) return L.override_[idx];
  const int64_t base = (int64_t)idx * L.dl;
  float a = 0.f, b = 0.f;
  for (int e = lane; e < L.dl; e += 64) {
    a = fmaf(L.lq1[base + e], L.lk1[base + e], a);
    b = fmaf(L.lq2[base + e], L.lk2[base + e], b);
  }
  a = wave_sum(a);
  b = wave_sum(b);
  return expf(a) - expf(b) + L.lam_init;
}

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// 16-byte load marked non-temporal: for data streamed once (a decode step's KV cache), so that it
// does not displace reused lines from the caches
__device__ __forceinline__ u32x4 load16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Workgroup order over (head, item) for a grid of x = heads, y = items per head.  Blocks are
// dealt to the 8 XCDs round-robin by linear index; the heads go in chunks of head_chunk (a
// multiple of 8, or all of them; the last chunk may be short), and within a chunk the items go
// in order with the heads running fastest, so that every item of one head lands on the same XCD
// (the head's tiles are shared through one L2) and the tiles that the running workgroups stream
// at once stay within the heads of one chunk.  Callers number the items heaviest first.
__device__ __forceinline__ void chunked_block(int head_chunk, int n_items, int& head, int& item) {
  const int64_t lin = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  const int64_t csz = (int64_t)head_chunk * n_items;
  const int chunk = (int)(lin / csz);
  const int cn = min(head_chunk, (int)gridDim.x - chunk * head_chunk);
  const int j = (int)(lin - chunk * csz);
  item = j / cn;
  head = chunk * head_chunk + j % cn;
}

}  // namespace da
