// Device helpers shared by the fused attention kernels (forward and backward): swizzled LDS tile
// layouts, the transposing LDS read, buffer resources, LDS DMA, and weight packing for MFMA
// operands.  All of it is layout plumbing; none of it is the method's arithmetic.
#pragma once
#include "device_common.hpp"

namespace da {
namespace tile {

constexpr int kDV = 128;  // value width of the tiles (V rows, O rows)
constexpr int kRsrcWord3 = 0x00020000;  // buffer resource flags word for gfx9-family targets

typedef __attribute__((address_space(3))) void lds_void;


// XOR swizzle of 16-byte chunk indices in a dense K tile row (64 banks of 4 bytes).
template <int DQK>
__device__ __forceinline__ int k_swz(int row) {
  return DQK == 64 ? ((row >> 1) & 7) : (row & 15);
}
// Element offset of (row, col) in a dense K tile.
template <int DQK>
__device__ __forceinline__ int k_off(int row, int col) {
  return row * DQK + ((((col >> 3) ^ k_swz<DQK>(row))) << 3) + (col & 7);
}
// Element offset of (row, col) in a dense V tile (128 channels) with 32-byte chunks swizzled.
__device__ __forceinline__ int v_off(int row, int col) {
  return row * kDV + ((((col >> 4) ^ (2 * (row & 3)))) << 4) + (col & 15);
}

// sum of x over the lane pair (l, l ^ 32).  (A v_permlane32_swap formulation was tried: the
// compiler treated both of its results as one value, so lane exchanges go through ds_bpermute.)
__device__ __forceinline__ float pair_sum(float x) { return x + __shfl_xor(x, 32); }

// Round 8 consecutive weights of s to a packed MFMA operand and add the rounded values to l
// (v_dot2 of each packed pair against (1, 1)).  Each pair is converted and summed on its own.
__device__ __forceinline__ bf16x8 cvt8_sum(const f32x16& s, int base, float& l) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(bf16)1.f, (bf16)1.f};
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 h = {(bf16)s[base + 2 * i], (bf16)s[base + 2 * i + 1]};
    l = __builtin_amdgcn_fdot2_f32_bf16(h, one, l, false);
    w[i] = __builtin_bit_cast(uint32_t, h);
  }
  return __builtin_bit_cast(bf16x8, w);
}
__device__ __forceinline__ f16x8 cvt8h_sum(const f32x16& s, int base, float& l) {
  const f16x2 one = {(_Float16)1.f, (_Float16)1.f};
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 h = {(_Float16)s[base + 2 * i], (_Float16)s[base + 2 * i + 1]};
    l = __builtin_amdgcn_fdot2(h, one, l, false);
    w[i] = __builtin_bit_cast(uint32_t, h);
  }
  return __builtin_bit_cast(f16x8, w);
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  f16x2 h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// Transposing LDS read (see file header): returns 4 consecutive-row elements of one column.
__device__ __forceinline__ u32x2 lds_read_tr(const bf16* p) {
  const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// One wavefront-wide 16-byte-per-lane DMA from a buffer into LDS (lane i lands at lds + 16 i).
// Issued from inline asm so that the compiler does not treat it as aliasing every later LDS read
// (it would otherwise wait for all outstanding DMA before each one, defeating the prefetch); the
// kernels order these writes themselves with explicit vmcnt waits and barriers.  M0 holds the LDS
// base (declared clobbered, so the compiler keeps nothing of its own there across the asm); one
// wait state separates the M0 write from the DMA.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, bf16* lds, uint32_t voff) {
  const uint32_t m0v = (uint32_t)(uintptr_t)(lds_void*)lds;
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(m0v), "v"(voff), "s"(r)
      : "memory", "m0");
}

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}


}  // namespace tile
}  // namespace da
