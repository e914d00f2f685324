// Fused V2 differential-attention prefill for gfx950: bf16 inputs, fp32 accumulation, bf16 out.
//
// What is computed (ai-engineering.academy "Atención Diferencial (V2)", sections "V1 vs V2: la
// diferencia" and "Ejercicios" 5): the query heads are doubled and paired, heads (2p, 2p+1) of
// pair p share KV head g = p * Hkv / P, and
//   out_p = softmax(q_2p K^T / sqrt(D)) V - lambda_p softmax(q_2p+1 K^T / sqrt(D)) V
// with no normalisation and no scale.  Neither map is written to memory.
//
// Design (one pass over K, V per block of 64 query rows of a pair):
//  * v2_values_kernel rewrites V once per call as fp16, region by region (16 keys x 64
//    channels), keeping the bf16 bits of a region that holds a value beyond the fp16 range, and
//    writes one flag byte per region.  P.V then runs on the fp16 MFMA (P and V with 11
//    significant bits instead of bf16's 8, which the unnormalised V2 output needs to meet the
//    bf16 tolerance with margin).
//  * A 256-thread workgroup owns 64 query rows of one pair; each of its four wavefronts owns 16
//    rows and runs BOTH heads of the pair on 16x16x32 MFMAs.  The two heads read the same K and
//    V, so every K operand and every V^T operand a wave reads from LDS feeds two MFMAs, and the
//    two heads' softmax chains are independent work inside the wave.  Registers: 64
//    accumulators, 32 for the two heads' Q operands, 16 for the scores: three waves per SIMD.
//  * Tiles of 32 keys stream global -> LDS through buffer loads that write LDS directly (dma16),
//    double buffered, one barrier per tile; rows past N read as zeros.  K rows XOR their 16-byte
//    chunk index with row & 15 (16 rows of a row-wise operand read hit 16 distinct chunks), V rows
//    their 32-byte chunk index with row & 7 (the 8 rows of a transposed read phase hit 8).
//  * Scores are formed transposed, S^T = K Q^T: lane (n, g) of the 16x16 accumulator holds query
//    row n and keys 16 h + 4 g + r of key half h; read as k-slot 8 g + 4 h + r that is exactly
//    the B operand P^T of O^T = V^T P^T, whose A operand takes V rows 4 g + r and 16 + 4 g + r
//    from two transposing LDS reads (ds_read_b64_tr_b16).
//  * Online softmax against a per-row reference max m, set from the exact row max of the wave's
//    first tile and moved only when a lane's weight sum for a tile exceeds 2^12 (a score jump):
//    every weight the fp16 MFMA sees is then at most 2^12.  softmax(s) does not depend on m, so the
//    result is that of an exact running max.  The row sums add the rounded weights.
//  * A tile whose V regions include a bf16 one (a value beyond the fp16 range) sends the wave to
//    a bf16 P.V loop from that tile on, where the fp16 regions are widened back to bf16 (exact
//    for every value fp16 holds with 8 or more significant bits).  The tile flags are read
//    through the scalar cache, so that no vector-memory wait sits between a tile's DMA and the
//    previous tile's products.
//  * Causal and sliding-window masks apply to the tiles that cross the diagonal, the window's
//    lower edge or the ragged end only.  Row blocks are issued heaviest first within chunks of KV
//    heads sized to the last-level cache; every row block of all pairs over one KV head lands on
//    one XCD (XCDs are dealt round robin), so a KV head's K/V is shared through one L2.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"
#include "tile_common.hpp"

namespace da {
namespace {

using namespace tile;
constexpr int kThreads = 256;
constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for the reference max
constexpr float kCapSum = 4096.f;    // largest lane weight sum per tile (2^12) before m moves
constexpr float kF16Max = 65504.f;   // largest fp16 magnitude
constexpr int kSBN = 32;             // keys per tile

// 8 packed fp16 values -> 8 packed bf16 values (RNE)
__device__ __forceinline__ u32x4 f16x8_to_bf16x8(u32x4 x) {
  const f16x8 h = __builtin_bit_cast(f16x8, x);
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)(float)h[i];
  return __builtin_bit_cast(u32x4, r);
}

// V2 values for the fp16 P.V: one workgroup per 32-key tile of a KV head, one wave per region
// of 16 keys x 64 channels (rows 16 (w >> 1) + q / 8, channels 64 (w & 1) + 8 (q % 8) for
// q = lane + 64 s).  A region is written as fp16 unless it holds a value beyond the fp16 range
// (then as its bf16 bits), and its flag byte says which.  Rows past N are neither read (the
// buffer range check returns zeros) nor written.
__global__ __launch_bounds__(kThreads) void v2_values_kernel(const PrefillParams p) {
  const int tile = blockIdx.x;
  const int bh = blockIdx.y;  // b * Hkv + KV head
  const int b = bh / p.Hkv, kvh = bh % p.Hkv;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int N = p.N;
  const int kt = tile * kSBN;
  const uint32_t v_row = (uint32_t)(p.sv.sn * 2);
  const char* vsrc = static_cast<const char*>(p.v) + 2 * (b * p.sv.sb + kvh * p.sv.sh);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vsrc + (size_t)kt * v_row, (uint32_t)(N - kt) * v_row);
  u32x4 x[2];
  int row[2], col[2];
  float mx = 0.f;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int q = lane + 64 * s;
    row[s] = 16 * (w >> 1) + (q >> 3);
    col[s] = 64 * (w & 1) + 8 * (q & 7);
    x[s] = bload16(rv, (uint32_t)row[s] * v_row + col[s] * 2);
#pragma unroll
    for (int m = 0; m < 4; ++m) mx = fmaxf(mx, fmaxf(fabsf(bf16_lo(x[s][m])), fabsf(bf16_hi(x[s][m]))));
  }
  const bool big = __any(mx > kF16Max);
  bf16* dst = static_cast<bf16*>(p.vh) + (int64_t)bh * N * kDV;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    u32x4 y = x[s];
    if (!big) {
#pragma unroll
      for (int m = 0; m < 4; ++m) y[m] = pack_h2(bf16_lo(x[s][m]), bf16_hi(x[s][m]));
    }
    if (kt + row[s] < N) store16(dst + (int64_t)(kt + row[s]) * kDV + col[s], y);
  }
  if (lane == 0) p.vflags[((int64_t)bh * gridDim.x + tile) * 4 + w] = big ? 1 : 0;
}

constexpr int kStage = 32 * 128 + 32 * kDV;  // [K | V] elements per tile buffer (16 KB)
constexpr uint32_t kStageBytes = kStage * 2;
// Element offset of (row, col) in a V tile: 32-byte chunks XOR row & 7.
__device__ __forceinline__ int v8_off(int row, int col) {
  return row * kDV + ((((col >> 4) ^ (row & 7))) << 4) + (col & 15);
}
// sum / max over the four lanes that hold one query row (lanes n, n + 16, n + 32, n + 48)
__device__ __forceinline__ float row4_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}
__device__ __forceinline__ float row4_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3)))
void prefill_v2_kernel(const PrefillParams p) {
  __shared__ __attribute__((aligned(1024))) bf16 smem[2 * kStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g = lane >> 4;
  // Order: the (batch, KV head)s in chunks of head_chunk (see chunked_block); within a chunk the
  // row blocks heaviest first, then the pair within its KV head, the KV head running fastest, so
  // that every block over one KV head lands on the same XCD
  int rb, pi, kv;
  {
    const int bk = p.B * p.Hkv;
    const int ppk = p.pairs_per_kv;
    const int64_t lin = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    const int64_t csz = (int64_t)p.head_chunk * ppk * p.n_row_blocks;
    const int chunk = (int)(lin / csz);
    const int cn = min(p.head_chunk, bk - chunk * p.head_chunk);  // the last may be short
    const int j = (int)(lin - chunk * csz);
    rb = p.n_row_blocks - 1 - j / (cn * ppk);  // heaviest row block first
    const int r = j % (cn * ppk);
    pi = r / cn;
    kv = chunk * p.head_chunk + r % cn;
  }
  const int row0 = rb * 64;
  const int wrow = row0 + 16 * w;
  const int N = p.N;
  const int b = kv / p.Hkv, kvh = kv % p.Hkv;
  const int qh = kvh * p.pairs_per_kv + pi;

  // Q^T operands of both heads: lane (n, g) holds row wrow + n, columns 32 ks + 8 g .. + 7
  bf16x8 qa[4], qb[4];
  {
    const bf16* q1b = static_cast<const bf16*>(p.q1) + b * p.sq1.sb + qh * p.sq1.sh;
    const bf16* q2b = static_cast<const bf16*>(p.q2) + b * p.sq2.sb + qh * p.sq2.sh;
    const __amdgpu_buffer_rsrc_t r1 = make_rsrc(q1b, (uint32_t)(N * p.sq1.sn * 2));
    const __amdgpu_buffer_rsrc_t r2 = make_rsrc(q2b, (uint32_t)(N * p.sq2.sn * 2));
    const uint32_t row = (uint32_t)(wrow + n16);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qa[ks] = __builtin_bit_cast(bf16x8, bload16(r1, row * (uint32_t)(p.sq1.sn * 2) + 64 * ks + 16 * g));
      qb[ks] = __builtin_bit_cast(bf16x8, bload16(r2, row * (uint32_t)(p.sq2.sn * 2) + 64 * ks + 16 * g));
    }
    __builtin_amdgcn_s_waitcnt(0);
  }
  const int kv_end = p.causal ? min(N, row0 + 64) : N;
  const int ntiles = (kv_end + 31) / 32;
  const int t_begin = p.window > 0 ? max(0, row0 - p.window + 1) / 32 : 0;
  const bool wave_has_rows = wrow < N;
  const int last_key = p.causal ? min(N, wrow + 16) : N;
  const int nt_wave = wave_has_rows ? min(ntiles, (last_key + 31) / 32) : 0;
  const int t0_wave = p.window > 0 ? max(t_begin, max(0, wrow - p.window + 1) / 32) : 0;

  // K from the input, V from the fp16 copy (contiguous 256-byte rows); the flag word of each
  // 32-key tile is read through the scalar cache
  const int64_t vhead = (int64_t)b * p.Hkv + kvh;
  const uint32_t k_row = (uint32_t)(p.sk1.sn * 2);
  const char* k_base = static_cast<const char*>(p.k1) + 2 * (b * p.sk1.sb + kvh * p.sk1.sh);
  const char* v_base = static_cast<const char*>(p.vh) + vhead * N * (kDV * 2);
  typedef const __attribute__((address_space(4))) uint32_t const_u32;
  const_u32* vflag_words = (const_u32*)(p.vflags) + vhead * ((N + 31) / 32);
  // tile loads: wave w issues the 1 KB DMA loads w and w + 4 of the K tile and of the V tile;
  // lane offsets are relative to the tile's first row, which moves into the buffer base
  uint32_t k_lane[2], v_lane[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = 512 * (w + 4 * i) + 8 * lane;
    const int row = e >> 7;
    const int slot = (e & 127) >> 3;
    k_lane[i] = (uint32_t)row * k_row + (uint32_t)((slot ^ (row & 15)) * 16);
    const int lcol = (((slot >> 1) ^ (row & 7)) << 4) + ((slot & 1) << 3);
    v_lane[i] = (uint32_t)row * (kDV * 2) + lcol * 2;
  }
  auto issue_tile = [&](int i) {
    const int kt = i * 32;
    bf16* st = smem + (i & 1) * kStage;
    const uint32_t rows_left = (uint32_t)(N - kt);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(k_base + (size_t)kt * k_row, rows_left * k_row);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(v_base + (size_t)kt * (kDV * 2), rows_left * (kDV * 2));
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(rk, st + 512 * (w + 4 * j), k_lane[j]);
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(rv, st + 32 * 128 + 512 * (w + 4 * j), v_lane[j]);
  };
  uint32_t fw_cur = 0, fw_next = 0;  // flag words of the tile being computed / being loaded
  // LDS byte addresses of the operands.  K operand (key half h, k-step ks): row 16 h + n, 16-byte
  // chunk (4 ks + g) ^ n, i.e. ka ^ 64 ks + 4096 h.  V^T operand of channel tile t: rows
  // 4 g + n / 4 (+ 16 for the upper read), channels 16 t + 4 (n % 4), i.e. va ^ 32 t.
  const uint32_t ka = (uint32_t)(n16 * 256 + 16 * (g ^ n16));
  const uint32_t va = 2u * (uint32_t)(32 * 128 + v8_off(4 * g + (n16 >> 2), 4 * (n16 & 3)));
  const char* sb = reinterpret_cast<const char*>(smem);

  f32x4 acca[8], accb[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) { acca[t] = f32x4{0.f, 0.f, 0.f, 0.f}; accb[t] = f32x4{0.f, 0.f, 0.f, 0.f}; }
  float ma = kNegBig, mb = kNegBig, la = 0.f, lb = 0.f;
  const float sl2 = p.scale_log2;
  float nma = -ma * sl2, nmb = -mb * sl2;  // -m log2(e)/sqrt(D) per head, formed when m moves

  auto k_op = [&](uint32_t kb, int h, int ks) {
    return *reinterpret_cast<const bf16x8*>(sb + ((kb ^ (64u * ks)) + 4096u * h));
  };
  // S^T of both heads, each K operand read once for the two MFMAs
  auto scores2 = [&](uint32_t kb, f32x4 (&sa)[2], f32x4 (&sbb)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sa[h] = f32x4{0.f, 0.f, 0.f, 0.f};
      sbb[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = k_op(kb, h, ks);
        sa[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qa[ks], sa[h], 0, 0, 0);
        sbb[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[ks], sbb[h], 0, 0, 0);
      }
    }
  };
  // S^T of one head (the rare path that moves its reference max)
  auto scores1 = [&](uint32_t kb, const bf16x8 (&qf)[4], f32x4 (&s)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      s[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) s[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_op(kb, h, ks), qf[ks], s[h], 0, 0, 0);
    }
  };
  // causal diagonal, window edge and ragged end only
  auto mask = [&](f32x4 (&s)[2], int kt) {
    const int qrow = wrow + n16;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kt + 16 * h + 4 * g + r;
        if (key >= N || (p.causal && key > qrow) || (p.window > 0 && key <= qrow - p.window)) s[h][r] = -INFINITY;
      }
  };
  // weights exp2((s - m) log2(e) / sqrt(D)) against the reference max m, packed as k-slot
  // 4 h + r (fp16, or bf16 on the bf16 path); tl gets the lane's sum of the rounded weights
  // nm: -m log2(e)/sqrt(D) for the head's reference max m, formed when m moves
  auto weights = [&](const f32x4 (&s)[2], float nm, float& tl, auto half_tag) {
    constexpr bool kHalf = decltype(half_tag)::value;
    u32x4 o;
    tl = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = i >> 1, r = 2 * (i & 1);
      const float e0 = __builtin_amdgcn_exp2f(fmaf(s[h][r], sl2, nm));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(s[h][r + 1], sl2, nm));
      if constexpr (kHalf) {
        const f16x2 hv = {(_Float16)e0, (_Float16)e1};
        const f16x2 one = {(_Float16)1.f, (_Float16)1.f};
        tl = __builtin_amdgcn_fdot2(hv, one, tl, false);
        o[i] = __builtin_bit_cast(uint32_t, hv);
      } else {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 hv = {(bf16)e0, (bf16)e1};
        const bf16x2 one = {(bf16)1.f, (bf16)1.f};
        tl = __builtin_amdgcn_fdot2_f32_bf16(hv, one, tl, false);
        o[i] = __builtin_bit_cast(uint32_t, hv);
      }
    }
    return o;
  };
  // the rare path: the tile's exact row max moves m; that head's sums and accumulators rescale
  auto move_max = [&](uint32_t kb, const bf16x8 (&qf)[4], int kt, bool masked, float& m, float& l,
                      f32x4 (&acc)[8], float& tl, auto half_tag) {
    f32x4 s[2];
    scores1(kb, qf, s);
    if (masked) mask(s, kt);
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = row4_max(mx);
    const float mnew = fmaxf(m, mx);
    const float alpha = exp2f((m - mnew) * sl2);
    m = mnew;
    l *= alpha;
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] *= alpha;
    return weights(s, -m * sl2, tl, half_tag);
  };
  // One tile, both heads: scores, weights (moving a head's m when some weight would exceed
  // 2^12), then O^T += V^T P^T with each V^T operand feeding both heads' MFMAs.  kSlow: the bf16
  // P.V path, taken from the first tile holding a bf16 V region on.
  auto compute_tile = [&](int i, auto slow_tag, auto first_tag) {
    constexpr bool kSlow = decltype(slow_tag)::value;
    constexpr bool kFirst = decltype(first_tag)::value;
    const int kt = i * 32;
    const uint32_t off = (uint32_t)(i & 1) * kStageBytes;
    const uint32_t kb = ka + off, vb = va + off;
    const bool masked = (p.causal && kt + 31 > wrow) || kt + 32 > N ||
                        (p.window > 0 && kt <= wrow + 15 - p.window);
    f32x4 sa[2], sbb[2];
    __builtin_amdgcn_s_setprio(1);
    scores2(kb, sa, sbb);
    __builtin_amdgcn_s_setprio(0);
    if (masked) { mask(sa, kt); mask(sbb, kt); }
    if constexpr (kFirst) {
      // the wave's first tile: each head's m starts at this tile's exact row max (nothing is
      // accumulated yet, so nothing rescales, and every weight is at most 1)
      auto tile_max = [](const f32x4 (&s)[2]) {
        return fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
      };
      ma = fmaxf(ma, row4_max(tile_max(sa)));
      mb = fmaxf(mb, row4_max(tile_max(sbb)));
      nma = -ma * sl2;
      nmb = -mb * sl2;
    }
    using HT = std::integral_constant<bool, !kSlow>;
    float tla, tlb;
    u32x4 pa = weights(sa, nma, tla, HT{});
    if (!kFirst && __any(!(tla <= kCapSum))) {
      pa = move_max(kb, qa, kt, masked, ma, la, acca, tla, HT{});
      nma = -ma * sl2;
    }
    la += tla;
    u32x4 pb = weights(sbb, nmb, tlb, HT{});
    if (!kFirst && __any(!(tlb <= kCapSum))) {
      pb = move_max(kb, qb, kt, masked, mb, lb, accb, tlb, HT{});
      nmb = -mb * sl2;
    }
    lb += tlb;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t a = vb ^ (32u * t);
      u32x2 lo = lds_read_tr(reinterpret_cast<const bf16*>(sb + a));
      u32x2 hi = lds_read_tr(reinterpret_cast<const bf16*>(sb + a + 16 * kDV * 2));
      if constexpr (!kSlow) {
        const u32x4 a4 = {lo[0], lo[1], hi[0], hi[1]};
        acca[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a4), __builtin_bit_cast(f16x8, pa), acca[t], 0, 0, 0);
        accb[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a4), __builtin_bit_cast(f16x8, pb), accb[t], 0, 0, 0);
      } else {
        // regions kept as fp16 are widened back to bf16: rows 4g.. are key half 0, 16 + 4g.. half 1
        const int c = t >> 2;
        u32x4 a4 = {lo[0], lo[1], hi[0], hi[1]};
        const u32x4 wide = f16x8_to_bf16x8(a4);
        if (((fw_cur >> (8 * c)) & 0xffu) == 0u) { a4[0] = wide[0]; a4[1] = wide[1]; }
        if (((fw_cur >> (8 * (2 + c))) & 0xffu) == 0u) { a4[2] = wide[2]; a4[3] = wide[3]; }
        acca[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a4), __builtin_bit_cast(bf16x8, pa), acca[t], 0, 0, 0);
        accb[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a4), __builtin_bit_cast(bf16x8, pb), accb[t], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- main loop: the loads of tile i + 1 are in flight during tile i.  A wave computes the
  // tiles from its first to its last visible key and otherwise only helps load and meets the
  // barriers, so that the loops carrying the accumulators have no path around them; from the
  // first tile with a bf16 region on, a wave stays on the bf16 path, in a loop of its own.
  auto load_flags = [&](int i) -> uint32_t { return vflag_words[i]; };
  if (t_begin < ntiles) issue_tile(t_begin);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (t_begin < ntiles) fw_cur = load_flags(t_begin);
  auto help = [&](int i) {
    if (i + 1 < ntiles) { issue_tile(i + 1); fw_next = load_flags(i + 1); }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    fw_cur = fw_next;
  };
  auto step = [&](int i, auto slow_tag, auto first_tag) {
    if (i + 1 < ntiles) { issue_tile(i + 1); fw_next = load_flags(i + 1); }
    compute_tile(i, slow_tag, first_tag);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    fw_cur = fw_next;
  };
  int it = t_begin;
  for (; it < t0_wave; ++it) help(it);
  if (it < nt_wave && fw_cur == 0u) step(it++, std::false_type{}, std::true_type{});
  for (; it < nt_wave; ++it) {
    if (fw_cur != 0u) break;
    step(it, std::false_type{}, std::false_type{});
  }
  for (; it < nt_wave; ++it) step(it, std::true_type{}, std::false_type{});
  for (; it < ntiles; ++it) help(it);

  // ---- epilogue: out = O_a / l_a - lambda O_b / l_b; lane (n, g) holds row wrow + n, channels
  // 16 t + 4 g + r
  const float lam = head_lambda(p.lam, qh, lane);
  if (p.lam.out != nullptr && b == 0 && rb == 0 && w == 0 && lane == 0) p.lam.out[qh] = lam;
  if (!wave_has_rows) return;
  const float ia = 1.f / row4_sum(la), ib = lam / row4_sum(lb);
  const int qrow = wrow + n16;
  if (qrow >= N) return;
  bf16* orow = static_cast<bf16*>(p.out) + b * p.so.sb + qh * p.so.sh + (int64_t)qrow * p.so.sn;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    bf16x4 v4;
#pragma unroll
    for (int r = 0; r < 4; ++r) v4[r] = (bf16)(acca[t][r] * ia - accb[t][r] * ib);
    *reinterpret_cast<bf16x4*>(orow + 16 * t + 4 * g) = v4;
  }
}

}  // namespace

hipError_t launch_v2_bf16(const PrefillParams& p, hipStream_t stream) {
  PrefillParams q = p;
  q.pairs_per_kv = p.heads / p.Hkv;
  q.n_row_blocks = (p.N + 63) / 64;
  q.head_chunk = head_chunk((int64_t)p.B * p.Hkv, (int64_t)p.N * 2 * kDV * 2);  // K, V of a KV head (D = 128)
  hipLaunchKernelGGL(v2_values_kernel, dim3((p.N + kSBN - 1) / kSBN, p.B * p.Hkv), dim3(kThreads), 0, stream, q);
  const dim3 grid(p.B * p.heads, q.n_row_blocks);
  hipLaunchKernelGGL(prefill_v2_kernel, grid, dim3(kThreads), 0, stream, q);
  return hipGetLastError();
}

}  // namespace da
