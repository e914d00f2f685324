// Fused differential-attention prefill for gfx950: bf16 inputs, fp32 accumulation, bf16 out.
//
// What is computed (Ultralytics glossary "Differential Transformer", section "Cómo funciona la
// atención diferencial"; ai-engineering.academy "Atención Diferencial (V2)", sections "La idea
// diferencial" and "V1 vs V2: la diferencia"):
//   two softmax branches  A_b = softmax(Q_b K_b^T / sqrt(d)),  O = A_1 V - lambda A_2 V,
//   V1: y = (1 - lambda_init) O / sqrt(mean(O^2) + eps)   (per head, over the 128 channels),
//   V2: branches are the two query heads of a pair over one shared KV head; y = O.
// Neither map is ever written to memory.
//
// Design (one pass over K/V per query block):
//  * A 256-thread workgroup owns a block of query rows; each of its four wavefronts owns 32 query
//    rows (V1: 4 x 32 rows of one head; V2: 2 pairs x 2 x 32 rows, or 1 pair x 4 x 32 rows).
//  * K and V tiles of 64 keys stream global -> LDS with buffer loads that write LDS directly
//    (no staging registers); the buffer range check returns zeros past the last row.  Tiles are
//    double buffered: the loads of tile t+1 are in flight during the MFMAs of tile t.  LDS rows
//    are dense and XOR-swizzled for the 64-bank (256 B per clock) LDS: 16-byte chunks of K by
//    (row >> 1) & 7 (128-byte rows) or row & 15 (256-byte rows), 32-byte chunks of V by
//    2 (row & 3), so the MFMA operand reads are conflict-free (measured with
//    SQ_LDS_BANK_CONFLICT).  Per-lane read offsets are computed once, outside the key loop.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16.  Its accumulator
//    gives each lane one query column and, per 32-key block, keys {8j + 4h + r}; split into two
//    16-key halves these are exactly the B operand P^T of O^T = V^T P^T.  The matching V^T
//    operand comes straight from the row-major V tile with ds_read_b64_tr_b16 (a transposing LDS
//    read: per 16-lane group, each lane receives one column of a 4-key x 16-channel block).
//  * Each branch keeps its own online-softmax state per query row.  The running max moves only
//    when a row's new max exceeds it by more than 2^8 in exp2 units (the accumulators are then
//    rescaled); otherwise the stale max is kept, which changes no result because numerator and
//    row sum share it.  exp is exp2 with log2(e)/sqrt(d) folded into one FMA; the row sums add
//    the rounded weights the MFMA consumes (v_dot2 of packed pairs against 1).
//  * Epilogue: O = acc_1 / l_1 - lambda acc_2 / l_2, V1 RMS norm + scale, bf16 RNE store.
//  * Causal: tiles past a wavefront's last row are skipped; only tiles crossing the diagonal or
//    the ragged end are masked element by element.  Row blocks are issued heaviest first and all
//    row blocks of one head land on one XCD when the head count is a multiple of 8.
//  * F16PV (V2): P.V runs on the fp16 MFMA (P and V rounded to fp16, 11 significant bits instead
//    of bf16's 8).  V is then staged through registers and converted; a V tile holding any
//    |v| > 65504 stays bf16 and is multiplied on the bf16 MFMA, decided by a workgroup vote.
#include "device_common.hpp"
#include "launch.hpp"

namespace da {
namespace {

constexpr int kBN = 64;     // keys per tile
constexpr int kDV = 128;    // value width
constexpr int kThreads = 256;
constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for the running max
constexpr float kLazyLog2 = 8.f;     // largest exp2 argument allowed before the max is moved
constexpr float kF16Max = 65504.f;   // largest fp16 magnitude
constexpr int kRsrcWord3 = 0x00020000;  // buffer resource flags word for gfx9-family targets

typedef __attribute__((address_space(3))) void lds_void;

template <int DQK, bool V2>
struct Cfg {
  static constexpr int NK = V2 ? 1 : 2;              // K tiles per stage (shared K in V2)
  static constexpr int K_ELEMS = kBN * DQK;          // one K tile, dense
  static constexpr int V_ELEMS = kBN * kDV;          // one V tile, dense
  static constexpr int STAGE = NK * K_ELEMS + V_ELEMS;
  static constexpr int K_LOADS = K_ELEMS * 2 / 1024; // 1 KB wavefront DMA loads per K tile
  static constexpr int V_LOADS = V_ELEMS * 2 / 1024;
  static constexpr int TQ = DQK / 16;                // MFMA k-steps over the head width
};

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

// max / sum of x over the lane pair (l, l ^ 32).  (A v_permlane32_swap formulation was tried:
// the compiler treated both of its results as one value, so the exchange goes through
// ds_bpermute.)
__device__ __forceinline__ float pair_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
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
// base; one wait state separates the M0 write from the DMA.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, bf16* lds, uint32_t voff) {
  const uint32_t m0v = (uint32_t)(uintptr_t)(lds_void*)lds;
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(m0v), "v"(voff), "s"(r)
      : "memory");
}

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

template <int DQK, bool V2, int PPW, bool F16PV>
__global__ __launch_bounds__(kThreads) void prefill_kernel(const PrefillParams p) {
  using C = Cfg<DQK, V2>;
  constexpr int WPP = V2 ? 4 / PPW : 4;  // wavefronts per head (pair)
  constexpr int BM = 32 * WPP;           // query rows per workgroup
  __shared__ __attribute__((aligned(1024))) bf16 smem[2 * C::STAGE];
  __shared__ int vote[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (scalar)
  const int c = lane & 31;   // query column within the wave's 32 rows
  const int hh = lane >> 5;  // half of the wavefront
  const int rb = p.n_row_blocks - 1 - (int)blockIdx.y;  // heaviest row block first
  const int row0 = rb * BM;

  int b, kvh, qh;
  int wrow;
  if (!V2) {
    b = blockIdx.x / p.heads;
    qh = blockIdx.x % p.heads;
    kvh = qh;
    wrow = row0 + 32 * w;
  } else {
    const int grp = blockIdx.x % p.groups_per_kv;
    const int bg = blockIdx.x / p.groups_per_kv;
    kvh = bg % p.Hkv;
    b = bg / p.Hkv;
    qh = kvh * p.pairs_per_kv + grp * PPW + w / WPP;
    wrow = row0 + 32 * (w % WPP);
  }
  const int N = p.N;

  // ---- lambda prologue (per head / pair)
  const float lam = head_lambda(p.lam, qh, lane);
  // each head (pair) is owned by exactly one wave group of the b == 0, rb == 0 workgroups
  if (p.lam.out != nullptr && b == 0 && rb == 0 && (w % WPP) == 0 && lane == 0) p.lam.out[qh] = lam;

  // ---- buffer resources over each head slice: rows >= N fall outside and read as zeros
  const bf16* q1 = static_cast<const bf16*>(p.q1) + b * p.sq1.sb + qh * p.sq1.sh;
  const bf16* q2 = static_cast<const bf16*>(p.q2) + b * p.sq2.sb + qh * p.sq2.sh;
  const __amdgpu_buffer_rsrc_t rq1 = make_rsrc(q1, (uint32_t)(N * p.sq1.sn * 2));
  const __amdgpu_buffer_rsrc_t rq2 = make_rsrc(q2, (uint32_t)(N * p.sq2.sn * 2));
  const uint32_t k1_row = (uint32_t)(p.sk1.sn * 2), k2_row = (uint32_t)(p.sk2.sn * 2);
  const uint32_t v_row = (uint32_t)(p.sv.sn * 2);

  // ---- Q^T B-operands: lane holds query row wrow + c, head-width elements 16t + 8hh .. +7
  bf16x8 qf[2][C::TQ];
  {
    const uint32_t r1 = (uint32_t)((wrow + c) * p.sq1.sn * 2), r2 = (uint32_t)((wrow + c) * p.sq2.sn * 2);
#pragma unroll
    for (int t = 0; t < C::TQ; ++t) {
      qf[0][t] = __builtin_bit_cast(bf16x8, bload16(rq1, r1 + 32 * t + 16 * hh));
      qf[1][t] = __builtin_bit_cast(bf16x8, bload16(rq2, r2 + 32 * t + 16 * hh));
    }
    __builtin_amdgcn_s_waitcnt(0);  // settle Q before the asm tile DMA starts
  }

  // ---- key range of this workgroup
  const int kv_end = p.causal ? min(N, row0 + BM) : N;
  const int ntiles = (kv_end + kBN - 1) / kBN;

  // ---- tile loads.  A wavefront DMA load writes 64 x 16 B contiguously at lane order; each
  // lane fetches the global chunk that belongs at its (swizzled) LDS slot.  The tile's first row
  // moves into the buffer base (scalar), so the per-lane offsets are loop invariant.
  constexpr int KPW = C::K_LOADS / 4;  // K DMA loads per wave per tensor
  constexpr int VPW = C::V_LOADS / 4;
  uint32_t k_lane[C::NK][KPW], v_lane[VPW];
#pragma unroll
  for (int nk = 0; nk < C::NK; ++nk)
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
      const int e = 512 * (w + 4 * i) + 8 * lane;  // element this lane's 16 B lands on
      const int row = e / DQK;
      const int lchunk = ((e % DQK) >> 3) ^ k_swz<DQK>(row);
      k_lane[nk][i] = (uint32_t)row * (nk == 0 ? k1_row : k2_row) + lchunk * 16;
    }
#pragma unroll
  for (int i = 0; i < VPW; ++i) {
    const int e = 512 * (w + 4 * i) + 8 * lane;
    const int row = e >> 7;
    const int slot = (e & 127) >> 3;  // physical 16-byte slot in the row
    const int lcol = ((((slot >> 1) ^ (2 * (row & 3)))) << 4) + ((slot & 1) << 3);
    v_lane[i] = (uint32_t)row * v_row + lcol * 2;
  }
  const char* k1_base = static_cast<const char*>(p.k1) + 2 * (b * p.sk1.sb + kvh * p.sk1.sh);
  const char* k2_base = static_cast<const char*>(p.k2) + 2 * (b * p.sk2.sb + kvh * p.sk2.sh);
  const char* v_base = static_cast<const char*>(p.v) + 2 * (b * p.sv.sb + kvh * p.sv.sh);

  u32x4 vreg[4];  // F16PV only: V chunks staged through registers
  auto issue_tile = [&](int kt, int buf) {
    bf16* st = smem + buf * C::STAGE;
    const int rows_left = N - kt;
#pragma unroll
    for (int nk = 0; nk < C::NK; ++nk) {
      const uint32_t krow = nk == 0 ? k1_row : k2_row;
      const __amdgpu_buffer_rsrc_t rk =
          make_rsrc((nk == 0 ? k1_base : k2_base) + (size_t)kt * krow, (uint32_t)rows_left * krow);
#pragma unroll
      for (int i = 0; i < KPW; ++i) dma16(rk, st + nk * C::K_ELEMS + 512 * (w + 4 * i), k_lane[nk][i]);
    }
    bf16* vt = st + C::NK * C::K_ELEMS;
    const __amdgpu_buffer_rsrc_t rvt = make_rsrc(v_base + (size_t)kt * v_row, (uint32_t)rows_left * v_row);
    if constexpr (!F16PV) {
#pragma unroll
      for (int i = 0; i < VPW; ++i) dma16(rvt, vt + 512 * (w + 4 * i), v_lane[i]);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int ch = tid + kThreads * s;  // 16-byte chunk of the 64 x 128 tile
        vreg[s] = bload16(rvt, (uint32_t)(ch >> 4) * v_row + ((ch & 15) << 4));
      }
    }
  };

  // F16PV: workgroup-wide vote -- does the staged V tile hold a value fp16 cannot represent?
  auto vote_big = [&]() -> bool {
    float mx = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        mx = fmaxf(mx, fmaxf(fabsf(bf16_lo(vreg[s][m])), fabsf(bf16_hi(vreg[s][m]))));
    const bool any = __any(mx > kF16Max);
    if (lane == 0) vote[w] = any ? 1 : 0;
    __syncthreads();
    return (vote[0] | vote[1] | vote[2] | vote[3]) != 0;
  };

  // F16PV: write the staged V chunks (converted to fp16 unless the tile is big) into LDS
  auto store_v = [&](int buf, bool big) {
    bf16* vt = smem + buf * C::STAGE + C::NK * C::K_ELEMS;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = tid + kThreads * s;
      const int row = ch >> 4;
      const int col = (ch & 15) << 3;
      u32x4 x = vreg[s];  // 8 channels of one row
      if (!big) {
#pragma unroll
        for (int m = 0; m < 4; ++m) x[m] = pack_h2(bf16_lo(vreg[s][m]), bf16_hi(vreg[s][m]));
      }
      store16(vt + v_off(row, col), x);
    }
  };

  // ---- per-wave running state
  f32x16 acc[2][4];
#pragma unroll
  for (int br = 0; br < 2; ++br)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[br][db][r] = 0.f;
  float mrun[2] = {kNegBig, kNegBig};
  float lrun[2] = {0.f, 0.f};
  const float sl2 = p.scale_log2;
  const bool wave_has_rows = wrow < N;

  // Per-lane LDS read offsets (elements), loop invariant.
  //  K operand of S^T: row kb*32 + c, chunk 2t + hh; the swizzle depends on the lane only.
  int k_rd[C::TQ];
#pragma unroll
  for (int t = 0; t < C::TQ; ++t) k_rd[t] = k_off<DQK>(c, 16 * t + 8 * hh);
  //  V^T operand: two transposing reads per operand.  In each 16-lane group lane j addresses row
  //  key0 + j/4, channels dv0 + 4 (j % 4) .. +3 (see the file header); row & 3 = (j >> 2) & 3,
  //  so the swizzle again depends on the lane only.
  int v_rd[4];
  {
    const int j = lane & 15, dh = (lane >> 4) & 1;
    const int row = 4 * hh + (j >> 2);
#pragma unroll
    for (int db = 0; db < 4; ++db) v_rd[db] = v_off(row, db * 32 + dh * 16 + 4 * (j & 3));
  }

  // One 32-key half of a tile at a time keeps only 2 x 16 score registers live.
  auto compute_tile = [&](int buf, int kt, bool bigv) {
    if (!wave_has_rows) return;
    const bf16* st = smem + buf * C::STAGE;
    const bf16* vt = st + C::NK * C::K_ELEMS;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kh = kt + 32 * kb;             // first key of this half
      if (p.causal && kh > wrow + 31) break;   // this half and the next are in the future

      // S^T = K Q^T for both branches: s[br] holds keys kh + 8j + 4hh + r (reg 4j + r)
      __builtin_amdgcn_s_setprio(1);
      f32x16 s[2];
#pragma unroll
      for (int br = 0; br < 2; ++br)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[br][r] = 0.f;
#pragma unroll
      for (int t = 0; t < C::TQ; ++t) {
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(st + kb * 32 * DQK + k_rd[t]);
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[0][t], s[0], 0, 0, 0);
        if constexpr (V2) {
          s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[1][t], s[1], 0, 0, 0);
        } else {
          const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(st + C::K_ELEMS + kb * 32 * DQK + k_rd[t]);
          s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[1][t], s[1], 0, 0, 0);
        }
      }

      __builtin_amdgcn_s_setprio(0);
      // masking: causal diagonal and ragged end
      if ((p.causal && kh + 31 > wrow) || kh + 32 > N) {
        const int qrow = wrow + c;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kh + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key >= N || (p.causal && key > qrow)) {
            s[0][r] = -INFINITY;
            s[1][r] = -INFINITY;
          }
        }
      }

      // online softmax per branch with a lazily moved max (P is left in s as fp32)
#pragma unroll
      for (int br = 0; br < 2; ++br) {
        float mx = s[br][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[br][r]);
        mx = pair_max(mx);
        if (__any((mx - mrun[br]) * sl2 > kLazyLog2)) {
          const float mnew = fmaxf(mrun[br], mx);
          const float alpha = exp2f((mrun[br] - mnew) * sl2);
          mrun[br] = mnew;
          lrun[br] *= alpha;
#pragma unroll
          for (int db = 0; db < 4; ++db) acc[br][db] *= alpha;
        }
        const float nm = -mrun[br] * sl2;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[br][r] = __builtin_amdgcn_exp2f(fmaf(s[br][r], sl2, nm));
      }

      // O^T += V^T P^T for both branches; the V^T operand (two transposing reads) is shared
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int rbase = (kb * 32 + 16 * u) * kDV;  // first row of this 16-key group
        if (F16PV && !bigv) {
          const f16x8 p0 = cvt8h_sum(s[0], 8 * u, lrun[0]);
          const f16x8 p1 = cvt8h_sum(s[1], 8 * u, lrun[1]);
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const u32x2 lo = lds_read_tr(vt + rbase + v_rd[db]);
            const u32x2 hi = lds_read_tr(vt + rbase + 8 * kDV + v_rd[db]);
            const u32x4 a4 = {lo[0], lo[1], hi[0], hi[1]};
            const f16x8 a = __builtin_bit_cast(f16x8, a4);
            acc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, p0, acc[0][db], 0, 0, 0);
            acc[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, p1, acc[1][db], 0, 0, 0);
          }
        } else {
          const bf16x8 p0 = cvt8_sum(s[0], 8 * u, lrun[0]);
          const bf16x8 p1 = cvt8_sum(s[1], 8 * u, lrun[1]);
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const u32x2 lo = lds_read_tr(vt + rbase + v_rd[db]);
            const u32x2 hi = lds_read_tr(vt + rbase + 8 * kDV + v_rd[db]);
            const u32x4 a4 = {lo[0], lo[1], hi[0], hi[1]};
            const bf16x8 a = __builtin_bit_cast(bf16x8, a4);
            acc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p0, acc[0][db], 0, 0, 0);
            acc[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p1, acc[1][db], 0, 0, 0);
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
    }
  };

  // ---- main loop: DMA of tile t+1 overlaps the MFMAs of tile t; one barrier per tile (plus the
  // vote's barrier on the F16PV path)
  if (ntiles > 0) {
    issue_tile(0, 0);
    bool big_cur = false;
    if constexpr (F16PV) {
      big_cur = vote_big();
      store_v(0, big_cur);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
      const bool more = it + 1 < ntiles;
      if (more) issue_tile((it + 1) * kBN, (it + 1) & 1);
      compute_tile(it & 1, it * kBN, big_cur);
      if constexpr (F16PV) {
        if (more) {
          const bool big_next = vote_big();
          store_v((it + 1) & 1, big_next);
          big_cur = big_next;
        }
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  // ---- epilogue
  if (!wave_has_rows) return;
  const int qrow = wrow + c;
  const float l1 = pair_sum(lrun[0]);
  const float l2 = pair_sum(lrun[1]);
  const float i1 = 1.f / l1;
  const float i2 = lam / l2;
  float o[4][16];
  float ss = 0.f;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float x = acc[0][db][r] * i1 - acc[1][db][r] * i2;
      o[db][r] = x;
      ss = fmaf(x, x, ss);
    }
  float rs = 1.f;
  if (!V2 && p.norm) {
    ss = pair_sum(ss);
    rs = p.out_scale * rsqrtf(ss * (1.f / kDV) + p.eps);
  }
  if (qrow >= N) return;
  bf16* orow = static_cast<bf16*>(p.out) + b * p.so.sb + qh * p.so.sh + (int64_t)qrow * p.so.sn;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4 v4;
#pragma unroll
      for (int r = 0; r < 4; ++r) v4[r] = (bf16)(o[db][4 * j + r] * rs);
      *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * j + 4 * hh) = v4;
    }
}

}  // namespace

hipError_t launch_v1_bf16(const PrefillParams& p, hipStream_t stream) {
  PrefillParams q = p;
  q.n_row_blocks = (p.N + 127) / 128;
  const dim3 grid(p.B * p.heads, q.n_row_blocks);
  hipLaunchKernelGGL((prefill_kernel<64, false, 1, false>), grid, dim3(kThreads), 0, stream, q);
  return hipGetLastError();
}

hipError_t launch_v2_bf16(const PrefillParams& p, int pairs_per_wg, hipStream_t stream) {
  PrefillParams q = p;
  q.pairs_per_kv = p.heads / p.Hkv;
  if (pairs_per_wg == 2) {
    q.groups_per_kv = q.pairs_per_kv / 2;
    q.n_row_blocks = (p.N + 63) / 64;
    const dim3 grid(p.B * p.Hkv * q.groups_per_kv, q.n_row_blocks);
    hipLaunchKernelGGL((prefill_kernel<128, true, 2, true>), grid, dim3(kThreads), 0, stream, q);
  } else {
    q.groups_per_kv = q.pairs_per_kv;
    q.n_row_blocks = (p.N + 127) / 128;
    const dim3 grid(p.B * p.Hkv * q.groups_per_kv, q.n_row_blocks);
    hipLaunchKernelGGL((prefill_kernel<128, true, 1, true>), grid, dim3(kThreads), 0, stream, q);
  }
  return hipGetLastError();
}

}  // namespace da
