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
//  * K and V tiles of 64 keys are staged through LDS with register double buffering: the global
//    loads of tile t+1 are issued before the MFMAs of tile t.  V is transposed on its way into LDS
//    (V^T rows = value channels) so that the P.V product reads contiguous key runs.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: the accumulator
//    layout then gives each lane one query column and 16 keys per 32-key block, which is exactly
//    the B-operand layout P^T needs for O^T = V^T P^T once the key order inside the V^T tile is
//    permuted (bits 2 and 3 of the key index swapped).  No shuffles are needed between the two
//    products.
//  * Each branch keeps its own online-softmax state (running max, running sum) per query row in
//    registers; the lane pair (c, c+32) holding one query column agrees on the max with one
//    cross-lane exchange.  exp is evaluated as exp2 with log2(e)/sqrt(d) folded into one FMA.
//  * Epilogue: O = acc_1 / l_1 - lambda acc_2 / l_2, V1 RMS norm + scale, bf16 RNE store.
//  * Causal: tiles past a wavefront's last row are skipped; only tiles crossing the diagonal or
//    the ragged end are masked element by element.  Row blocks are issued heaviest first and
//    all blocks of one head land on one XCD when the head count is a multiple of 8.
#include "device_common.hpp"
#include "launch.hpp"

namespace da {
namespace {

constexpr int kBN = 64;     // keys per tile
constexpr int kDV = 128;    // value width
constexpr int kThreads = 256;
constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for the running max

template <int DQK, bool V2>
struct Cfg {
  static constexpr int KSTR = DQK + 8;               // LDS row stride (elements) of a K tile
  static constexpr int VSTR = kBN + 8;               // LDS row stride (elements) of a V^T tile
  static constexpr int NK = V2 ? 1 : 2;              // K tiles per stage (shared K in V2)
  static constexpr int K_ELEMS = kBN * KSTR;
  static constexpr int V_ELEMS = kDV * VSTR;
  static constexpr int STAGE = NK * K_ELEMS + V_ELEMS;
  static constexpr int KCH = kBN * DQK / 8 / kThreads;  // 16-byte K chunks per thread per tensor
  static constexpr int TQ = DQK / 16;                // MFMA k-steps over the head width
};

// Position of key `kk` (0..63) inside a V^T tile row: bits 2 and 3 swapped.
__device__ __forceinline__ int vt_pos(int kk) { return (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1); }

__device__ __forceinline__ bf16x8 lds_read8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ bf16x8 cvt8(const f32x16& s, int base) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)s[base + i];
  return r;
}

__device__ __forceinline__ f16x8 cvt8h(const f32x16& s, int base) {
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (_Float16)s[base + i];
  return r;
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  f16x2 h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// Largest magnitude an fp16 operand may take without overflowing.
constexpr float kF16Max = 65504.f;

// F16PV: the P.V product runs on the fp16 MFMA (P and V rounded to fp16, 11 significant bits,
// instead of bf16's 8).  A V tile holding any |v| > 65504 is staged and multiplied in bf16
// instead, decided by a workgroup-wide vote, so no input range is lost.
template <int DQK, bool V2, int PPW, bool F16PV>
__global__ __launch_bounds__(kThreads) void prefill_kernel(const PrefillParams p) {
  using C = Cfg<DQK, V2>;
  constexpr int WPP = V2 ? 4 / PPW : 4;  // wavefronts per head (pair)
  constexpr int BM = 32 * WPP;           // query rows per workgroup
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * C::STAGE];
  __shared__ int vote[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
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

  const bf16* q1 = static_cast<const bf16*>(p.q1) + b * p.sq1.sb + qh * p.sq1.sh;
  const bf16* q2 = static_cast<const bf16*>(p.q2) + b * p.sq2.sb + qh * p.sq2.sh;
  const bf16* kb1 = static_cast<const bf16*>(p.k1) + b * p.sk1.sb + kvh * p.sk1.sh;
  const bf16* kb2 = static_cast<const bf16*>(p.k2) + b * p.sk2.sb + kvh * p.sk2.sh;
  const bf16* vb = static_cast<const bf16*>(p.v) + b * p.sv.sb + kvh * p.sv.sh;

  // ---- Q^T B-operands: lane holds query row wrow + c, head-width elements 16t + 8hh .. +7
  bf16x8 qf[2][C::TQ];
  {
    const int row = wrow + c;
    const bool ok = row < N;
#pragma unroll
    for (int t = 0; t < C::TQ; ++t) {
      u32x4 a = {0u, 0u, 0u, 0u}, e = {0u, 0u, 0u, 0u};
      if (ok) {
        a = load16(q1 + (int64_t)row * p.sq1.sn + 16 * t + 8 * hh);
        e = load16(q2 + (int64_t)row * p.sq2.sn + 16 * t + 8 * hh);
      }
      qf[0][t] = __builtin_bit_cast(bf16x8, a);
      qf[1][t] = __builtin_bit_cast(bf16x8, e);
    }
  }

  // ---- key range of this workgroup
  const int kv_end = p.causal ? min(N, row0 + BM) : N;
  const int ntiles = (kv_end + kBN - 1) / kBN;

  // ---- global -> register staging of one K/V tile
  u32x4 kreg[C::NK][C::KCH];
  u32x4 vreg[4];
  const int v_kq = tid & 15;  // keys 4*v_kq .. +3 of the tile
  const int v_cc = tid >> 4;  // value channels 8*v_cc .. +7

  auto load_tile = [&](int kt) {
#pragma unroll
    for (int nk = 0; nk < C::NK; ++nk) {
      const bf16* kb = nk == 0 ? kb1 : kb2;
      const int64_t sn = nk == 0 ? p.sk1.sn : p.sk2.sn;
#pragma unroll
      for (int s = 0; s < C::KCH; ++s) {
        const int ch = tid + kThreads * s;
        const int row = ch / (DQK / 8);
        const int col = (ch % (DQK / 8)) * 8;
        const int key = kt + row;
        kreg[nk][s] = key < N ? load16(kb + (int64_t)key * sn + col) : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = kt + 4 * v_kq + r;
      vreg[r] = key < N ? load16(vb + (int64_t)key * p.sv.sn + 8 * v_cc) : u32x4{0u, 0u, 0u, 0u};
    }
  };

  auto store_tile = [&](int buf, bool big) {
    bf16* st = smem + buf * C::STAGE;
#pragma unroll
    for (int nk = 0; nk < C::NK; ++nk) {
#pragma unroll
      for (int s = 0; s < C::KCH; ++s) {
        const int ch = tid + kThreads * s;
        const int row = ch / (DQK / 8);
        const int col = (ch % (DQK / 8)) * 8;
        store16(st + nk * C::K_ELEMS + row * C::KSTR + col, kreg[nk][s]);
      }
    }
    // transpose 4 keys x 8 channels into 8 channel rows x 4 keys
    bf16* vt = st + C::NK * C::K_ELEMS;
    const int pos = vt_pos(4 * v_kq);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t w0 = vreg[0][m], w1 = vreg[1][m], w2 = vreg[2][m], w3 = vreg[3][m];
      u32x2 lo, hi;  // channel 2m (low halves) and 2m+1 (high halves)
      if (F16PV && !big) {
        lo[0] = pack_h2(bf16_lo(w0), bf16_lo(w1));
        lo[1] = pack_h2(bf16_lo(w2), bf16_lo(w3));
        hi[0] = pack_h2(bf16_hi(w0), bf16_hi(w1));
        hi[1] = pack_h2(bf16_hi(w2), bf16_hi(w3));
      } else {
        lo[0] = (w0 & 0xffffu) | (w1 << 16);
        lo[1] = (w2 & 0xffffu) | (w3 << 16);
        hi[0] = (w0 >> 16) | (w1 & 0xffff0000u);
        hi[1] = (w2 >> 16) | (w3 & 0xffff0000u);
      }
      *reinterpret_cast<u32x2*>(vt + (8 * v_cc + 2 * m) * C::VSTR + pos) = lo;
      *reinterpret_cast<u32x2*>(vt + (8 * v_cc + 2 * m + 1) * C::VSTR + pos) = hi;
    }
  };

  // Workgroup-wide vote: does the staged V tile hold a value fp16 cannot represent?
  // (Called by every thread between two barriers; returns the same answer everywhere.)
  auto vote_big = [&]() -> bool {
    if constexpr (!F16PV) {
      return true;
    } else {
      float mx = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          mx = fmaxf(mx, fmaxf(fabsf(bf16_lo(vreg[r][m])), fabsf(bf16_hi(vreg[r][m]))));
      const bool any = __any(mx > kF16Max);
      if (lane == 0) vote[w] = any ? 1 : 0;
      __syncthreads();
      const bool big = (vote[0] | vote[1] | vote[2] | vote[3]) != 0;
      return big;
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

  auto compute_tile = [&](int buf, int kt, bool big) {
    if (!wave_has_rows) return;
    if (p.causal && kt > wrow + 31) return;  // every key of the tile is in this wave's future
    const bf16* st = smem + buf * C::STAGE;
    const bf16* vt = st + C::NK * C::K_ELEMS;

    // S^T = K Q^T for both branches: s[br][kb] holds keys kb*32 + 8j + 4hh + r (reg 4j + r)
    f32x16 s[2][2];
#pragma unroll
    for (int br = 0; br < 2; ++br) {
      const bf16* kt_lds = st + (V2 ? 0 : br) * C::K_ELEMS;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[br][kb][r] = 0.f;
#pragma unroll
        for (int t = 0; t < C::TQ; ++t) {
          const bf16x8 a = lds_read8(kt_lds + (kb * 32 + c) * C::KSTR + 16 * t + 8 * hh);
          s[br][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[br][t], s[br][kb], 0, 0, 0);
        }
      }
    }

    // masking: causal diagonal and ragged end
    const bool need_mask = (p.causal && kt + kBN - 1 > wrow) || (kt + kBN > N);
    if (need_mask) {
      const int qrow = wrow + c;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          const bool masked = key >= N || (p.causal && key > qrow);
          if (masked) {
            s[0][kb][r] = -INFINITY;
            s[1][kb][r] = -INFINITY;
          }
        }
    }

    // online softmax per branch (P is left in s as fp32)
#pragma unroll
    for (int br = 0; br < 2; ++br) {
      float mx = s[br][0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[br][kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mrun[br], mx);
      const float alpha = exp2f((mrun[br] - mnew) * sl2);
      mrun[br] = mnew;
      const float nm = -mnew * sl2;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(s[br][kb][r], sl2, nm));
          s[br][kb][r] = e;
          ls += e;
        }
      lrun[br] = lrun[br] * alpha + ls;
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[br][db] *= alpha;
    }

    // O^T += V^T P^T for both branches (the V^T operand is shared)
    if (F16PV && !big) {
      f16x8 ph[2][2][2];
#pragma unroll
      for (int br = 0; br < 2; ++br)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          ph[br][kb][0] = cvt8h(s[br][kb], 0);
          ph[br][kb][1] = cvt8h(s[br][kb], 8);
        }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const f16x8 a = *reinterpret_cast<const f16x8*>(vt + (db * 32 + c) * C::VSTR + kb * 32 + 16 * u + 8 * hh);
            acc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, ph[0][kb][u], acc[0][db], 0, 0, 0);
            acc[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, ph[1][kb][u], acc[1][db], 0, 0, 0);
          }
    } else {
      bf16x8 pb[2][2][2];
#pragma unroll
      for (int br = 0; br < 2; ++br)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          pb[br][kb][0] = cvt8(s[br][kb], 0);
          pb[br][kb][1] = cvt8(s[br][kb], 8);
        }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const bf16x8 a = lds_read8(vt + (db * 32 + c) * C::VSTR + kb * 32 + 16 * u + 8 * hh);
            acc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[0][kb][u], acc[0][db], 0, 0, 0);
            acc[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[1][kb][u], acc[1][db], 0, 0, 0);
          }
    }
  };

  // ---- main loop: one barrier per tile (plus the vote's barrier on the fp16 path)
  if (ntiles > 0) {
    load_tile(0);
    bool big_cur = vote_big();
    store_tile(0, big_cur);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
      const bool more = it + 1 < ntiles;
      if (more) load_tile((it + 1) * kBN);
      compute_tile(it & 1, it * kBN, big_cur);
      if (more) {
        const bool big_next = vote_big();
        store_tile((it + 1) & 1, big_next);
        big_cur = big_next;
      }
      __syncthreads();
    }
  }

  // ---- epilogue
  if (!wave_has_rows) return;
  const int qrow = wrow + c;
  const float l1 = lrun[0] + __shfl_xor(lrun[0], 32);
  const float l2 = lrun[1] + __shfl_xor(lrun[1], 32);
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
    ss += __shfl_xor(ss, 32);
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
