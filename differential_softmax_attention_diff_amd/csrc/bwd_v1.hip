// Backward pass of the V1 differential attention for gfx950: bf16 inputs, fp32 accumulation,
// fp32 gradients.
//
// What is differentiated (Ultralytics glossary "Differential Transformer", section "Cómo funciona
// la atención diferencial"; ai-engineering.academy "Atención Diferencial (V2)", section "La idea
// diferencial"): per head, S_b = Q_b K_b^T / sqrt(d), A_b = softmax(S_b), O = A_1 V - lambda A_2 V,
// y = (1 - lambda_init) O / sqrt(mean(O^2) + eps), lambda = exp(<lq1,lk1>) - exp(<lq2,lk2>) +
// lambda_init.  The chain rule gives
//   dO   = g r dy - g r^3 (O . dy) O / 2d          (g = 1 - lambda_init, r = 1/rms(O))
//   dV   = A_1^T dO - lambda A_2^T dO
//   dS_b = A_b * (dP_b - D_b),  dP_1 = dO V^T, dP_2 = -lambda dO V^T,
//   D_1  = dO . O_1,  D_2 = -lambda dO . O_2       (row-wise; O_b = A_b V from the forward)
//   dQ_b = dS_b K_b / sqrt(d),  dK_b = dS_b^T Q_b / sqrt(d),
//   dlambda = -sum(dO . O_2), and the four lambda vectors through the exponentials.
// With c_1 = 1, c_2 = -lambda and Dt_b = dO . O_b, dS_b = c_b A_b * (dO V^T - Dt_b): the kernels
// form A_b * (dO V^T - Dt_b), starting the dO V^T accumulator at -Dt_b, and apply c_b once to the
// finished dQ_b, dK_b and branch-2 part of dV.
//
// Kernels (A_b is never stored: each kernel rebuilds the weights it needs from the scores and the
// forward's base-2 log-sum-exp, P = exp2(s log2(e)/sqrt(d) - LSE)):
//  * bwd_dq (first): one workgroup per 128 query rows, one wave per 32 of them doing both
//    branches.  Its prologue forms, for its rows, O, r and dO (bf16, for the MFMAs), -Dt_1, -Dt_2
//    and the row's share of dlambda, 16 lanes per row, and stores them for the dK/dV kernel; its
//    own operands come through LDS.  Then V dO^T is formed once for both branches while it
//    streams K_1, K_2, V tiles: S_b^T = K_b Q_b^T, P_b^T, X^T = V dO^T, dS_b^T,
//    dQ_b^T += K_b^T dS_b^T.
//  * bwd_dkdv: one 256-thread workgroup per 64 keys of a head, one wave per 16 of them doing
//    both branches.  Each wave keeps its keys' K_1, K_2 and V as MFMA operands in registers and
//    streams 32-row query tiles (Q_1, Q_2, dO, LSE, -Dt) through LDS: S_b = Q_b K_b^T and one
//    X = dO V^T for both branches on 16x16x32 bf16 MFMAs, P_b, dS_b, then dV^T += dO^T (P_1 -
//    lambda P_2) once and dK_b^T += Q_b^T dS_b, the transposed operands read by
//    ds_read_b64_tr_b16.  The accumulator layout feeds the next product directly.
//  * bwd_lambda: per head, the sum of the rows' dlambda shares (one 1024-thread workgroup, fixed
//    order) and the four vector gradients.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"
#include "tile_common.hpp"

namespace da {
namespace {

using namespace tile;
constexpr int kD = 64;        // query / key half width
constexpr int kT = 32;        // rows (keys or queries) per tile
constexpr int kThreads = 256;

__device__ __forceinline__ float lam_of(const BwdParams& p, int h, int lane) {
  return head_lambda(p.lam, h, lane);
}

// ---------------------------------------------------------------------------------------------
// prep (in the dQ kernel's prologue): dO through the norm, -Dt_b, dlambda shares; 16 lanes per
// row (8 of its 2d channels each), four rows per wavefront pass, eight passes for a wave's rows
constexpr int kPrepGroup = 2;  // passes whose loads are issued together

// sum over the 16 lanes that share a row (xor partners stay inside the group)
__device__ __forceinline__ float row16_sum(float x) {
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

// One row of the prep pass, 16 lanes per row (lane sub holds channels 8 sub .. 8 sub + 7):
// O = O_1 - lambda O_2, r = 1/rms(O), dO = g r dy - g r^3 (O . dy) O / 2d rounded to bf16 (dq),
// -Dt_1 = -dO . O_1 and -Dt_2 = -dO . O_2 from the rounded dO, and -dO . O_2 from the unrounded
// one (the row's share of dlambda).  prep_load reads the row's stash and dy (row rc must be a
// valid row), prep_row does the arithmetic.
struct PrepIn {
  f32x4 a1l, a1h, a2l, a2h;
  u32x4 yw;
};
__device__ __forceinline__ PrepIn prep_load(const BwdParams& p, int b, int h, int64_t r, int rc, int sub,
                                            int64_t BHN) {
  const float* o1 = p.stash_o + r * kDV + 8 * sub;
  const float* o2 = p.stash_o + (BHN + r) * kDV + 8 * sub;
  const bf16* dy = static_cast<const bf16*>(p.dy) + b * p.sdy.sb + h * p.sdy.sh + (int64_t)rc * p.sdy.sn + 8 * sub;
  // read once: non-temporal
  PrepIn in;
  in.a1l = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(o1));
  in.a1h = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(o1 + 4));
  in.a2l = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(o2));
  in.a2h = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(o2 + 4));
  in.yw = load16_nt(dy);
  return in;
}
__device__ __forceinline__ void prep_row(const BwdParams& p, const PrepIn& in, float lam, bf16x8& dq,
                                         float& nd1, float& nd2, float& ndl) {
  const f32x4 a1l = in.a1l, a1h = in.a1h, a2l = in.a2l, a2h = in.a2h;
  const u32x4 yw = in.yw;
  float a1[8], a2[8], y[8], x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a1[i] = a1l[i]; a1[4 + i] = a1h[i];
    a2[i] = a2l[i]; a2[4 + i] = a2h[i];
    y[2 * i] = bf16_lo(yw[i]);
    y[2 * i + 1] = bf16_hi(yw[i]);
  }
  float ss = 0.f, dot = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = a1[i] - lam * a2[i];
    ss = fmaf(x[i], x[i], ss);
    dot = fmaf(x[i], y[i], dot);
  }
  ss = row16_sum(ss);
  dot = row16_sum(dot);
  const float rr = rsqrtf(ss * (1.f / kDV) + p.eps);
  const float k1 = p.g * rr, k2 = p.g * rr * rr * rr * dot * (1.f / kDV);
  float e1 = 0.f, e2 = 0.f, g2 = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float d = k1 * y[i] - k2 * x[i];
    dq[i] = (bf16)d;
    // Dt_b from the rounded dO the MFMAs use, so that c_b Dt_b equals the row sum of P_b * dP_b
    // that they form (the softmax Jacobian's subtraction then cancels what it should)
    const float dr = (float)dq[i];
    e1 = fmaf(dr, a1[i], e1);
    e2 = fmaf(dr, a2[i], e2);
    g2 = fmaf(d, a2[i], g2);
  }
  // minus the row terms without the branch factor: D_b = c_b * Dt_b with Dt_b = dO . O_b,
  // c_1 = 1, c_2 = -lambda (the consumers start an accumulator at -Dt_b)
  nd1 = -row16_sum(e1);
  nd2 = -row16_sum(e2);
  ndl = -row16_sum(g2);
}

// ---------------------------------------------------------------------------------------------
// dK_1, dK_2, dV: per 64 keys of a head, 16 per wave, both branches in each wave
// LDS layouts of the dK/dV kernel's tiles, each read both row by row (16x16x32 MFMA A operand:
// lane n of each 16-lane group takes row n, the group index picks the 16-byte chunk) and
// transposed (ds_read_b64_tr_b16: 8 rows of 32 bytes per 32-lane half).  The 16-byte chunk index
// is XORed with the row's low three bits (Q tiles, 8 chunks per row) or with twice them (dO,
// 16 chunks per row).  Both read patterns of both tiles then measure free of bank conflicts
// (SQ_LDS_BANK_CONFLICT = 0 on gfx950, in an access-pattern probe); the earlier choices, which
// also folded row bit 3 into the chunk index, were 2-way conflicted on the row-wise reads.
__device__ __forceinline__ int q16_swz(int row) { return row & 7; }
__device__ __forceinline__ int q16_off(int row, int col) {
  return row * kD + ((((col >> 3) ^ q16_swz(row))) << 3) + (col & 7);
}
__device__ __forceinline__ int o16_swz(int row) { return (row & 7) << 1; }
__device__ __forceinline__ int o16_off(int row, int col) {
  return row * kDV + ((((col >> 3) ^ o16_swz(row))) << 3) + (col & 7);
}

__global__ __launch_bounds__(kThreads) void bwd_dkdv_kernel(const BwdParams p) {
  // (One wave per 16 keys with both branches, on 16x16x32 MFMAs: X = dO V^T and the dV product
  // are formed once for the two branches -- 32 MFMAs of 16x16x32 per 16 keys and query tile
  // instead of 48 of the 32x32x16 shape per 32 keys for one branch, i.e. a third fewer MFMA
  // cycles; measured 7 % faster for the whole backward.)
  // per stage: Q_1, Q_2 [32][64], dO [32][128], then LSE_1, LSE_2, -Dt_1, -Dt_2 [32] (+ 1 KB for
  // the row data: one wavefront DMA writes 64 x 16 bytes, of which the first 512 hold them; the
  // rest read past the buffer's end and land as zeros)
  constexpr int QT = kT * kD;
  constexpr int OT = kT * kDV;
  constexpr int STAGE = 2 * QT + OT + 512;
  __shared__ __attribute__((aligned(1024))) bf16 smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g = lane >> 4;       // MFMA 16x16x32: column / row group
  int bh, kb;
  chunked_block(p.head_chunk, p.n_row_blocks, bh, kb);  // heads in chunks, see chunked_block
  const int b = bh / p.H, h = bh % p.H;
  const int key0 = kb * 64;                       // heaviest (earliest keys) first
  const int kw = key0 + 16 * w;                   // this wave's 16 keys, both branches
  const int N = p.N;
  const float lam = lam_of(p, h, lane);
  const float sl2 = p.scale_log2;
  const int64_t BHN = (int64_t)p.B * p.H * N;
  const int W = p.window;

  // K_1^T, K_2^T, V^T as B operands: lane n = key kw + n16, k = 32 ks + 8 g .. + 7
  bf16x8 kf1[2], kf2[2], vf[4];
  {
    const bf16* k1b = static_cast<const bf16*>(p.k1) + b * p.sk1.sb + h * p.sk1.sh;
    const bf16* k2b = static_cast<const bf16*>(p.k2) + b * p.sk2.sb + h * p.sk2.sh;
    const bf16* vb = static_cast<const bf16*>(p.v) + b * p.sv.sb + h * p.sv.sh;
    const __amdgpu_buffer_rsrc_t rk1 = make_rsrc(k1b, (uint32_t)(N * p.sk1.sn * 2));
    const __amdgpu_buffer_rsrc_t rk2 = make_rsrc(k2b, (uint32_t)(N * p.sk2.sn * 2));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, (uint32_t)(N * p.sv.sn * 2));
    const uint32_t key = (uint32_t)(kw + n16);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      kf1[ks] = __builtin_bit_cast(bf16x8, bload16(rk1, key * (uint32_t)(p.sk1.sn * 2) + 64 * ks + 16 * g));
      kf2[ks] = __builtin_bit_cast(bf16x8, bload16(rk2, key * (uint32_t)(p.sk2.sn * 2) + 64 * ks + 16 * g));
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      vf[ks] = __builtin_bit_cast(bf16x8, bload16(rv, key * (uint32_t)(p.sv.sn * 2) + 64 * ks + 16 * g));
    __builtin_amdgcn_s_waitcnt(0);  // settle before the asm tile DMA starts
  }

  // ---- query tiles: DMA of Q_1 / Q_2 (1 KB each per wave), dO (2 KB per wave), row data
  const uint32_t q1_row = (uint32_t)(p.sq1.sn * 2), q2_row = (uint32_t)(p.sq2.sn * 2);
  const char* q1_base = static_cast<const char*>(p.q1) + 2 * (b * p.sq1.sb + h * p.sq1.sh);
  const char* q2_base = static_cast<const char*>(p.q2) + 2 * (b * p.sq2.sb + h * p.sq2.sh);
  const char* do_base = static_cast<const char*>(p.d_o) + (int64_t)bh * N * kDV * 2;
  int q_lrow;
  uint32_t q_lchunk, o_lane[2];
  {
    const int e = 512 * w + 8 * lane;
    q_lrow = e / kD;
    q_lchunk = (uint32_t)((((e % kD) >> 3) ^ q16_swz(q_lrow)) * 16);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ev = 512 * (w + 4 * i) + 8 * lane;
      const int vrow = ev >> 7;
      const int slot = (ev & 127) >> 3;
      o_lane[i] = (uint32_t)vrow * (kDV * 2) + (uint32_t)((slot ^ o16_swz(vrow)) << 4);
    }
  }
  const __amdgpu_buffer_rsrc_t r_ld = make_rsrc(p.lse_d, (uint32_t)(4 * BHN * 4));
  auto issue_tile = [&](int q0, int buf) __attribute__((always_inline)) {
    bf16* st = smem + buf * STAGE;
    const int rows_left = N - q0;
    const __amdgpu_buffer_rsrc_t r1 = make_rsrc(q1_base + (size_t)q0 * q1_row, (uint32_t)rows_left * q1_row);
    const __amdgpu_buffer_rsrc_t r2 = make_rsrc(q2_base + (size_t)q0 * q2_row, (uint32_t)rows_left * q2_row);
    dma16(r1, st + 512 * w, (uint32_t)q_lrow * q1_row + q_lchunk);
    dma16(r2, st + QT + 512 * w, (uint32_t)q_lrow * q2_row + q_lchunk);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(do_base + (size_t)q0 * kDV * 2, (uint32_t)rows_left * kDV * 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(ro, st + 2 * QT + 512 * (w + 4 * i), o_lane[i]);
    if (w == 0) {
      // lanes 0..31: 16 bytes of LSE_1, LSE_2, -Dt_1, -Dt_2 for rows q0 .. q0+31; the rest read
      // past the buffer's end and land as zeros
      const int k = lane >> 3, piece = lane & 7;
      const uint32_t off = lane < 32 ? (uint32_t)((((int64_t)k * BHN + (int64_t)bh * N + q0) * 4) + piece * 16)
                                     : (uint32_t)(4 * BHN * 4);
      dma16(r_ld, st + 2 * QT + OT, off);
    }
  };

  // accumulators: dV^T [128 ch x 16 keys] (8 tiles), dK_b^T [64 d x 16 keys] (4 tiles each);
  // lane: key kw + n16, rows (ch or d) 16 t + 4 g + r
  f32x4 dv[8], dk1[4], dk2[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) dv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) { dk1[i] = f32x4{0.f, 0.f, 0.f, 0.f}; dk2[i] = f32x4{0.f, 0.f, 0.f, 0.f}; }

  // LDS element offsets within a stage.  Row-wise A operands (rows 16 j + n16, chunk 4 ks + g):
  // base XOR 32 ks (Q) / 32 ks (dO, in 16-element units per ks step of 32 columns).
  const int qa_rd = q16_off(n16, 8 * g);
  const int oa_rd = o16_off(n16, 8 * g);
  // transposed reads: lane n16 of group g addresses row 4 g + n16 / 4 (+ 16 for the upper half),
  // columns 16 t + 4 (n16 % 4); it receives column 16 t + n16 of those four rows
  const int tr_row = 4 * g + (n16 >> 2), tr_col = 4 * (n16 & 3);

  const int qt_begin = p.causal ? key0 / kT : 0;
  const int nq = W > 0 ? min((N + kT - 1) / kT, (key0 + 63 + W - 1) / kT + 1) : (N + kT - 1) / kT;
  const int qt_wave = p.causal ? kw / kT : 0;
  const int qt_wave_end = W > 0 ? (kw + 15 + W - 1) / kT + 1 : nq;
  const bool wave_has_keys = kw < N;

  // MASK: the tile holds a query before the diagonal or past N, a key past N, or a pair outside
  // the window (wave-uniform); BUF: the stage buffer, a compile-time constant
  auto compute = [&](int qt, auto buf_tag, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const bf16* st = smem + decltype(buf_tag)::value * STAGE;
    const float* rowd = reinterpret_cast<const float*>(st + 2 * QT + OT);  // [4][32]
    const int q0 = qt * kT;
    // S_b [q][key] and X = dO V^T [q][key] per 16-row half j: lane key kw + n16, rows 4 g + r
    f32x4 s1[2], s2[2], x[2];
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      s1[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      s2[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      x[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int off = (qa_rd ^ (32 * ks)) + 16 * j * kD;
        s1[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(st + off), kf1[ks], s1[j], 0, 0, 0);
        s2[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(st + QT + off), kf2[ks], s2[j], 0, 0, 0);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int off = (oa_rd ^ (32 * ks)) + 16 * j * kDV;
        x[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(st + 2 * QT + off), vf[ks], x[j], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // P_b, dS_b / c_b = P_b (X - Dt_b), and P' = P_1 - lambda P_2 for dV
    float pc[2][4], d1[2][4], d2[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int ql = 16 * j + 4 * g;
      const f32x4 lse1 = *reinterpret_cast<const f32x4*>(rowd + ql);
      const f32x4 lse2 = *reinterpret_cast<const f32x4*>(rowd + kT + ql);
      const f32x4 nd1 = *reinterpret_cast<const f32x4*>(rowd + 2 * kT + ql);
      const f32x4 nd2 = *reinterpret_cast<const f32x4*>(rowd + 3 * kT + ql);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float e1 = fmaf(s1[j][r], sl2, -lse1[r]);
        float e2 = fmaf(s2[j][r], sl2, -lse2[r]);
        if constexpr (MASK) {
          const int q = q0 + ql + r, key = kw + n16;
          const bool vis = q < N && key < N && (!p.causal || key <= q) && (W == 0 || q - key < W);
          e1 = vis ? e1 : -INFINITY;
          e2 = vis ? e2 : -INFINITY;
        }
        const float p1 = __builtin_amdgcn_exp2f(e1);
        const float p2 = __builtin_amdgcn_exp2f(e2);
        pc[j][r] = fmaf(-lam, p2, p1);
        d1[j][r] = p1 * (x[j][r] + nd1[r]);
        d2[j][r] = p2 * (x[j][r] + nd2[r]);
      }
    }
    // B operands: lane key kw + n16, k = 8 g + i <-> query 4 g + i (i < 4) / 16 + 4 g + i - 4
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    auto pack = [](const float (&v)[2][4]) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x2 hv = {(bf16)v[i >> 1][2 * (i & 1)], (bf16)v[i >> 1][2 * (i & 1) + 1]};
        o[i] = __builtin_bit_cast(uint32_t, hv);
      }
      return __builtin_bit_cast(bf16x8, o);
    };
    const bf16x8 pb = pack(pc), sb1 = pack(d1), sb2 = pack(d2);
    __builtin_amdgcn_s_setprio(1);
    // dV^T += dO^T P' (8 channel tiles), dK_b^T += Q_b^T (dS_b / c_b) (4 d tiles each)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const u32x2 lo = lds_read_tr(st + 2 * QT + o16_off(tr_row, 16 * t + tr_col));
      const u32x2 hi = lds_read_tr(st + 2 * QT + o16_off(16 + tr_row, 16 * t + tr_col));
      const u32x4 a4 = {lo[0], lo[1], hi[0], hi[1]};
      dv[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a4), pb, dv[t], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const u32x2 lo1 = lds_read_tr(st + q16_off(tr_row, 16 * t + tr_col));
      const u32x2 hi1 = lds_read_tr(st + q16_off(16 + tr_row, 16 * t + tr_col));
      const u32x4 a1 = {lo1[0], lo1[1], hi1[0], hi1[1]};
      dk1[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1), sb1, dk1[t], 0, 0, 0);
      const u32x2 lo2 = lds_read_tr(st + QT + q16_off(tr_row, 16 * t + tr_col));
      const u32x2 hi2 = lds_read_tr(st + QT + q16_off(16 + tr_row, 16 * t + tr_col));
      const u32x4 a2 = {lo2[0], lo2[1], hi2[0], hi2[1]};
      dk2[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a2), sb2, dk2[t], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  issue_tile(qt_begin * kT, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  auto step = [&](int qt, auto buf_tag, auto mask_tag) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_tag)::value;
    if (qt + 1 < nq) issue_tile((qt + 1) * kT, BUF ^ 1);
    if (wave_has_keys && qt >= qt_wave && qt < qt_wave_end) compute(qt, buf_tag, mask_tag);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  auto run = [&](int qa, int qb, auto mask_tag) __attribute__((always_inline)) {
    int qt = qa;
    if (qt < qb && ((qt - qt_begin) & 1) != 0) step(qt++, std::integral_constant<int, 1>{}, mask_tag);
    for (; qt + 1 < qb; qt += 2) {
      step(qt, std::integral_constant<int, 0>{}, mask_tag);
      step(qt + 1, std::integral_constant<int, 1>{}, mask_tag);
    }
    if (qt < qb) step(qt, std::integral_constant<int, 0>{}, mask_tag);
  };
  const bool keys_full = key0 + 64 <= N;
  const int fa = keys_full ? min(nq, p.causal ? qt_begin + 2 : qt_begin) : nq;
  int fb = keys_full ? max(fa, N / kT) : nq;
  if (W > 0) fb = max(fa, min(fb, key0 + W - kT >= 0 ? (key0 + W - kT) / kT + 1 : 0));
  run(qt_begin, fa, std::true_type{});
  run(fa, fb, std::false_type{});
  run(fb, nq, std::true_type{});

  // ---- epilogue: dK_b (times c_b / sqrt(d)) and dV, lane key kw + n16, rows 16 t + 4 g + r
  const int key = kw + n16;
  if (!wave_has_keys || key >= N) return;
  float* dk1p = p.dk1 + ((int64_t)bh * N + key) * kD;
  float* dk2p = p.dk2 + ((int64_t)bh * N + key) * kD;
  float* dvp = p.dv + ((int64_t)bh * N + key) * kDV;
  const float ks1 = p.scale, ks2 = -lam * p.scale;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    *reinterpret_cast<f32x4*>(dk1p + 16 * t + 4 * g) = dk1[t] * ks1;
    *reinterpret_cast<f32x4*>(dk2p + 16 * t + 4 * g) = dk2[t] * ks2;
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) *reinterpret_cast<f32x4*>(dvp + 16 * t + 4 * g) = dv[t];
}

// ---------------------------------------------------------------------------------------------
// dQ_1, dQ_2: per 128 query rows, 32 per wave, both branches in each wave
// LDS layout of the dQ kernel's K tiles (32 rows x 64 columns), read row by row (lane c = lane %
// 32 takes row c, lane / 32 the 16-byte chunk) and transposed (ds_read_b64_tr_b16, four 4-row
// groups of 16-byte runs per 32-lane half).  The chunk index is XORed with a linear function of
// row bits 1-3 (6 r1 ^ 2 r2 ^ 3 r3) that keeps both patterns free of bank conflicts (measured
// SQ_LDS_BANK_CONFLICT = 0 in an access-pattern probe; the forward's (row >> 1) & 7 layout is
// 2-way conflicted on these transposed reads).
__device__ __forceinline__ int kq_swz(int row) {
  return (((row >> 1) & 1) * 6) ^ (((row >> 2) & 1) * 2) ^ (((row >> 3) & 1) * 3);
}
__device__ __forceinline__ int kq_off(int row, int col) {
  return row * kD + ((((col >> 3) ^ kq_swz(row))) << 3) + (col & 7);
}

__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(const BwdParams p) {
  constexpr int KT = kT * kD;                  // one K tile
  constexpr int STAGE = 2 * KT + kT * kDV;     // K_1 | K_2 | V
  constexpr int BR = 128;                      // query rows per workgroup (32 per wave)
  // (both branches in one wave share X^T = V dO^T: 24 MFMAs per key tile for the two branches
  // instead of 32, at 2 waves/SIMD instead of 3; measured 6 % faster for the whole backward)
  // (+ 1 KB: the prologue's -Dt_1, -Dt_2 of the workgroup's rows, behind its 32 KB dO tile)
  static_assert(2 * STAGE >= 4 * 32 * kDV, "the prologue's dO tile fits the stage buffers");
  __shared__ __attribute__((aligned(1024))) bf16 smem[2 * STAGE + 512];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, hh = lane >> 5;
  const int N = p.N;
  const int nrb = (N + BR - 1) / BR;
  int bh, rb;
  chunked_block(p.head_chunk, nrb, bh, rb);  // heads in chunks, see chunked_block
  rb = nrb - 1 - rb;                         // heaviest first
  const int b = bh / p.H, h = bh % p.H;
  const int row0 = rb * BR;
  const int wrow = row0 + 32 * w;
  const float lam = lam_of(p, h, lane);
  const float sl2 = p.scale_log2;
  const int64_t BHN = (int64_t)p.B * p.H * N;
  const bool wave_has_rows = wrow < N;
  const int qrow = wrow + c;
  const int W = p.window;

  // Q_1^T, Q_2^T and dO^T as B operands: lane n = query wrow + c, k = 16 t + 8 hh .. + 7; the
  // lane's row statistics LSE_b and -Dt_b
  bf16x8 qf1[kD / 16], qf2[kD / 16], of[kDV / 16];
  float lse1 = 0.f, lse2 = 0.f, ndd1 = 0.f, ndd2 = 0.f;
  {
    const bf16* qb1 = static_cast<const bf16*>(p.q1) + b * p.sq1.sb + h * p.sq1.sh;
    const bf16* qb2 = static_cast<const bf16*>(p.q2) + b * p.sq2.sb + h * p.sq2.sh;
    const __amdgpu_buffer_rsrc_t rq1 = make_rsrc(qb1, (uint32_t)(N * p.sq1.sn * 2));
    const __amdgpu_buffer_rsrc_t rq2 = make_rsrc(qb2, (uint32_t)(N * p.sq2.sn * 2));
#pragma unroll
    for (int t = 0; t < kD / 16; ++t) {
      qf1[t] = __builtin_bit_cast(bf16x8, bload16(rq1, (uint32_t)(qrow * p.sq1.sn * 2) + 32 * t + 16 * hh));
      qf2[t] = __builtin_bit_cast(bf16x8, bload16(rq2, (uint32_t)(qrow * p.sq2.sn * 2) + 32 * t + 16 * hh));
    }
    // dO through the norm for this wave's 32 rows (the backward's first step, done where the rows
    // are used first): 4 rows per pass, 16 lanes per row; dO, -Dt_1, -Dt_2 and the dlambda share
    // go to memory for the dK/dV kernel, and through LDS into this wave's operand layout
    // [32][128] bf16, 16-byte chunk k of row r at chunk k ^ (r & 15), so that the operand reads
    // (one chunk of 32 rows at a time) spread over the banks
    bf16* do_lds = smem + w * (32 * kDV);
    float* dt_lds = reinterpret_cast<float*>(smem + 4 * 32 * kDV) + w * 64;  // [32][2]
    {
      const int sub = lane & 15;
#pragma unroll
      for (int half = 0; half < 8 / kPrepGroup; ++half) {
      // the loads of kPrepGroup passes, then their arithmetic (2 measured best of 1, 2, 4, 8)
      PrepIn in[kPrepGroup];
#pragma unroll
      for (int j = 0; j < kPrepGroup; ++j) {
        const int row = wrow + 4 * (kPrepGroup * half + j) + (lane >> 4);
        const int rc = min(row, N - 1);
        in[j] = prep_load(p, b, h, (int64_t)bh * N + rc, rc, sub, BHN);
      }
#pragma unroll
      for (int j = 0; j < kPrepGroup; ++j) {
        const int it = kPrepGroup * half + j;
        const int lr = 4 * it + (lane >> 4);  // row within the wave
        const int row = wrow + lr;
        // rows past N compute on row N-1 (so every lane of a group takes part) and store nothing
        const int rc = min(row, N - 1);
        const int64_t r = (int64_t)bh * N + rc;
        bf16x8 d8;
        float nd1, nd2, ndl;
        prep_row(p, in[j], lam, d8, nd1, nd2, ndl);
        *reinterpret_cast<bf16x8*>(do_lds + lr * kDV + 8 * (sub ^ (lr & 15))) = d8;
        if (sub == 0) {
          dt_lds[2 * lr] = nd1;
          dt_lds[2 * lr + 1] = nd2;
        }
        if (row < N) {
          *reinterpret_cast<bf16x8*>(static_cast<bf16*>(p.d_o) + r * kDV + 8 * sub) = d8;
          if (sub == 0) {
            p.lse_d[2 * BHN + r] = nd1;
            p.lse_d[3 * BHN + r] = nd2;
            p.dl_row[r] = ndl;
          }
        }
      }
      }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kDV / 16; ++t)
      of[t] = *reinterpret_cast<const bf16x8*>(do_lds + c * kDV + 8 * ((2 * t + hh) ^ (c & 15)));
    ndd1 = dt_lds[2 * c];
    ndd2 = dt_lds[2 * c + 1];
    __syncthreads();  // every wave has its operands before the tile loads reuse the buffers
    if (qrow < N) {
      const int64_t r = (int64_t)bh * N + qrow;
      lse1 = p.lse_d[r];
      lse2 = p.lse_d[BHN + r];
    }
    __builtin_amdgcn_s_waitcnt(0);
  }

  const uint32_t k1_row = (uint32_t)(p.sk1.sn * 2), k2_row = (uint32_t)(p.sk2.sn * 2);
  const uint32_t v_row = (uint32_t)(p.sv.sn * 2);
  const char* k1_base = static_cast<const char*>(p.k1) + 2 * (b * p.sk1.sb + h * p.sk1.sh);
  const char* k2_base = static_cast<const char*>(p.k2) + 2 * (b * p.sk2.sb + h * p.sk2.sh);
  const char* v_base = static_cast<const char*>(p.v) + 2 * (b * p.sv.sb + h * p.sv.sh);
  int k_lrow;
  uint32_t k_lchunk, v_lane[2];
  {
    const int e = 512 * w + 8 * lane;
    k_lrow = e / kD;
    k_lchunk = (uint32_t)((((e % kD) >> 3) ^ kq_swz(k_lrow)) * 16);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ev = 512 * (w + 4 * i) + 8 * lane;
      const int vrow = ev >> 7;
      const int slot = (ev & 127) >> 3;
      v_lane[i] = (uint32_t)vrow * v_row + (uint32_t)((slot ^ k_swz<kDV>(vrow)) << 4);
    }
  }
  auto issue_tile = [&](int k0, int buf) __attribute__((always_inline)) {
    bf16* st = smem + buf * STAGE;
    const int rows_left = N - k0;
    const __amdgpu_buffer_rsrc_t r1 = make_rsrc(k1_base + (size_t)k0 * k1_row, (uint32_t)rows_left * k1_row);
    const __amdgpu_buffer_rsrc_t r2 = make_rsrc(k2_base + (size_t)k0 * k2_row, (uint32_t)rows_left * k2_row);
    dma16(r1, st + 512 * w, (uint32_t)k_lrow * k1_row + k_lchunk);
    dma16(r2, st + KT + 512 * w, (uint32_t)k_lrow * k2_row + k_lchunk);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(v_base + (size_t)k0 * v_row, (uint32_t)rows_left * v_row);
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(rv, st + 2 * KT + 512 * (w + 4 * i), v_lane[i]);
  };

  f32x16 dq1[2], dq2[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dq1[i][r] = 0.f; dq2[i][r] = 0.f; }

  const int k_rd = kq_off(c, 8 * hh);
  // the V tile is only read row by row here, so it takes the 128-column K-tile layout, whose
  // row-wise reads are free of bank conflicts
  const int v_rd = k_off<kDV>(c, 8 * hh);
  const int jj = lane & 15, dh = (lane >> 4) & 1;
  const int trow = 4 * hh + (jj >> 2);
  const int tcol = dh * 16 + 4 * (jj & 3);

  // MASK: the tile holds a key past the diagonal, outside the window or past N, or a row past N
  // (wave-uniform); BUF: the stage buffer, a compile-time constant (see the dK/dV kernel)
  auto compute = [&](int kt, auto buf_tag, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const bf16* st = smem + decltype(buf_tag)::value * STAGE;
    const int k0 = kt * kT;
    f32x16 s1, s2, x;
#pragma unroll
    for (int r = 0; r < 16; ++r) { s1[r] = 0.f; s2[r] = 0.f; x[r] = 0.f; }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int t = 0; t < kD / 16; ++t) {
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(st + (k_rd ^ (16 * t))), qf1[t], s1, 0, 0, 0);
      s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(st + KT + (k_rd ^ (16 * t))), qf2[t], s2, 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < kDV / 16; ++t) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(st + 2 * KT + (v_rd ^ (16 * t)));
      x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, of[t], x, 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    // registers r: key k0 + 8 (r/4) + 4 hh + r % 4; query qrow.  dS_b^T / c_b = P_b^T (X^T - Dt_b)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float e1 = fmaf(s1[r], sl2, -lse1);
      float e2 = fmaf(s2[r], sl2, -lse2);
      if constexpr (MASK) {
        const int key = k0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        const bool vis = key < N && qrow < N && (!p.causal || key <= qrow) && (W == 0 || qrow - key < W);
        e1 = vis ? e1 : -INFINITY;
        e2 = vis ? e2 : -INFINITY;
      }
      s1[r] = __builtin_amdgcn_exp2f(e1) * (x[r] + ndd1);
      s2[r] = __builtin_amdgcn_exp2f(e2) * (x[r] + ndd2);
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float dummy = 0.f;
      const bf16x8 sb1 = cvt8_sum(s1, 8 * u, dummy);
      const bf16x8 sb2 = cvt8_sum(s2, 8 * u, dummy);
#pragma unroll
      for (int dbk = 0; dbk < 2; ++dbk) {
        const u32x2 lo1 = lds_read_tr(st + kq_off(16 * u + trow, 32 * dbk + tcol));
        const u32x2 hi1 = lds_read_tr(st + kq_off(16 * u + 8 + trow, 32 * dbk + tcol));
        const u32x4 a1 = {lo1[0], lo1[1], hi1[0], hi1[1]};
        dq1[dbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a1), sb1, dq1[dbk], 0, 0, 0);
        const u32x2 lo2 = lds_read_tr(st + KT + kq_off(16 * u + trow, 32 * dbk + tcol));
        const u32x2 hi2 = lds_read_tr(st + KT + kq_off(16 * u + 8 + trow, 32 * dbk + tcol));
        const u32x4 a2 = {lo2[0], lo2[1], hi2[0], hi2[1]};
        dq2[dbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a2), sb2, dq2[dbk], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // key tiles: up to the block's last row (causal); from the first key its first row sees through
  // the window; each wave computes its own sub-range and otherwise only helps load
  const int kv_end = p.causal ? min(N, row0 + BR) : N;
  const int ntiles = (kv_end + kT - 1) / kT;
  const int last_key = p.causal ? min(N, wrow + 32) : N;
  const int nt_wave = wave_has_rows ? min(ntiles, (last_key + kT - 1) / kT) : 0;
  const int kt_begin = W > 0 ? max(0, row0 - W + 1) / kT : 0;
  const int kt_wave = W > 0 ? max(0, wrow - W + 1) / kT : 0;
  issue_tile(kt_begin * kT, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // key tile kt sits in buffer (kt - kt_begin) & 1; two tiles per iteration keep the buffer index
  // static
  auto step = [&](int kt, auto buf_tag, auto mask_tag) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_tag)::value;
    if (kt + 1 < ntiles) issue_tile((kt + 1) * kT, BUF ^ 1);
    if (kt >= kt_wave && kt < nt_wave) compute(kt, buf_tag, mask_tag);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  auto run = [&](int ka, int kb, auto mask_tag) __attribute__((always_inline)) {
    int kt = ka;
    if (kt < kb && ((kt - kt_begin) & 1) != 0) step(kt++, std::integral_constant<int, 1>{}, mask_tag);
    for (; kt + 1 < kb; kt += 2) {
      step(kt, std::integral_constant<int, 0>{}, mask_tag);
      step(kt + 1, std::integral_constant<int, 1>{}, mask_tag);
    }
    if (kt < kb) step(kt, std::integral_constant<int, 0>{}, mask_tag);
  };
  // Key tiles [fs, fe) need no mask for any wave: their keys precede every row of the block
  // (causal), every row is inside N, and (window) the block's last row still sees their first
  // key, k0 >= row0 + BR - W.  The band's lower edge, the diagonal and the tail run masked.
  const int fe = row0 + BR <= N ? (p.causal ? row0 / kT : N / kT) : 0;
  const int fs = W > 0 ? min(max(kt_begin, (row0 + BR - W + kT - 1 >= 0 ? (row0 + BR - W + kT - 1) / kT : 0)), max(kt_begin, fe))
                       : 0;
  run(kt_begin, fs, std::true_type{});
  run(fs, max(fs, fe), std::false_type{});
  run(max(fs, fe), ntiles, std::true_type{});
  if (!wave_has_rows || qrow >= N) return;
  // dQ_b = c_b dS_b K_b / sqrt(d), c_1 = 1, c_2 = -lambda
  float* dqp1 = p.dq1 + ((int64_t)bh * N + qrow) * kD;
  float* dqp2 = p.dq2 + ((int64_t)bh * N + qrow) * kD;
  const float qs1 = p.scale, qs2 = -lam * p.scale;
#pragma unroll
  for (int dbk = 0; dbk < 2; ++dbk)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 v1 = {dq1[dbk][4 * j] * qs1, dq1[dbk][4 * j + 1] * qs1, dq1[dbk][4 * j + 2] * qs1, dq1[dbk][4 * j + 3] * qs1};
      *reinterpret_cast<f32x4*>(dqp1 + dbk * 32 + 8 * j + 4 * hh) = v1;
      const f32x4 v2 = {dq2[dbk][4 * j] * qs2, dq2[dbk][4 * j + 1] * qs2, dq2[dbk][4 * j + 2] * qs2, dq2[dbk][4 * j + 3] * qs2};
      *reinterpret_cast<f32x4*>(dqp2 + dbk * 32 + 8 * j + 4 * hh) = v2;
    }
}

// ---------------------------------------------------------------------------------------------
// dlambda per head and the four vector gradients
constexpr int kLambdaThreads = 1024;
constexpr int kLambdaBatch = 8;  // row shares per thread loaded at once

__global__ __launch_bounds__(kLambdaThreads) void bwd_lambda_kernel(const BwdParams p) {
  __shared__ float part[kLambdaThreads / 64];
  const int h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // this thread's shares in the order (batch, row tid + r kLambdaThreads), loaded kLambdaBatch at a
  // time so that their loads are in flight together, and added in that order
  float s = 0.f;
  const int per_b = tid < p.N ? (p.N - tid + kLambdaThreads - 1) / kLambdaThreads : 0;
  const int tot = p.B * per_b;
  for (int t0 = 0; t0 < tot; t0 += kLambdaBatch) {
    float v[kLambdaBatch];
#pragma unroll
    for (int j = 0; j < kLambdaBatch; ++j) {
      v[j] = 0.f;
      const int t = t0 + j;
      if (t < tot) {
        const int b = t / per_b, r = t - b * per_b;
        v[j] = p.dl_row[((int64_t)b * p.H + h) * p.N + tid + r * kLambdaThreads];
      }
    }
#pragma unroll
    for (int j = 0; j < kLambdaBatch; ++j)
      if (t0 + j < tot) s += v[j];
  }
  s = wave_sum(s);
  if (lane == 0) part[w] = s;
  __syncthreads();
  if (w != 0) return;
  const float dlam = wave_sum(lane < kLambdaThreads / 64 ? part[lane] : 0.f);
  const LambdaArgs& L = p.lam;
  if (L.override_ != nullptr) return;  // lambda given directly: no vector gradients
  const int64_t base = (int64_t)h * L.dl;
  float a = 0.f, c2 = 0.f;
  for (int e = lane; e < L.dl; e += 64) {
    a = fmaf(L.lq1[base + e], L.lk1[base + e], a);
    c2 = fmaf(L.lq2[base + e], L.lk2[base + e], c2);
  }
  const float ea = expf(wave_sum(a)), eb = expf(wave_sum(c2));
  for (int e = lane; e < L.dl; e += 64) {
    p.dlq1[base + e] = dlam * ea * L.lk1[base + e];
    p.dlk1[base + e] = dlam * ea * L.lq1[base + e];
    p.dlq2[base + e] = -dlam * eb * L.lk2[base + e];
    p.dlk2[base + e] = -dlam * eb * L.lq2[base + e];
  }
}

}  // namespace

hipError_t launch_bwd_v1(const BwdParams& p, hipStream_t stream) {
  BwdParams q = p;
  q.n_row_blocks = (p.N + 63) / 64;
  // a head's streamed tiles: Q_1, Q_2, dO and four row terms (dK/dV); K_1, K_2, V (dQ)
  q.head_chunk = head_chunk((int64_t)p.B * p.H, (int64_t)p.N * (2 * kD * 2 + kDV * 2 + 16));
  // dQ first: its workgroups also form dO and the row terms the dK/dV kernel reads
  hipLaunchKernelGGL(bwd_dq_kernel, dim3(p.B * p.H, (p.N + 127) / 128), dim3(kThreads), 0, stream, q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dkdv_kernel, dim3(p.B * p.H, q.n_row_blocks), dim3(kThreads), 0, stream, q);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_lambda_kernel, dim3(p.H), dim3(kLambdaThreads), 0, stream, q);
  return hipGetLastError();
}

}  // namespace da
