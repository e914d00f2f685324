// One V1 decode step for gfx950: every sequence's new query token attends to its whole cache.
//
// What is computed (Ultralytics glossary "Differential Transformer", section "Cómo funciona la
// atención diferencial"; ai-engineering.academy "Atención Diferencial (V2)", section "V1 vs V2:
// la diferencia"): per head h the new token's two query halves q1, q2 (d = 64) score against
// the cached key halves K1, K2, and
//   out_h = (1 - lambda_init) RMSnorm( softmax(q1 K1^T / sqrt(d)) V - lambda_h softmax(q2 K2^T / sqrt(d)) V )
// with V twice as wide (2d = 128).  The page's remark on V1 decode is that the value cache is
// needed by both softmax branches; here each K1, K2 and V byte is read exactly once per step and
// one pass over V feeds both branches.
//
// Bandwidth-bound design (split-K over the cache, then a log-sum-exp merge):
//  * decode_v1_partial: one 256-thread workgroup per (split s, head h, batch b) streams keys
//    [s*chunk, min(L, (s+1)*chunk)) in blocks of 256 (64 per wavefront), with every K1, K2 and V
//    load of a block issued before its arithmetic:
//      - scores with v_mfma_f32_16x16x32_bf16: the A operand holds the branch's query in row 0
//        (rows 1..15 zero), the B operand takes K rows straight from global memory;
//      - one wavefront per branch takes the block max / exp2 / sum over the 256 scores in LDS;
//      - P.V on the vector ALUs: 16 lanes cover one 256-byte V row (8 channels each) and read
//        the key's two branch weights as one LDS broadcast;
//    it writes, per branch, the split's (running max, running sum, un-normalised accumulator).
//  * decode_v1_combine: per (head, batch) merges the splits of each branch by log-sum-exp,
//    forms O = O_1 - lambda O_2, applies the RMS norm over the 128 channels and the
//    (1 - lambda_init) scale, and stores bf16.
#include "device_common.hpp"
#include "launch.hpp"

namespace da {
namespace {

constexpr int kDQK = 64;   // query / key half width
constexpr int kDV = 128;   // value width
constexpr int kKB = 256;   // keys per block (64 per wavefront)
constexpr int kThreads = 256;
constexpr float kNegBig = -1.0e30f;
constexpr int kCombineBatch = 8;  // split partials per branch that the combine loads at once

__global__ __launch_bounds__(kThreads) void decode_v1_partial_kernel(const DecodeV1Params p) {
  __shared__ float sc_lds[2][kKB];                               // scores of the block, per branch
  __shared__ __attribute__((aligned(8))) float pw_lds[kKB][2];   // exp-weights, per key
  __shared__ float alpha_lds[2];
  __shared__ float red_lds[4][2][kDV];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int l16 = lane & 15;
  const int grp = lane >> 4;

  const int k_begin = split * p.chunk;
  const int k_end = min(p.L, k_begin + p.chunk);
  const float c2 = p.scale_log2;

  const bf16* kb[2] = {static_cast<const bf16*>(p.k1) + b * p.sk1.sb + h * p.sk1.sh,
                       static_cast<const bf16*>(p.k2) + b * p.sk2.sb + h * p.sk2.sh};
  const int64_t ksn[2] = {p.sk1.sn, p.sk2.sn};
  const bf16* vbase = static_cast<const bf16*>(p.v) + b * p.sv.sb + h * p.sv.sh;

  // A operands: row m = l16 (only row 0 is the query), k = 32t + 8*grp + i
  bf16x8 qa[2][2];
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const bf16* q[2] = {static_cast<const bf16*>(p.q1) + b * p.sq1.sb + h * p.sq1.sh,
                        static_cast<const bf16*>(p.q2) + b * p.sq2.sb + h * p.sq2.sh};
#pragma unroll
    for (int br = 0; br < 2; ++br)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        qa[br][t] = __builtin_bit_cast(bf16x8, l16 == 0 ? load16(q[br] + 32 * t + 8 * grp) : z);
  }

  float mrun = kNegBig, lrun = 0.f;  // softmax state of branch w (wavefronts 0 and 1)
  float acc[2][8];
#pragma unroll
  for (int br = 0; br < 2; ++br)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[br][e] = 0.f;

  // A block's K1, K2 rows are loaded while the block before it finishes, into the registers its
  // score products are done with, as soon as they are; V at the block's start
  u32x4 kf[2][4][2];
  auto load_k = [&](int blk) {
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      const int key = blk + 64 * w + 16 * sb + l16;
#pragma unroll
      for (int br = 0; br < 2; ++br)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          kf[br][sb][t] = key < k_end ? load16_nt(kb[br] + (int64_t)key * ksn[br] + 32 * t + 8 * grp)
                                      : u32x4{0u, 0u, 0u, 0u};
    }
  };
  if (k_begin < k_end) load_k(k_begin);
  for (int blk = k_begin; blk < k_end; blk += kKB) {
    u32x4 vf[16];
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int key = blk + 64 * w + 4 * st + grp;
      vf[st] = key < k_end ? load16_nt(vbase + (int64_t)key * p.sv.sn + 8 * l16) : u32x4{0u, 0u, 0u, 0u};
    }

    // scores: D[m][n = key l16]; row m = 0 (lanes grp == 0, register 0) is the query's
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      const int kl = 64 * w + 16 * sb + l16;
      const bool valid = blk + kl < k_end;
#pragma unroll
      for (int br = 0; br < 2; ++br) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 2; ++t)
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[br][t], __builtin_bit_cast(bf16x8, kf[br][sb][t]), s, 0, 0, 0);
        if (grp == 0) sc_lds[br][kl] = valid ? s[0] : -INFINITY;
      }
    }
    if (blk + kKB < k_end) load_k(blk + kKB);
    __syncthreads();

    // block softmax statistics: wavefront 0 owns branch 1, wavefront 1 branch 2
    if (w < 2) {
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = sc_lds[w][lane + 64 * i];
      const float mx = wave_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
      const float mnew = fmaxf(mrun, mx);
      const float alpha = exp2f((mrun - mnew) * c2);
      mrun = mnew;
      const float nm = -mnew * c2;
      float ls = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = __builtin_amdgcn_exp2f(fmaf(x[i], c2, nm));
        pw_lds[lane + 64 * i][w] = e;
        ls += e;
      }
      lrun = lrun * alpha + wave_sum(ls);
      if (lane == 0) alpha_lds[w] = alpha;
    }
    __syncthreads();

    // P.V for both branches from one read of V: lane covers channels 8*l16 .. +7 of keys
    // 64w + 4st + grp
    const float a0 = alpha_lds[0], a1 = alpha_lds[1];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[0][e] *= a0;
      acc[1][e] *= a1;
    }
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int kl = 64 * w + 4 * st + grp;
      typedef float f32x2 __attribute__((ext_vector_type(2)));
      const f32x2 pw = *reinterpret_cast<const f32x2*>(&pw_lds[kl][0]);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float lo = bf16_lo(vf[st][m]), hi = bf16_hi(vf[st][m]);
        acc[0][2 * m] = fmaf(pw[0], lo, acc[0][2 * m]);
        acc[0][2 * m + 1] = fmaf(pw[0], hi, acc[0][2 * m + 1]);
        acc[1][2 * m] = fmaf(pw[1], lo, acc[1][2 * m]);
        acc[1][2 * m + 1] = fmaf(pw[1], hi, acc[1][2 * m + 1]);
      }
    }
    __syncthreads();
  }

  // reduce the four key groups of each wavefront, then the four wavefronts
#pragma unroll
  for (int br = 0; br < 2; ++br)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[br][e];
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc[br][e] = x;
    }
  if (grp == 0) {
#pragma unroll
    for (int br = 0; br < 2; ++br)
#pragma unroll
      for (int e = 0; e < 8; ++e) red_lds[w][br][8 * l16 + e] = acc[br][e];
  }
  const int64_t row0 = ((int64_t)b * p.H + h) * 2;  // first (head, branch) row of this head
  if (w < 2 && lane == 0) {
    float* ml = p.ws_ml + ((row0 + w) * p.splits + split) * 2;
    ml[0] = mrun;
    ml[1] = lrun;
  }
  __syncthreads();
  for (int idx = tid; idx < 2 * kDV; idx += kThreads) {
    const int br = idx / kDV;
    const int ch = idx % kDV;
    const float s = red_lds[0][br][ch] + red_lds[1][br][ch] + red_lds[2][br][ch] + red_lds[3][br][ch];
    p.ws_acc[((row0 + br) * p.splits + split) * kDV + ch] = s;
  }
}

__global__ __launch_bounds__(kDV) void decode_v1_combine_kernel(const DecodeV1Params p) {
  __shared__ float ss_lds[2];
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int ch = threadIdx.x;
  const int lane = ch & 63;
  const float lam = head_lambda(p.lam, h, lane);
  if (p.lam.out != nullptr && b == 0 && ch == 0) p.lam.out[h] = lam;
  const int64_t row0 = ((int64_t)b * p.H + h) * 2;
  float o[2];
  if (p.splits <= kCombineBatch) {
    // every partial of both branches loaded at once (their loads in flight together), then
    // merged in split order
    float mv[2][kCombineBatch], lv[2][kCombineBatch], av[2][kCombineBatch];
#pragma unroll
    for (int br = 0; br < 2; ++br) {
      const float* ml = p.ws_ml + (row0 + br) * p.splits * 2;
      const float* ac = p.ws_acc + (row0 + br) * p.splits * kDV;
#pragma unroll
      for (int s = 0; s < kCombineBatch; ++s) {
        mv[br][s] = kNegBig;
        lv[br][s] = av[br][s] = 0.f;
        if (s < p.splits) {
          mv[br][s] = ml[2 * s];
          lv[br][s] = ml[2 * s + 1];
          av[br][s] = ac[(int64_t)s * kDV + ch];
        }
      }
    }
#pragma unroll
    for (int br = 0; br < 2; ++br) {
      float m = kNegBig;
#pragma unroll
      for (int s = 0; s < kCombineBatch; ++s) m = fmaxf(m, mv[br][s]);
      float l = 0.f, x = 0.f;
#pragma unroll
      for (int s = 0; s < kCombineBatch; ++s) {
        if (s < p.splits) {
          const float wgt = exp2f((mv[br][s] - m) * p.scale_log2);
          l = fmaf(lv[br][s], wgt, l);
          x = fmaf(av[br][s], wgt, x);
        }
      }
      o[br] = x / l;
    }
  } else {
#pragma unroll
    for (int br = 0; br < 2; ++br) {
      const float* ml = p.ws_ml + (row0 + br) * p.splits * 2;
      const float* ac = p.ws_acc + (row0 + br) * p.splits * kDV;
      float m = kNegBig;
      for (int s = 0; s < p.splits; ++s) m = fmaxf(m, ml[2 * s]);
      float l = 0.f, x = 0.f;
      for (int s = 0; s < p.splits; ++s) {
        const float wgt = exp2f((ml[2 * s] - m) * p.scale_log2);
        l = fmaf(ml[2 * s + 1], wgt, l);
        x = fmaf(ac[(int64_t)s * kDV + ch], wgt, x);
      }
      o[br] = x / l;
    }
  }
  const float x = o[0] - lam * o[1];
  float rs = 1.f;
  if (p.norm) {
    const float ws = wave_sum(x * x);
    if (lane == 0) ss_lds[ch >> 6] = ws;
    __syncthreads();
    rs = p.out_scale * rsqrtf((ss_lds[0] + ss_lds[1]) * (1.f / kDV) + p.eps);
  }
  bf16* out = static_cast<bf16*>(p.out) + b * p.so.sb + h * p.so.sh;
  out[ch] = (bf16)(x * rs);
}

}  // namespace

hipError_t launch_decode_v1(const DecodeV1Params& p, hipStream_t stream) {
  hipLaunchKernelGGL(decode_v1_partial_kernel, dim3(p.splits, p.H, p.B), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_v1_combine_kernel, dim3(p.H, p.B), dim3(kDV), 0, stream, p);
  return hipGetLastError();
}

}  // namespace da
