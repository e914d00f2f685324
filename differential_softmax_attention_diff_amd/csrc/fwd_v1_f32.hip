// V1 differential attention, fp32 in / fp32 out, fp32 arithmetic (correctness-grade path).
//
// Computes, per head and query row i (Ultralytics glossary "Differential Transformer", section
// "Cómo funciona la atención diferencial"):
//   O_i = sum_j (A1_ij - lambda A2_ij) V_j,  A_b = softmax(Q_b K_b^T / sqrt(d)),
//   y_i = (1 - lambda_init) * O_i / sqrt(mean(O_i^2) + eps)      (unless norm is off).
// One 64-lane wavefront owns one query row.  The softmax is the exact two-pass form: a first
// sweep over the visible keys finds each branch's row maximum, a second sweep forms
// exp(s - max), the row sums and the two weighted value sums.  Lanes own keys while scoring and
// value channels (c and c + 64) while accumulating; the weights of each group of 64 keys are
// broadcast lane by lane.  Head width d = 64, value width 128.
#include "device_common.hpp"
#include "launch.hpp"

namespace da {
namespace {

constexpr int kD = 64;
constexpr int kDV = 128;
constexpr int kRowsPerBlock = 4;  // one wavefront per query row

__device__ __forceinline__ float dot64(const float (&q)[kD], const float* __restrict__ k) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < kD; e += 4) {
    const float4 kv = *reinterpret_cast<const float4*>(k + e);
    s = fmaf(q[e + 0], kv.x, s);
    s = fmaf(q[e + 1], kv.y, s);
    s = fmaf(q[e + 2], kv.z, s);
    s = fmaf(q[e + 3], kv.w, s);
  }
  return s;
}

__global__ __launch_bounds__(256) void v1_f32_kernel(const PrefillParams p) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int b = blockIdx.y / p.heads;
  const int h = blockIdx.y % p.heads;
  const int i = blockIdx.x * kRowsPerBlock + w;

  const float lam = head_lambda(p.lam, h, lane);
  if (p.lam.out != nullptr && b == 0 && blockIdx.x == 0 && w == 0 && lane == 0) p.lam.out[h] = lam;
  if (i >= p.N) return;  // wave-uniform; the kernel has no block-wide barrier

  const float* q1 = static_cast<const float*>(p.q1) + b * p.sq1.sb + h * p.sq1.sh + (int64_t)i * p.sq1.sn;
  const float* q2 = static_cast<const float*>(p.q2) + b * p.sq2.sb + h * p.sq2.sh + (int64_t)i * p.sq2.sn;
  const float* k1 = static_cast<const float*>(p.k1) + b * p.sk1.sb + h * p.sk1.sh;
  const float* k2 = static_cast<const float*>(p.k2) + b * p.sk2.sb + h * p.sk2.sh;
  const float* v = static_cast<const float*>(p.v) + b * p.sv.sb + h * p.sv.sh;
  float* out = static_cast<float*>(p.out) + b * p.so.sb + h * p.so.sh + (int64_t)i * p.so.sn;

  float q1r[kD], q2r[kD];
#pragma unroll
  for (int e = 0; e < kD; e += 4) {
    const float4 a = *reinterpret_cast<const float4*>(q1 + e);
    const float4 c = *reinterpret_cast<const float4*>(q2 + e);
    q1r[e] = a.x; q1r[e + 1] = a.y; q1r[e + 2] = a.z; q1r[e + 3] = a.w;
    q2r[e] = c.x; q2r[e + 1] = c.y; q2r[e + 2] = c.z; q2r[e + 3] = c.w;
  }

  const int nk = p.causal ? i + 1 : p.N;  // visible keys: j0 <= j < nk
  const int jb = p.window > 0 ? max(0, i - p.window + 1) : 0;

  // sweep 1: row maxima of both branches
  float m1 = -INFINITY, m2 = -INFINITY;
  for (int j0 = jb; j0 < nk; j0 += 64) {
    const int j = j0 + lane;
    if (j < nk) {
      m1 = fmaxf(m1, dot64(q1r, k1 + (int64_t)j * p.sk1.sn) * p.scale);
      m2 = fmaxf(m2, dot64(q2r, k2 + (int64_t)j * p.sk2.sn) * p.scale);
    }
  }
  m1 = wave_max(m1);
  m2 = wave_max(m2);

  // sweep 2: exp(s - max), row sums, weighted value sums
  float l1 = 0.f, l2 = 0.f;
  float a1[2] = {0.f, 0.f}, a2[2] = {0.f, 0.f};
  for (int j0 = jb; j0 < nk; j0 += 64) {
    const int j = j0 + lane;
    float e1 = 0.f, e2 = 0.f;
    if (j < nk) {
      e1 = expf(dot64(q1r, k1 + (int64_t)j * p.sk1.sn) * p.scale - m1);
      e2 = expf(dot64(q2r, k2 + (int64_t)j * p.sk2.sn) * p.scale - m2);
    }
    l1 += e1;
    l2 += e2;
    const int cnt = min(64, nk - j0);
    for (int jj = 0; jj < cnt; ++jj) {
      const float w1 = __shfl(e1, jj);
      const float w2 = __shfl(e2, jj);
      const float* vr = v + (int64_t)(j0 + jj) * p.sv.sn;
      const float v0 = vr[lane];
      const float v1 = vr[lane + 64];
      a1[0] = fmaf(w1, v0, a1[0]);
      a1[1] = fmaf(w1, v1, a1[1]);
      a2[0] = fmaf(w2, v0, a2[0]);
      a2[1] = fmaf(w2, v1, a2[1]);
    }
  }
  l1 = wave_sum(l1);
  l2 = wave_sum(l2);

  // difference of the two normalised branches, then per-head RMS norm and scale
  float o0 = a1[0] / l1 - lam * (a2[0] / l2);
  float o1 = a1[1] / l1 - lam * (a2[1] / l2);
  if (p.norm) {
    const float ss = wave_sum(o0 * o0 + o1 * o1);
    const float r = p.out_scale / sqrtf(ss / (float)kDV + p.eps);
    o0 *= r;
    o1 *= r;
  }
  out[lane] = o0;
  out[lane + 64] = o1;
}

}  // namespace

hipError_t launch_v1_f32(const PrefillParams& p, hipStream_t stream) {
  const dim3 grid((p.N + kRowsPerBlock - 1) / kRowsPerBlock, p.B * p.heads);
  hipLaunchKernelGGL(v1_f32_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace da
