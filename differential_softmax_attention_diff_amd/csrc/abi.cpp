// C-ABI entry points of libdiffattn: host-side argument checks, then kernel launches.
//
// Every check runs before anything is enqueued, and no HIP runtime call is made on an error
// path, so invalid calls are safe (and testable) on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "diffattn.h"
#include "launch.hpp"

namespace {

constexpr int kMaxGridY = 65535;
constexpr int kDecodeBlock = 256;  // keys per decode block; split chunks are multiples of it

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A 4-D (or 3-D) strided tensor argument: pointer present and 16-byte aligned, strides
// non-negative and keeping every row start 16-byte aligned.
da_status check_tensor(const da_tensor& t, int elem_bytes) {
  if (t.ptr == nullptr || !aligned16(t.ptr)) return DA_ERR_NULL;
  const int64_t q = 16 / elem_bytes;
  if (t.sb < 0 || t.sh < 0 || t.sn < 0) return DA_ERR_SHAPE;
  if (t.sb % q != 0 || t.sh % q != 0 || t.sn % q != 0) return DA_ERR_SHAPE;
  return DA_OK;
}

da_status check_lambda(const da_lambda* lam, int32_t dl_expected_max) {
  if (lam == nullptr) return DA_ERR_NULL;
  if (lam->layer < 1) return DA_ERR_SHAPE;
  if (lam->lambda_override == nullptr) {
    if (!lam->lq1 || !lam->lk1 || !lam->lq2 || !lam->lk2) return DA_ERR_NULL;
    if (lam->dl < 1 || lam->dl > dl_expected_max) return DA_ERR_SHAPE;
  }
  return DA_OK;
}

da::LambdaArgs lambda_args(const da_lambda* lam) {
  da::LambdaArgs a;
  a.lq1 = lam->lq1;
  a.lk1 = lam->lk1;
  a.lq2 = lam->lq2;
  a.lk2 = lam->lk2;
  a.dl = lam->dl;
  a.lam_init = static_cast<float>(diffattn_lambda_init(lam->layer));
  a.override_ = lam->lambda_override;
  a.out = lam->lambda_out;
  return a;
}

da::Strides strides(const da_tensor& t) { return da::Strides{t.sb, t.sh, t.sn}; }

// The bf16 prefill addresses each head slice with 32-bit byte offsets (buffer loads whose range
// check zero-fills rows past N), so a slice of N + 256 rows must span less than 4 GiB.
bool rows_fit_32bit(const da_tensor& t, int32_t N, int elem_bytes) {
  return ((int64_t)N + 256) * t.sn * elem_bytes < ((int64_t)1 << 32);
}

int decode_chunk(int32_t B, int32_t Hkv, int32_t L, int32_t num_splits) {
  int splits = num_splits;
  if (splits <= 0) {
    // aim for >= 4096 workgroups over the 256 CUs, but keep >= one block per split
    const int64_t bh = (int64_t)B * Hkv;
    splits = (int)std::max<int64_t>(1, (4096 + bh - 1) / bh);
  }
  const int max_splits = (L + kDecodeBlock - 1) / kDecodeBlock;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int chunk = (L + splits - 1) / splits;
  chunk = ((chunk + kDecodeBlock - 1) / kDecodeBlock) * kDecodeBlock;
  return chunk;
}

da_status hip_status(hipError_t e) { return e == hipSuccess ? DA_OK : DA_ERR_HIP; }

}  // namespace

extern "C" {

double diffattn_lambda_init(int32_t layer) {
  if (layer < 1) return NAN;
  return 0.8 - 0.6 * std::exp(-0.3 * (double)(layer - 1));
}

const char* diffattn_status_string(da_status s) {
  switch (s) {
    case DA_OK: return "DA_OK";
    case DA_ERR_NULL: return "DA_ERR_NULL: required pointer is NULL or not 16-byte aligned";
    case DA_ERR_SHAPE: return "DA_ERR_SHAPE: invalid sizes, strides, layer or eps";
    case DA_ERR_UNSUPPORTED: return "DA_ERR_UNSUPPORTED: head width, dtype or head ratio not implemented";
    case DA_ERR_WORKSPACE: return "DA_ERR_WORKSPACE: decode workspace missing or too small";
    case DA_ERR_HIP: return "DA_ERR_HIP: HIP runtime or launch error";
  }
  return "unknown status";
}

const char* diffattn_version(void) { return "diffattn-gfx950 0.1.0"; }

}  // extern "C"

namespace {

da_status fwd_v1(da_tensor q1, da_tensor q2, da_tensor k1, da_tensor k2, da_tensor v,
                 da_tensor out, int32_t B, int32_t H, int32_t N, int32_t d, da_dtype dtype,
                 const da_lambda* lam, int32_t causal, int32_t window, float eps, uint32_t flags,
                 void* stream, float* stash = nullptr) {
  if (B < 0 || H < 0 || N < 0 || window < 0) return DA_ERR_SHAPE;
  if (window > 0 && !causal) return DA_ERR_SHAPE;  // the window is a causal one
  if (B == 0 || H == 0 || N == 0) return DA_OK;
  if (dtype != DA_F32 && dtype != DA_BF16) return DA_ERR_UNSUPPORTED;
  if (d != 64) return d <= 0 ? DA_ERR_SHAPE : DA_ERR_UNSUPPORTED;
  if (!(eps >= 0.f) || !std::isfinite(eps)) return DA_ERR_SHAPE;
  if ((flags & ~DA_V1_NO_NORM) != 0u) return DA_ERR_UNSUPPORTED;
  if ((int64_t)B * H > (int64_t)INT32_MAX || (N + 63) / 64 > kMaxGridY) return DA_ERR_UNSUPPORTED;
  const int eb = dtype == DA_F32 ? 4 : 2;
  for (const da_tensor* t : {&q1, &q2, &k1, &k2, &v, &out}) {
    const da_status s = check_tensor(*t, eb);
    if (s != DA_OK) return s;
  }
  da_status s = check_lambda(lam, 256);
  if (s != DA_OK) return s;

  da::PrefillParams p{};
  p.q1 = q1.ptr; p.q2 = q2.ptr; p.k1 = k1.ptr; p.k2 = k2.ptr; p.v = v.ptr; p.out = out.ptr;
  p.sq1 = strides(q1); p.sq2 = strides(q2); p.sk1 = strides(k1); p.sk2 = strides(k2);
  p.sv = strides(v); p.so = strides(out);
  p.B = B; p.heads = H; p.Hkv = H; p.N = N;
  p.causal = causal ? 1 : 0;
  p.window = window;
  p.norm = (flags & DA_V1_NO_NORM) ? 0 : 1;
  p.scale = (float)(1.0 / std::sqrt((double)d));
  p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
  p.eps = eps;
  p.out_scale = (float)(1.0 - diffattn_lambda_init(lam->layer));
  p.lam = lambda_args(lam);
  if (stash != nullptr) {
    const int64_t bhn = (int64_t)B * H * N;
    p.stash_o = stash;                      // [2, B, H, N, 2d]
    p.stash_lse = stash + 2 * bhn * 2 * d;  // rows 0 and 1 of [4, B, H, N]
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == DA_F32) return hip_status(da::launch_v1_f32(p, st));
  for (const da_tensor* t : {&q1, &q2, &k1, &k2, &v})
    if (!rows_fit_32bit(*t, N, 2)) return DA_ERR_UNSUPPORTED;
  return hip_status(da::launch_v1_bf16(p, st));
}

// Bytes of the V2 prefill workspace: the fp16 copy of V, then one flag byte per 16-key x
// 64-channel region (4 per 32-key tile), the flags starting on a 256-byte boundary.
int64_t v2_values_bytes(int32_t B, int32_t Hkv, int32_t N) { return ((int64_t)B * Hkv * N * 128 * 2 + 255) / 256 * 256; }
int64_t v2_workspace_bytes(int32_t B, int32_t Hkv, int32_t N) {
  return v2_values_bytes(B, Hkv, N) + (int64_t)B * Hkv * ((N + 31) / 32) * 4;
}

da_status fwd_v2(da_tensor q1, da_tensor q2, da_tensor k, da_tensor v, da_tensor out, int32_t B,
                 int32_t P, int32_t Hkv, int32_t N, int32_t D, da_dtype dtype,
                 const da_lambda* lam, int32_t causal, int32_t window, void* workspace,
                 size_t workspace_bytes, void* stream) {
  if (B < 0 || P < 0 || Hkv < 0 || N < 0 || window < 0) return DA_ERR_SHAPE;
  if (window > 0 && !causal) return DA_ERR_SHAPE;
  if (B == 0 || P == 0 || N == 0) return DA_OK;
  if (Hkv == 0) return DA_ERR_SHAPE;
  if (dtype != DA_BF16) return DA_ERR_UNSUPPORTED;
  if (D != 128) return D <= 0 ? DA_ERR_SHAPE : DA_ERR_UNSUPPORTED;
  if (P % Hkv != 0) return DA_ERR_SHAPE;
  if ((int64_t)B * P > (int64_t)INT32_MAX || (N + 63) / 64 > kMaxGridY) return DA_ERR_UNSUPPORTED;
  if ((int64_t)B * Hkv > kMaxGridY) return DA_ERR_UNSUPPORTED;
  for (const da_tensor* t : {&q1, &q2, &k, &v, &out}) {
    const da_status s = check_tensor(*t, 2);
    if (s != DA_OK) return s;
  }
  da_status s = check_lambda(lam, 256);
  if (s != DA_OK) return s;
  for (const da_tensor* t : {&q1, &q2, &k, &v})
    if (!rows_fit_32bit(*t, N, 2)) return DA_ERR_UNSUPPORTED;
  if (workspace == nullptr || !aligned16(workspace) ||
      workspace_bytes < (size_t)v2_workspace_bytes(B, Hkv, N))
    return DA_ERR_WORKSPACE;

  da::PrefillParams p{};
  p.q1 = q1.ptr; p.q2 = q2.ptr; p.k1 = k.ptr; p.k2 = k.ptr; p.v = v.ptr; p.out = out.ptr;
  p.sq1 = strides(q1); p.sq2 = strides(q2); p.sk1 = strides(k); p.sk2 = strides(k);
  p.sv = strides(v); p.so = strides(out);
  p.B = B; p.heads = P; p.Hkv = Hkv; p.N = N;
  p.causal = causal ? 1 : 0;
  p.window = window;
  p.norm = 0;
  p.scale = (float)(1.0 / std::sqrt((double)D));
  p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  p.eps = 0.f;
  p.out_scale = 1.f;
  p.lam = lambda_args(lam);
  p.vh = workspace;
  p.vflags = static_cast<uint8_t*>(workspace) + v2_values_bytes(B, Hkv, N);
  return hip_status(da::launch_v2_bf16(p, reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

da_status diffattn_fwd_v1(da_tensor q1, da_tensor q2, da_tensor k1, da_tensor k2, da_tensor v,
                          da_tensor out, int32_t B, int32_t H, int32_t N, int32_t d,
                          da_dtype dtype, const da_lambda* lam, int32_t causal, float eps,
                          uint32_t flags, void* stream) {
  return fwd_v1(q1, q2, k1, k2, v, out, B, H, N, d, dtype, lam, causal, 0, eps, flags, stream);
}

da_status diffattn_fwd_v1_window(da_tensor q1, da_tensor q2, da_tensor k1, da_tensor k2,
                                 da_tensor v, da_tensor out, int32_t B, int32_t H, int32_t N,
                                 int32_t d, da_dtype dtype, const da_lambda* lam, int32_t window,
                                 float eps, uint32_t flags, void* stream) {
  if (window < 1) return DA_ERR_SHAPE;
  return fwd_v1(q1, q2, k1, k2, v, out, B, H, N, d, dtype, lam, 1, window, eps, flags, stream);
}

size_t diffattn_fwd_v2_workspace_bytes(int32_t B, int32_t Hkv, int32_t N, int32_t D) {
  if (B <= 0 || Hkv <= 0 || N <= 0 || D != 128) return 0;
  return (size_t)v2_workspace_bytes(B, Hkv, N);
}

da_status diffattn_fwd_v2(da_tensor q1, da_tensor q2, da_tensor k, da_tensor v, da_tensor out,
                          int32_t B, int32_t P, int32_t Hkv, int32_t N, int32_t D,
                          da_dtype dtype, const da_lambda* lam, int32_t causal, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return fwd_v2(q1, q2, k, v, out, B, P, Hkv, N, D, dtype, lam, causal, 0, workspace,
                workspace_bytes, stream);
}

da_status diffattn_fwd_v2_window(da_tensor q1, da_tensor q2, da_tensor k, da_tensor v,
                                 da_tensor out, int32_t B, int32_t P, int32_t Hkv, int32_t N,
                                 int32_t D, da_dtype dtype, const da_lambda* lam, int32_t window,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (window < 1) return DA_ERR_SHAPE;
  return fwd_v2(q1, q2, k, v, out, B, P, Hkv, N, D, dtype, lam, 1, window, workspace,
                workspace_bytes, stream);
}

size_t diffattn_decode_workspace_bytes(int32_t B, int32_t P, int32_t Hkv, int32_t L, int32_t D,
                                       int32_t num_splits) {
  if (B <= 0 || P <= 0 || Hkv <= 0 || L <= 0 || D != 128 || P % Hkv != 0) return 0;
  const int chunk = decode_chunk(B, Hkv, L, num_splits);
  const int64_t splits = (L + chunk - 1) / chunk;
  return (size_t)((int64_t)B * 2 * P * splits * (D + 2) * (int64_t)sizeof(float));
}

}  // extern "C"

namespace {

// Checks of one V2 decode step (everything but the workspace); DA_OK with *empty set when the
// call has nothing to do.
da_status check_decode(const da_tensor& q1, const da_tensor& q2, const da_tensor& kcache,
                       const da_tensor& vcache, const da_tensor& out, int32_t B, int32_t P,
                       int32_t Hkv, int32_t L, int32_t D, da_dtype dtype, const da_lambda* lam,
                       bool* empty) {
  *empty = false;
  if (B < 0 || P < 0 || Hkv < 0 || L < 0) return DA_ERR_SHAPE;
  if (B == 0 || P == 0) {
    *empty = true;
    return DA_OK;
  }
  if (L == 0 || Hkv == 0) return DA_ERR_SHAPE;  // the new token's own row is always present
  if (dtype != DA_BF16) return DA_ERR_UNSUPPORTED;
  if (D != 128) return D <= 0 ? DA_ERR_SHAPE : DA_ERR_UNSUPPORTED;
  if (P % Hkv != 0) return DA_ERR_SHAPE;
  const int G = 2 * P / Hkv;
  if (G != 2 && G != 4 && G != 8 && G != 16) return DA_ERR_UNSUPPORTED;
  if (B > kMaxGridY || Hkv > kMaxGridY || P > INT32_MAX / 2) return DA_ERR_UNSUPPORTED;
  for (const da_tensor* t : {&q1, &q2, &kcache, &vcache, &out}) {
    const da_status s = check_tensor(*t, 2);
    if (s != DA_OK) return s;
  }
  return check_lambda(lam, 256);
}

// Launch one checked V2 decode step with its split partials in `workspace`.
da_status run_decode(const da_tensor& q1, const da_tensor& q2, const da_tensor& kcache,
                     const da_tensor& vcache, const da_tensor& out, int32_t B, int32_t P,
                     int32_t Hkv, int32_t L, int32_t D, const da_lambda* lam, int32_t num_splits,
                     void* workspace, void* stream) {
  da::DecodeParams p{};
  p.q1 = q1.ptr; p.q2 = q2.ptr; p.k = kcache.ptr; p.v = vcache.ptr; p.out = out.ptr;
  p.sq1 = strides(q1); p.sq2 = strides(q2); p.sk = strides(kcache); p.sv = strides(vcache);
  p.so = strides(out);
  p.B = B; p.P = P; p.Hkv = Hkv; p.L = L; p.D = D;
  p.chunk = decode_chunk(B, Hkv, L, num_splits);
  p.splits = (L + p.chunk - 1) / p.chunk;
  p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  const int64_t n_rows = (int64_t)B * 2 * P * p.splits;
  p.ws_acc = static_cast<float*>(workspace);
  p.ws_ml = p.ws_acc + n_rows * D;
  p.lam = lambda_args(lam);
  return hip_status(da::launch_decode_v2(p, reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

da_status diffattn_decode(da_tensor q1, da_tensor q2, da_tensor kcache, da_tensor vcache,
                          da_tensor out, int32_t B, int32_t P, int32_t Hkv, int32_t L, int32_t D,
                          da_dtype dtype, const da_lambda* lam, int32_t num_splits,
                          void* workspace, size_t workspace_bytes, void* stream) {
  bool empty = false;
  const da_status s = check_decode(q1, q2, kcache, vcache, out, B, P, Hkv, L, D, dtype, lam, &empty);
  if (s != DA_OK || empty) return s;
  const size_t need = diffattn_decode_workspace_bytes(B, P, Hkv, L, D, num_splits);
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need) return DA_ERR_WORKSPACE;
  return run_decode(q1, q2, kcache, vcache, out, B, P, Hkv, L, D, lam, num_splits, workspace, stream);
}

da_status diffattn_decode_noalloc(da_tensor q1, da_tensor q2, da_tensor kcache, da_tensor vcache,
                                  da_tensor out, int32_t B, int32_t P, int32_t Hkv, int32_t L,
                                  int32_t D, da_dtype dtype, const da_lambda* lam,
                                  int32_t num_splits, void* stream) {
  bool empty = false;
  const da_status s = check_decode(q1, q2, kcache, vcache, out, B, P, Hkv, L, D, dtype, lam, &empty);
  if (s != DA_OK || empty) return s;
  const size_t need = diffattn_decode_workspace_bytes(B, P, Hkv, L, D, num_splits);
  static_assert(da::kNoAllocScratchBytes == DIFFATTN_DECODE_NOALLOC_MAX_BYTES, "header constant");
  if (need > da::kNoAllocScratchBytes) return DA_ERR_WORKSPACE;
  void* scratch = da::noalloc_scratch();
  if (scratch == nullptr) return DA_ERR_HIP;
  return run_decode(q1, q2, kcache, vcache, out, B, P, Hkv, L, D, lam, num_splits, scratch, stream);
}

size_t diffattn_v1_train_stash_bytes(int32_t B, int32_t H, int32_t N, int32_t d) {
  if (B <= 0 || H <= 0 || N <= 0 || d != 64) return 0;
  const int64_t bhn = (int64_t)B * H * N;
  return (size_t)((2 * bhn * 2 * d + 4 * bhn) * (int64_t)sizeof(float));
}

size_t diffattn_bwd_v1_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t d) {
  if (B <= 0 || H <= 0 || N <= 0 || d != 64) return 0;
  const int64_t bhn = (int64_t)B * H * N;
  return (size_t)(bhn * 2 * d * 2 + bhn * (int64_t)sizeof(float));
}

da_status diffattn_fwd_v1_train(da_tensor q1, da_tensor q2, da_tensor k1, da_tensor k2,
                                da_tensor v, da_tensor out, int32_t B, int32_t H, int32_t N,
                                int32_t d, da_dtype dtype, const da_lambda* lam, int32_t causal,
                                int32_t window, float eps, void* stash, size_t stash_bytes,
                                void* stream) {
  if (B < 0 || H < 0 || N < 0 || window < 0) return DA_ERR_SHAPE;
  if (window > 0 && !causal) return DA_ERR_SHAPE;  // the window is a causal one
  if (B == 0 || H == 0 || N == 0) return DA_OK;
  if (dtype != DA_BF16) return DA_ERR_UNSUPPORTED;
  if (d != 64) return d <= 0 ? DA_ERR_SHAPE : DA_ERR_UNSUPPORTED;
  if ((int64_t)B * H * N * 16 >= ((int64_t)1 << 32)) return DA_ERR_UNSUPPORTED;
  const size_t need = diffattn_v1_train_stash_bytes(B, H, N, d);
  if (stash == nullptr || !aligned16(stash) || stash_bytes < need) return DA_ERR_WORKSPACE;
  return fwd_v1(q1, q2, k1, k2, v, out, B, H, N, d, dtype, lam, causal, window, eps, 0u, stream,
                static_cast<float*>(stash));
}

da_status diffattn_bwd_v1(da_tensor q1, da_tensor q2, da_tensor k1, da_tensor k2, da_tensor v,
                          da_tensor dy, float* dq1, float* dq2, float* dk1, float* dk2, float* dv,
                          int32_t B, int32_t H, int32_t N, int32_t d, da_dtype dtype,
                          const da_lambda* lam, const da_lambda_grad* dlam, int32_t causal,
                          int32_t window, float eps, const void* stash, size_t stash_bytes,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || H < 0 || N < 0 || window < 0) return DA_ERR_SHAPE;
  if (window > 0 && !causal) return DA_ERR_SHAPE;
  if (B == 0 || H == 0 || N == 0) return DA_OK;
  if (dtype != DA_BF16) return DA_ERR_UNSUPPORTED;
  if (d != 64) return d <= 0 ? DA_ERR_SHAPE : DA_ERR_UNSUPPORTED;
  if (!(eps >= 0.f) || !std::isfinite(eps)) return DA_ERR_SHAPE;
  // grids: (B*H, N/128) for the dQ kernel, (B*H, N/64) for the dK/dV kernel
  if ((int64_t)B * H > (int64_t)INT32_MAX || (N + 63) / 64 > kMaxGridY) return DA_ERR_UNSUPPORTED;
  if ((int64_t)B * H * N * 16 >= ((int64_t)1 << 32)) return DA_ERR_UNSUPPORTED;
  for (const da_tensor* t : {&q1, &q2, &k1, &k2, &v, &dy}) {
    const da_status s = check_tensor(*t, 2);
    if (s != DA_OK) return s;
    if (t != &dy && !rows_fit_32bit(*t, N, 2)) return DA_ERR_UNSUPPORTED;
  }
  for (const float* g : {dq1, dq2, dk1, dk2, dv})
    if (g == nullptr || !aligned16(g)) return DA_ERR_NULL;
  da_status s = check_lambda(lam, 256);
  if (s != DA_OK) return s;
  if (lam->lambda_override == nullptr &&
      (dlam == nullptr || !dlam->dlq1 || !dlam->dlk1 || !dlam->dlq2 || !dlam->dlk2))
    return DA_ERR_NULL;
  if (stash == nullptr || !aligned16(stash) || stash_bytes < diffattn_v1_train_stash_bytes(B, H, N, d))
    return DA_ERR_WORKSPACE;
  if (workspace == nullptr || !aligned16(workspace) ||
      workspace_bytes < diffattn_bwd_v1_workspace_bytes(B, H, N, d))
    return DA_ERR_WORKSPACE;

  da::BwdParams p{};
  p.q1 = q1.ptr; p.q2 = q2.ptr; p.k1 = k1.ptr; p.k2 = k2.ptr; p.v = v.ptr; p.dy = dy.ptr;
  p.sq1 = strides(q1); p.sq2 = strides(q2); p.sk1 = strides(k1); p.sk2 = strides(k2);
  p.sv = strides(v); p.sdy = strides(dy);
  p.dq1 = dq1; p.dq2 = dq2; p.dk1 = dk1; p.dk2 = dk2; p.dv = dv;
  p.B = B; p.H = H; p.N = N;
  p.causal = causal ? 1 : 0;
  p.window = window >= N ? 0 : window;  // a window covering every row is plain causal
  p.scale = (float)(1.0 / std::sqrt((double)d));
  p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
  p.eps = eps;
  p.g = (float)(1.0 - diffattn_lambda_init(lam->layer));
  const int64_t bhn = (int64_t)B * H * N;
  float* st = static_cast<float*>(const_cast<void*>(stash));
  p.stash_o = st;
  p.lse_d = st + 2 * bhn * 2 * d;
  p.d_o = workspace;
  p.dl_row = reinterpret_cast<float*>(static_cast<char*>(workspace) + bhn * 2 * d * 2);
  p.lam = lambda_args(lam);
  if (dlam != nullptr) {
    p.dlq1 = dlam->dlq1; p.dlk1 = dlam->dlk1; p.dlq2 = dlam->dlq2; p.dlk2 = dlam->dlk2;
  }
  return hip_status(da::launch_bwd_v1(p, reinterpret_cast<hipStream_t>(stream)));
}

da_status diffattn_decode_paged(da_tensor q1, da_tensor q2, const void* k_pages,
                                const void* v_pages, const int32_t* block_table,
                                const int32_t* seq_lens, da_tensor out, int32_t B, int32_t P,
                                int32_t Hkv, int32_t D, int32_t page_size, int32_t num_pages,
                                int32_t max_blocks, int32_t max_len, da_dtype dtype,
                                const da_lambda* lam, int32_t num_splits, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (B < 0 || P < 0 || Hkv < 0) return DA_ERR_SHAPE;
  if (B == 0 || P == 0) return DA_OK;
  if (Hkv == 0 || max_len < 1 || num_pages < 1 || max_blocks < 1) return DA_ERR_SHAPE;
  if (page_size < 1 || page_size > (1 << 16) || (page_size & (page_size - 1)) != 0) return DA_ERR_SHAPE;
  if ((int64_t)max_blocks * page_size < max_len) return DA_ERR_SHAPE;
  if (dtype != DA_BF16) return DA_ERR_UNSUPPORTED;
  if (D != 128) return D <= 0 ? DA_ERR_SHAPE : DA_ERR_UNSUPPORTED;
  if (P % Hkv != 0) return DA_ERR_SHAPE;
  const int G = 2 * P / Hkv;
  if (G != 2 && G != 4 && G != 8 && G != 16) return DA_ERR_UNSUPPORTED;
  if (B > kMaxGridY || Hkv > kMaxGridY || P > INT32_MAX / 2) return DA_ERR_UNSUPPORTED;
  for (const da_tensor* t : {&q1, &q2, &out}) {
    const da_status s = check_tensor(*t, 2);
    if (s != DA_OK) return s;
  }
  if (!k_pages || !v_pages || !aligned16(k_pages) || !aligned16(v_pages)) return DA_ERR_NULL;
  if (!block_table || !seq_lens || (reinterpret_cast<uintptr_t>(block_table) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u) != 0)
    return DA_ERR_NULL;
  da_status s = check_lambda(lam, 256);
  if (s != DA_OK) return s;
  const size_t need = diffattn_decode_workspace_bytes(B, P, Hkv, max_len, D, num_splits);
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need) return DA_ERR_WORKSPACE;

  da::DecodeParams p{};
  p.q1 = q1.ptr; p.q2 = q2.ptr; p.k = k_pages; p.v = v_pages; p.out = out.ptr;
  p.sq1 = strides(q1); p.sq2 = strides(q2); p.so = strides(out);
  p.sk = da::Strides{0, 0, 0}; p.sv = da::Strides{0, 0, 0};
  p.B = B; p.P = P; p.Hkv = Hkv; p.L = max_len; p.D = D;
  p.chunk = decode_chunk(B, Hkv, max_len, num_splits);
  p.splits = (max_len + p.chunk - 1) / p.chunk;
  p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  const int64_t n_rows = (int64_t)B * 2 * P * p.splits;
  p.ws_acc = static_cast<float*>(workspace);
  p.ws_ml = p.ws_acc + n_rows * D;
  p.lam = lambda_args(lam);
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.max_blocks = max_blocks;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  p.page_shift = shift;
  p.num_pages = num_pages;
  return hip_status(da::launch_decode_v2_paged(p, reinterpret_cast<hipStream_t>(stream)));
}

size_t diffattn_decode_v1_workspace_bytes(int32_t B, int32_t H, int32_t L, int32_t d,
                                          int32_t num_splits) {
  if (B <= 0 || H <= 0 || L <= 0 || d != 64) return 0;
  const int chunk = decode_chunk(B, H, L, num_splits);
  const int64_t splits = (L + chunk - 1) / chunk;
  return (size_t)((int64_t)B * H * 2 * splits * (2 * d + 2) * (int64_t)sizeof(float));
}

da_status diffattn_decode_v1(da_tensor q1, da_tensor q2, da_tensor k1cache, da_tensor k2cache,
                             da_tensor vcache, da_tensor out, int32_t B, int32_t H, int32_t L,
                             int32_t d, da_dtype dtype, const da_lambda* lam, float eps,
                             uint32_t flags, int32_t num_splits, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (B < 0 || H < 0 || L < 0) return DA_ERR_SHAPE;
  if (B == 0 || H == 0) return DA_OK;
  if (L == 0) return DA_ERR_SHAPE;  // the new token's own row is always present
  if (dtype != DA_BF16) return DA_ERR_UNSUPPORTED;
  if (d != 64) return d <= 0 ? DA_ERR_SHAPE : DA_ERR_UNSUPPORTED;
  if (!(eps >= 0.f) || !std::isfinite(eps)) return DA_ERR_SHAPE;
  if ((flags & ~DA_V1_NO_NORM) != 0u) return DA_ERR_UNSUPPORTED;
  if (B > kMaxGridY || H > kMaxGridY) return DA_ERR_UNSUPPORTED;
  for (const da_tensor* t : {&q1, &q2, &k1cache, &k2cache, &vcache, &out}) {
    const da_status s = check_tensor(*t, 2);
    if (s != DA_OK) return s;
  }
  da_status s = check_lambda(lam, 256);
  if (s != DA_OK) return s;
  const size_t need = diffattn_decode_v1_workspace_bytes(B, H, L, d, num_splits);
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need) return DA_ERR_WORKSPACE;

  da::DecodeV1Params p{};
  p.q1 = q1.ptr; p.q2 = q2.ptr; p.k1 = k1cache.ptr; p.k2 = k2cache.ptr; p.v = vcache.ptr;
  p.out = out.ptr;
  p.sq1 = strides(q1); p.sq2 = strides(q2); p.sk1 = strides(k1cache); p.sk2 = strides(k2cache);
  p.sv = strides(vcache); p.so = strides(out);
  p.B = B; p.H = H; p.L = L;
  p.chunk = decode_chunk(B, H, L, num_splits);
  p.splits = (L + p.chunk - 1) / p.chunk;
  p.norm = (flags & DA_V1_NO_NORM) ? 0 : 1;
  p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
  p.eps = eps;
  p.out_scale = (float)(1.0 - diffattn_lambda_init(lam->layer));
  const int64_t n_rows = (int64_t)B * H * 2 * p.splits;
  p.ws_acc = static_cast<float*>(workspace);
  p.ws_ml = p.ws_acc + n_rows * 2 * d;
  p.lam = lambda_args(lam);
  return hip_status(da::launch_decode_v1(p, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
