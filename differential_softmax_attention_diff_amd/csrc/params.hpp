// Plain-old-data parameter blocks handed from the C-ABI layer to the kernel launchers.
// No HIP types here: the ABI layer and the kernels' translation units both include it.
#pragma once
#include <stdint.h>

namespace da {

// Lambda inputs of one call: four fp32 vectors per head (or head pair), the 1-based layer's
// lambda_init, and the optional override / readback buffers (all device pointers).
struct LambdaArgs {
  const float* lq1;
  const float* lk1;
  const float* lq2;
  const float* lk2;
  int32_t dl;
  float lam_init;
  const float* override_;
  float* out;
};

struct Strides {
  int64_t sb, sh, sn;
};

// Prefill (V1 and V2).  For V1 `heads` is H and k2 is used; for V2 `heads` is the number of
// pairs P, k1 == k2 == k, and q1 / q2 hold the even / odd query heads.
struct PrefillParams {
  const void* q1;
  const void* q2;
  const void* k1;
  const void* k2;
  const void* v;
  void* out;
  Strides sq1, sq2, sk1, sk2, sv, so;
  int32_t B, heads, Hkv, N;
  int32_t causal;
  int32_t window;        // causal sliding window: row i sees keys i-window+1 .. i (0: none)
  int32_t norm;          // V1: apply RMS norm + (1 - lambda_init) scale
  int32_t n_row_blocks;  // query row blocks per (batch, head group)
  int32_t pairs_per_kv;  // V2: P / Hkv
  int32_t head_chunk;    // heads (V2: KV heads) whose row blocks are issued together (chunked_block)
  float scale_log2;      // log2(e) / sqrt(d)
  float scale;           // 1 / sqrt(d)
  float eps;
  float out_scale;       // 1 - lambda_init
  LambdaArgs lam;
  // V1 training forward: per-branch normalised outputs O_b = A_b V and base-2 log-sum-exp of the
  // scaled scores, for the backward pass (null: not written)
  float* stash_o;        // [2, B, H, N, 2d]
  float* stash_lse;      // [2, B, H, N]
  // V2: V rewritten once per call as fp16, contiguous [B, Hkv, N, 128], per region of 16 keys x
  // 64 channels (kept as bf16 where the region holds a value beyond the fp16 range), and one flag
  // byte per region, [B, Hkv, ceil(N / 32), 4]: byte 2u + c of a 32-key tile is its key half u,
  // channel half c (1: bf16)
  void* vh;
  uint8_t* vflags;
};

// V1 backward.  Inputs bf16 (strided); gradients fp32, contiguous.
struct BwdParams {
  const void* q1;
  const void* q2;
  const void* k1;
  const void* k2;
  const void* v;
  const void* dy;
  Strides sq1, sq2, sk1, sk2, sv, sdy;
  float* dq1;            // [B, H, N, d]
  float* dq2;
  float* dk1;
  float* dk2;
  float* dv;             // [B, H, N, 2d]
  int32_t B, H, N;
  int32_t causal;
  int32_t window;        // causal sliding window of the forward (0: none)
  int32_t n_row_blocks;  // 64-key blocks of the dK/dV kernel
  int32_t head_chunk;    // heads whose blocks are issued together (see chunked_block)
  float scale;           // 1 / sqrt(d)
  float scale_log2;      // log2(e) / sqrt(d)
  float eps;
  float g;               // 1 - lambda_init
  const float* stash_o;  // [2, B, H, N, 2d] from the training forward
  float* lse_d;          // [4, B, H, N]: LSE_1, LSE_2 (forward, base 2), -Dt_1, -Dt_2 (dQ prologue)
  void* d_o;             // [B, H, N, 2d] bf16: upstream gradient through the norm (dQ prologue)
  float* dl_row;         // [B, H, N]: each row's share of dlambda (dQ prologue)
  LambdaArgs lam;
  float* dlq1;           // [H, dl] lambda-vector gradients
  float* dlk1;
  float* dlq2;
  float* dlk2;
};

// One V2 decode step: split-K partial pass + combine pass.
struct DecodeParams {
  const void* q1;
  const void* q2;
  const void* k;
  const void* v;
  void* out;
  Strides sq1, sq2, sk, sv, so;
  int32_t B, P, Hkv, L, D;
  int32_t splits;        // key-axis splits per (batch, KV head)
  int32_t chunk;         // keys per split (multiple of the block size)
  float scale_log2;
  float* ws_acc;         // [B, 2P, splits, D]
  float* ws_ml;          // [B, 2P, splits, 2]  (running max in score units, sum)
  LambdaArgs lam;
  // Paged cache (serving layout); k / v then point at pages [num_pages, Hkv, page_size, D].
  const int32_t* block_table;  // [B, max_blocks] page index of each page_size-key block
  const int32_t* seq_lens;     // [B] keys of each sequence (1 .. L; L is the longest)
  int32_t max_blocks;
  int32_t page_shift;          // log2(page_size)
  int32_t num_pages;
  // Paged cache only: > 0 deals all sequences' blocks evenly to this many workgroups per KV
  // head (partials at [2P, stream_wgs + B] rows); 0 splits every sequence into `splits` pieces.
  int32_t stream_wgs;
};

// One V1 decode step: split-K partial pass + combine pass (norm and scale in the combine).
struct DecodeV1Params {
  const void* q1;
  const void* q2;
  const void* k1;
  const void* k2;
  const void* v;
  void* out;
  Strides sq1, sq2, sk1, sk2, sv, so;
  int32_t B, H, L;
  int32_t splits;        // key-axis splits per (batch, head)
  int32_t chunk;         // keys per split (multiple of the block size)
  int32_t norm;          // apply RMS norm + (1 - lambda_init) scale
  float scale_log2;
  float eps;
  float out_scale;       // 1 - lambda_init
  float* ws_acc;         // [B, H, 2, splits, 2d]
  float* ws_ml;          // [B, H, 2, splits, 2]  (running max in score units, sum)
  LambdaArgs lam;
};

}  // namespace da
