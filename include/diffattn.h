/*
 * diffattn.h -- C ABI of the MI355X (gfx950) differential-attention forward library.
 *
 * Differential attention computes, for each head, two ordinary softmax maps
 *   A1 = softmax(Q1 K1^T / sqrt(d)),   A2 = softmax(Q2 K2^T / sqrt(d))
 * and returns (A1 - lambda * A2) V.  lambda is one learnable scalar per head,
 *   lambda = exp(<lq1, lk1>) - exp(<lq2, lk2>) + lambda_init(l),
 *   lambda_init(l) = 0.8 - 0.6 * exp(-0.3 * (l - 1))     (l = 1-based layer index).
 * Sources: Ultralytics glossary "Differential Transformer", section "Cómo funciona la atención
 * diferencial" (the two maps, their difference times V, the lambda schedule, per-head
 * normalisation followed by the (1 - lambda_init) scale, half the heads with V twice as wide);
 * ai-engineering.academy "Atención Diferencial (V2)", sections "La idea diferencial" (maps,
 * difference, lambda from four vectors) and "V1 vs V2: la diferencia" (V2: doubled query heads
 * over unchanged KV heads, outputs of a pair subtracted, no per-head RMSNorm; decode reads the
 * KV cache once).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are described by da_tensor: a DEVICE pointer to element [0,0,0(,0)] and the
 *    element strides of the batch, head and row axes.  The last axis is always contiguous
 *    (stride 1) and must start 16-byte aligned in every row (strides multiples of 8 elements
 *    for bf16, 4 for fp32).
 *  - The caller owns every buffer.  The library allocates no device or host memory; the
 *    decode path writes its split partials into a caller-provided device workspace.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null stream).
 *    The library never synchronises; a result is valid once the stream has reached it.  Calls
 *    enqueue kernels only (no allocation, memset or copy), so they can be captured in a HIP
 *    graph and replayed with new contents in the same buffers.
 *  - All argument checks run on the host before anything is enqueued.  On any error nothing
 *    is launched and no output byte is written.  Empty problems (a zero batch, head or pair
 *    count, or N == 0 in a prefill) return DA_OK and enqueue nothing, before any pointer is
 *    looked at.  A decode step with L == 0 is DA_ERR_SHAPE: its cache holds at least the new
 *    token.  No entry point aborts, throws or prints.
 *  - Apart from the one scratch array of diffattn_decode_noalloc, the library keeps no
 *    mutable global state; concurrent calls on different streams are safe as long as their
 *    output/workspace buffers do not overlap.
 *  - Causal masking: query row i sees key j iff j <= i (square problem, N queries, N keys).
 */
#ifndef DIFFATTN_H
#define DIFFATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DA_OK = 0,
  DA_ERR_NULL = 1,        /* a required pointer is NULL or not 16-byte aligned              */
  DA_ERR_SHAPE = 2,       /* non-positive / inconsistent sizes or strides, layer < 1, eps<0 */
  DA_ERR_UNSUPPORTED = 3, /* head width, dtype or head-count ratio not implemented          */
  DA_ERR_WORKSPACE = 4,   /* decode workspace missing or smaller than required              */
  DA_ERR_HIP = 5          /* a HIP runtime call or kernel launch reported an error          */
} da_status;

typedef enum { DA_F32 = 0, DA_BF16 = 1 } da_dtype;

/* A strided 3-D or 4-D device tensor [batch, head, row, col]; col is contiguous. */
typedef struct {
  void* ptr;  /* device pointer to element [0,0,0,0]                                 */
  int64_t sb; /* element stride between batches                                      */
  int64_t sh; /* element stride between heads                                        */
  int64_t sn; /* element stride between rows (ignored for the 3-D decode q/out)      */
} da_tensor;

/* Lambda parameters: four device fp32 vectors per head (V1) or per head pair (V2/decode),
 * stored as row-major [n_lambda, dl] arrays (row h belongs to head/pair h). */
typedef struct {
  const float* lq1;
  const float* lk1;
  const float* lq2;
  const float* lk2;
  int32_t dl;                   /* length of each vector, 1..256                              */
  int32_t layer;                /* 1-based layer index l of lambda_init(l)                    */
  const float* lambda_override; /* nullable device fp32 [n_lambda]: use these lambdas instead */
  float* lambda_out;            /* nullable device fp32 [n_lambda]: receives the lambdas used */
} da_lambda;

/* Gradients of the four lambda vectors (device fp32 [H, dl] each), written by diffattn_bwd_v1. */
typedef struct {
  float* dlq1;
  float* dlk1;
  float* dlq2;
  float* dlk2;
} da_lambda_grad;

/* flags for diffattn_fwd_v1 */
#define DA_V1_NO_NORM 1u /* return the core (A1 - lambda A2) V without RMS norm and scale */

/*
 * diffattn_fwd_v1 -- V1 layout (Ultralytics glossary "Differential Transformer", section
 * "Cómo funciona la atención diferencial"): every head splits its query and key projections
 * into two halves of width d and reads a value row twice as wide.
 *
 *   q1, q2, k1, k2 : [B, H, N, d]   (dtype)            V : [B, H, N, 2d]   (dtype)
 *   out            : [B, H, N, 2d]  (dtype)            lambda vectors: [H, dl]
 *   out[b,h,i,:] = (1 - lambda_init(l)) * O / sqrt(mean(O^2) + eps),
 *   O = sum_j (A1[i,j] - lambda_h A2[i,j]) V[b,h,j,:]   (RMS over the 2d channels, no gain)
 *   With flags & DA_V1_NO_NORM, out = O.
 *
 * Supported: d == 64; dtype DA_BF16 (bf16 in/out, fp32 accumulation, MFMA) or DA_F32
 * (fp32 in/out, fp32 arithmetic).  Other d or dtypes return DA_ERR_UNSUPPORTED.
 */
da_status diffattn_fwd_v1(da_tensor q1, da_tensor q2, da_tensor k1, da_tensor k2, da_tensor v,
                          da_tensor out, int32_t B, int32_t H, int32_t N, int32_t d,
                          da_dtype dtype, const da_lambda* lam, int32_t causal, float eps,
                          uint32_t flags, void* stream);

/*
 * Bytes of device workspace diffattn_fwd_v2 and diffattn_fwd_v2_window need: the value tensor
 * rewritten once per call in the 16-bit format the P.V products use (B * Hkv * N * 256 bytes,
 * rounded up to 256) plus one byte per 16-key x 64-channel region (B * Hkv * ceil(N / 32) * 4).
 * Returns 0 for unsupported sizes (D != 128, non-positive dimensions).
 */
size_t diffattn_fwd_v2_workspace_bytes(int32_t B, int32_t Hkv, int32_t N, int32_t D);

/*
 * diffattn_fwd_v2 -- V2 layout (ai-engineering.academy "Atención Diferencial (V2)", sections
 * "V1 vs V2: la diferencia" and "Ejercicios" 5): 2P query heads of full width D paired as
 * (2p, 2p+1) over Hkv shared KV heads; pair p reads KV head p * Hkv / P.
 *
 *   q1 : [B, P, N, D]  query heads 2p   (e.g. a stride-2 view of a [B, 2P, N, D] tensor)
 *   q2 : [B, P, N, D]  query heads 2p+1
 *   k, v : [B, Hkv, N, D]                out : [B, P, N, D]       lambda vectors: [P, dl]
 *   out[b,p,i,:] = softmax(q1 k^T / sqrt(D)) v - lambda_p softmax(q2 k^T / sqrt(D)) v
 *   (no normalisation, no scale).
 *   workspace : device buffer of at least diffattn_fwd_v2_workspace_bytes(B, Hkv, N, D) bytes,
 *               16-byte aligned, owned by the caller; its contents on entry do not matter and are
 *               clobbered (DA_ERR_WORKSPACE if NULL, misaligned or too small).  Calls that share
 *               one workspace must be ordered (one stream).
 *
 * Supported: D == 128, dtype DA_BF16, P % Hkv == 0, B * Hkv <= 65535.
 */
da_status diffattn_fwd_v2(da_tensor q1, da_tensor q2, da_tensor k, da_tensor v, da_tensor out,
                          int32_t B, int32_t P, int32_t Hkv, int32_t N, int32_t D,
                          da_dtype dtype, const da_lambda* lam, int32_t causal, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * diffattn_fwd_v1_window, diffattn_fwd_v2_window -- the same two layouts restricted to a causal
 * sliding window, for the window layers of hybrid DIFF / sliding-window stacks
 * (ai-engineering.academy "Atención Diferencial (V2)", section "Úselo").  Query row i sees keys
 * i - window + 1 .. i (its last `window` positions, itself included); window >= N is plain
 * causal.  Arguments, layouts and results (and the V2 workspace) are those of diffattn_fwd_v1 /
 * diffattn_fwd_v2 with causal = 1, and:
 *   window : >= 1 (DA_ERR_SHAPE otherwise).
 * A decode step over a window needs no entry point of its own: pass the last `window` cache
 * rows (a strided view) to diffattn_decode / diffattn_decode_v1.
 */
da_status diffattn_fwd_v1_window(da_tensor q1, da_tensor q2, da_tensor k1, da_tensor k2,
                                 da_tensor v, da_tensor out, int32_t B, int32_t H, int32_t N,
                                 int32_t d, da_dtype dtype, const da_lambda* lam, int32_t window,
                                 float eps, uint32_t flags, void* stream);
da_status diffattn_fwd_v2_window(da_tensor q1, da_tensor q2, da_tensor k, da_tensor v,
                                 da_tensor out, int32_t B, int32_t P, int32_t Hkv, int32_t N,
                                 int32_t D, da_dtype dtype, const da_lambda* lam, int32_t window,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Training: diffattn_fwd_v1_train is diffattn_fwd_v1 (bf16, d == 64, norm on; window as in
 * diffattn_fwd_v1_window, 0 for none, >= 1 only with causal = 1, DA_ERR_SHAPE otherwise) that
 * also writes a stash for the backward pass: each branch's normalised output O_b = A_b V and the
 * base-2 log-sum-exp of its scaled scores per row ([2, B, H, N, 2d] then [2, B, H, N] fp32,
 * followed by [2, B, H, N] fp32 that diffattn_bwd_v1 fills).  Size it with
 * diffattn_v1_train_stash_bytes; 16-byte aligned; DA_ERR_WORKSPACE if missing or short.
 *
 * diffattn_bwd_v1 -- gradients of the V1 output (Ultralytics glossary "Differential
 * Transformer", section "Cómo funciona la atención diferencial"; ai-engineering.academy
 * "Atención Diferencial (V2)", section "La idea diferencial"): given dy = dL/dout [B, H, N, 2d]
 * (bf16, strided) and the same inputs, lambda, causal flag, window and eps as the training
 * forward whose stash is passed, it writes
 *   dq1, dq2, dk1, dk2 : fp32 contiguous [B, H, N, d];   dv : fp32 contiguous [B, H, N, 2d]
 *   dlam->dlq1 .. dlk2  : fp32 [H, dl] (required unless lam->lambda_override is set, in which
 *                         case lambda is an input with no vector gradients)
 * workspace: at least diffattn_bwd_v1_workspace_bytes(B, H, N, d) bytes, 16-byte aligned.
 * Supported: d == 64, dtype DA_BF16, B * H * N < 2^28.  B, H or N == 0: DA_OK and nothing is
 * written (no row contributes, so a caller that wants the lambda-vector gradients of an empty
 * batch sets them to zero itself).
 */
size_t diffattn_v1_train_stash_bytes(int32_t B, int32_t H, int32_t N, int32_t d);
size_t diffattn_bwd_v1_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t d);
da_status diffattn_fwd_v1_train(da_tensor q1, da_tensor q2, da_tensor k1, da_tensor k2,
                                da_tensor v, da_tensor out, int32_t B, int32_t H, int32_t N,
                                int32_t d, da_dtype dtype, const da_lambda* lam, int32_t causal,
                                int32_t window, float eps, void* stash, size_t stash_bytes,
                                void* stream);
da_status diffattn_bwd_v1(da_tensor q1, da_tensor q2, da_tensor k1, da_tensor k2, da_tensor v,
                          da_tensor dy, float* dq1, float* dq2, float* dk1, float* dk2, float* dv,
                          int32_t B, int32_t H, int32_t N, int32_t d, da_dtype dtype,
                          const da_lambda* lam, const da_lambda_grad* dlam, int32_t causal,
                          int32_t window, float eps, const void* stash, size_t stash_bytes,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace diffattn_decode needs for these sizes and split count
 * (num_splits <= 0 selects the library's default).  Returns 0 for unsupported sizes.
 */
size_t diffattn_decode_workspace_bytes(int32_t B, int32_t P, int32_t Hkv, int32_t L, int32_t D,
                                       int32_t num_splits);

/*
 * diffattn_decode -- one V2 decode step (ai-engineering.academy "Atención Diferencial (V2)",
 * section "V1 vs V2: la diferencia": the KV cache is read once per step for both heads of a
 * pair).  Each sequence has one new query token whose own K/V already sits in cache row L-1;
 * it attends to all L rows.
 *
 *   q1, q2 : [B, P, D]   (3-D: sb, sh used, sn ignored)     out : [B, P, D]
 *   kcache, vcache : [B, Hkv, L, D]                        lambda vectors: [P, dl]
 *   out[b,p,:] = last row of diffattn_fwd_v2 with N = L.
 *   workspace: device buffer of at least diffattn_decode_workspace_bytes(...) bytes, 16-byte
 *   aligned; its contents on entry do not matter and are clobbered.
 *
 * Supported: D == 128, dtype DA_BF16, P % Hkv == 0, 2P / Hkv <= 16.
 */
da_status diffattn_decode(da_tensor q1, da_tensor q2, da_tensor kcache, da_tensor vcache,
                          da_tensor out, int32_t B, int32_t P, int32_t Hkv, int32_t L, int32_t D,
                          da_dtype dtype, const da_lambda* lam, int32_t num_splits,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * diffattn_decode_noalloc -- diffattn_decode for callers that cannot allocate device memory or
 * pass a workspace (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, layouts, result and kernels as diffattn_decode, without the
 * workspace: the split partials go to a fixed scratch array of DIFFATTN_DECODE_NOALLOC_MAX_BYTES
 * (16 MiB) in device memory that the library holds on every GPU it runs on until the process
 * ends.  The call allocates nothing (no hipMalloc, no allocating library routine).
 *   - DA_ERR_WORKSPACE if diffattn_decode_workspace_bytes(B, P, Hkv, L, D, num_splits) exceeds
 *     DIFFATTN_DECODE_NOALLOC_MAX_BYTES (e.g. B = 64, 32 query heads, the default 8 splits at
 *     L = 32768 need 8.5 MB: fits); nothing is enqueued then.
 *   - DA_ERR_HIP if the scratch's device address cannot be found on the current device.
 *   - Every call on one GPU uses that GPU's one scratch array, and nothing in it needs clearing
 *     (each call writes every partial it reads): calls that overlap on one GPU (several streams
 *     or threads at once) race and must be ordered by the caller.
 */
#define DIFFATTN_DECODE_NOALLOC_MAX_BYTES ((size_t)16 << 20)
da_status diffattn_decode_noalloc(da_tensor q1, da_tensor q2, da_tensor kcache, da_tensor vcache,
                                  da_tensor out, int32_t B, int32_t P, int32_t Hkv, int32_t L,
                                  int32_t D, da_dtype dtype, const da_lambda* lam,
                                  int32_t num_splits, void* stream);

/*
 * diffattn_decode_paged -- the V2 decode step on the serving layout: a pool of KV pages addressed
 * through a per-sequence block table, each sequence with its own length (the layout of the
 * production inference servers that ai-engineering.academy "Atención Diferencial (V2)", section
 * "Úselo", names for V2).  Same computation as diffattn_decode with L = seq_lens[b] for
 * sequence b (its own K/V sits at row seq_lens[b] - 1).
 *
 *   q1, q2 : [B, P, D]  (3-D: sb, sh used, sn ignored)            out : [B, P, D]
 *   k_pages, v_pages : contiguous [num_pages, Hkv, page_size, D] bf16, 16-byte aligned
 *   block_table : contiguous int32 [B, max_blocks]; key j of sequence b lives in page
 *                 block_table[b][j / page_size], row j % page_size
 *   seq_lens    : int32 [B], each in 1 .. max_len (device data: not checked on the host; values
 *                 are clamped to [0, max_len] and page indices to [0, num_pages), so a bad entry
 *                 gives wrong values but no access outside the buffers; a length of 0 gives NaN)
 *   max_len     : host-side bound on seq_lens (<= max_blocks * page_size); sizes the
 *                 workspace, diffattn_decode_workspace_bytes(B, P, Hkv, max_len, D, num_splits)
 *                 bytes, which hold S pieces per sequence (S as for diffattn_decode with
 *                 L = max_len).  With S >= 2 the blocks of all sequences, whatever their lengths,
 *                 are dealt evenly to min(W, B (S - 1)) workgroups per KV head, W being what the
 *                 GPU holds at once; with S = 1 (num_splits = 1, or max_len <= 256) each
 *                 sequence is one piece.
 *   page_size   : a power of two, 1 .. 65536.
 *
 * Supported: D == 128, dtype DA_BF16, P % Hkv == 0, 2P / Hkv <= 16.
 */
da_status diffattn_decode_paged(da_tensor q1, da_tensor q2, const void* k_pages,
                                const void* v_pages, const int32_t* block_table,
                                const int32_t* seq_lens, da_tensor out, int32_t B, int32_t P,
                                int32_t Hkv, int32_t D, int32_t page_size, int32_t num_pages,
                                int32_t max_blocks, int32_t max_len, da_dtype dtype,
                                const da_lambda* lam, int32_t num_splits, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace diffattn_decode_v1 needs for these sizes and split count
 * (num_splits <= 0 selects the library's default).  Returns 0 for unsupported sizes.
 */
size_t diffattn_decode_v1_workspace_bytes(int32_t B, int32_t H, int32_t L, int32_t d,
                                          int32_t num_splits);

/*
 * diffattn_decode_v1 -- one V1 decode step (Ultralytics glossary "Differential Transformer",
 * section "Cómo funciona la atención diferencial"; ai-engineering.academy "Atención Diferencial
 * (V2)", section "V1 vs V2: la diferencia", which notes that V1 decode needs the value cache for
 * both softmax branches).  Each sequence has one new query token (halves q1, q2) whose own K1,
 * K2, V already sit in cache row L-1; it attends to all L rows.  K1, K2 and V are each read once
 * per step; one pass over V feeds both branches.
 *
 *   q1, q2 : [B, H, d]   (3-D: sb, sh used, sn ignored)     out : [B, H, 2d]
 *   k1cache, k2cache : [B, H, L, d]    vcache : [B, H, L, 2d]     lambda vectors: [H, dl]
 *   out[b,h,:] = last row of diffattn_fwd_v1 with N = L (same eps, same flags:
 *   DA_V1_NO_NORM returns the core (A1 - lambda A2) V row).
 *   workspace: device buffer of at least diffattn_decode_v1_workspace_bytes(...) bytes, 16-byte
 *   aligned; its contents on entry do not matter and are clobbered.
 *
 * Supported: d == 64, dtype DA_BF16.
 */
da_status diffattn_decode_v1(da_tensor q1, da_tensor q2, da_tensor k1cache, da_tensor k2cache,
                             da_tensor vcache, da_tensor out, int32_t B, int32_t H, int32_t L,
                             int32_t d, da_dtype dtype, const da_lambda* lam, float eps,
                             uint32_t flags, int32_t num_splits, void* workspace,
                             size_t workspace_bytes, void* stream);

/* lambda_init(l) = 0.8 - 0.6 exp(-0.3 (l - 1)) in double precision; NaN for l < 1. */
double diffattn_lambda_init(int32_t layer);

/* Static, human-readable name of a status code. */
const char* diffattn_status_string(da_status status);

/* Library version string. */
const char* diffattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DIFFATTN_H */
