// Fused V1 differential-attention prefill for gfx950: bf16 inputs, fp32 accumulation, bf16 out.
//
// What is computed (Ultralytics glossary "Differential Transformer", section "Cómo funciona la
// atención diferencial"; ai-engineering.academy "Atención Diferencial (V2)", section "La idea
// diferencial"):
//   two softmax branches  A_b = softmax(Q_b K_b^T / sqrt(d)),  O = A_1 V - lambda A_2 V,
//   y = (1 - lambda_init) O / sqrt(mean(O^2) + eps)   (per head, over the 128 channels).
// Neither map is ever written to memory.  (The V2 layout has its own kernel, prefill_v2_bf16.)
//
// Design (one pass over K/V per block of 64 query rows):
//  * A 256-thread workgroup owns 64 query rows of one head.  Its four wavefronts are (branch,
//    row half): each runs ONE softmax branch over 32 rows, so it holds 64 fp32 accumulators
//    (32 rows x 128 channels) and only its own branch's Q operand.  That keeps the kernel at 128
//    VGPRs (4 waves per SIMD); the waves of different workgroups on a SIMD overlap one another's
//    softmax and MFMA work.
//  * Tiles of 32 keys stream global -> LDS through buffer loads that write LDS directly (issued
//    from inline asm, see dma16), double buffered: the loads of tile t+1 are in flight during
//    the MFMAs of tile t; one barrier per tile.  The buffer range check returns zeros past the
//    last row.  LDS rows are XOR-swizzled for the 64-bank LDS (16-byte chunks of K by
//    (row >> 1) & 7, 32-byte chunks of V by 2 (row & 3)): the MFMA operand reads are
//    conflict-free (SQ_LDS_BANK_CONFLICT = 0).
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16.  Its accumulator
//    gives each lane one query column and keys {8j + 4h + r}; split into two 16-key halves these
//    are exactly the B operand P^T of O^T = V^T P^T.  The V^T operand comes straight from the
//    row-major V tile through ds_read_b64_tr_b16 (a transposing LDS read: per 16-lane group, each
//    lane receives one column of a 4-key x 16-channel block).
//  * Online softmax without a per-tile max: weights exp2((s - m) log2(e)/sqrt(d)) are formed
//    against a per-row reference max m, set from the exact row max of the wave's first tile and
//    moved only when a lane's weight sum for a tile exceeds 2^12 (a score jump); then the tile's
//    exact max is taken, the accumulators rescaled and the weights formed again.  The row sums
//    add the rounded weights the MFMA consumes (v_dot2 of packed pairs against 1).
//  * Epilogue: the branch-2 wave of a row half writes lambda acc_2 / l_2 to LDS; the branch-1
//    wave forms acc_1 / l_1 minus it, applies the RMS norm and scale, and stores bf16 (RNE).  The
//    training forward also stores each branch's O_b and base-2 log-sum-exp.
//  * Causal: a wave computes tiles up to its last visible key and then only helps load; only
//    tiles crossing the diagonal, the window's lower edge or the ragged end are masked element
//    by element.  Row blocks are issued heaviest first; all row blocks of a head land on one XCD.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"
#include "tile_common.hpp"

namespace da {
namespace {

using namespace tile;
constexpr int kThreads = 256;
constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for the running max
constexpr float kCapSum = 4096.f;    // largest lane weight sum per tile (2^12) before the max moves
constexpr int kSBN = 32;  // keys per tile
// Tile buffers in LDS.  Three (loads two tiles ahead) measured 7 % slower for V1: 48 KB per
// workgroup allows 3 workgroups per CU instead of 4, and load latency was not the limit.
constexpr int kStagesV1 = 2;

template <int DQK, int NS>
struct SCfg {
  static constexpr int NK = 2;                          // K tensors per tile (K_1, K_2)
  static constexpr int K_ELEMS = kSBN * DQK;            // one K tensor tile
  static constexpr int KBUF = NK * K_ELEMS;             // one K buffer (all K tensors)
  static constexpr int VBUF = kSBN * kDV;               // one V buffer
  static constexpr int K_LOADS = K_ELEMS * 2 / 1024;    // 1 KB wavefront DMA loads per K tile
  static constexpr int V_LOADS = VBUF * 2 / 1024;
  static constexpr int TQ = DQK / 16;                   // MFMA k-steps over the head width
  static constexpr int SMEM = NS * (KBUF + VBUF);       // [K0 .. K(NS-1) | V0 .. V(NS-1)]
};

template <int DQK, int NS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void prefill_kernel(const PrefillParams p) {
  using C = SCfg<DQK, NS>;
  constexpr int BM = 64;
  __shared__ __attribute__((aligned(1024))) bf16 smem[C::SMEM];
  static_assert(C::SMEM * 2 >= 2 * 64 * 64 * 4, "epilogue exchange must fit the tile buffers");
  constexpr uint32_t kKB = C::KBUF * 2, kVB = C::VBUF * 2;  // bytes per K / V buffer

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int br = w >> 1;     // softmax branch of this wave
  const int rh = w & 1;      // row half
  const int c = lane & 31;
  const int hh = lane >> 5;
  // Heads in chunks (chunked_block), heaviest row block first within a chunk: every row block of
  // one head lands on the same XCD (its K/V shared through one L2), heaviest first keeps the
  // causal tail short (a head-major order measured slower despite 6x less HBM fetch), and the
  // chunk bounds the K/V that the running workgroups stream at once to what the last-level cache
  // holds.  Without chunks, 256 heads at N = 4K (512 MB of K/V) ran 45 % slower than in chunks of
  // 64, from HBM; long sequences take 8 heads at a time, one per XCD, so that each XCD streams one
  // head's K/V (at N = 128K 4.5 % faster than all heads at once; a chunk's tail is short next to
  // its thousands of row blocks).
  int rb, hx;
  chunked_block(p.head_chunk, p.n_row_blocks, hx, rb);
  rb = p.n_row_blocks - 1 - rb;  // heaviest row block first
  const int row0 = rb * BM;
  const int wrow = row0 + 32 * rh;
  const int N = p.N;

  const int b = hx / p.heads;
  const int qh = hx % p.heads;


  // ---- this wave's Q^T operand (its own branch): lane holds row wrow + c, cols 16t + 8hh .. +7
  const bf16* qb = br == 0 ? static_cast<const bf16*>(p.q1) + b * p.sq1.sb + qh * p.sq1.sh
                           : static_cast<const bf16*>(p.q2) + b * p.sq2.sb + qh * p.sq2.sh;
  const int64_t qsn = br == 0 ? p.sq1.sn : p.sq2.sn;
  bf16x8 qf[C::TQ];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb, (uint32_t)(N * qsn * 2));
    const uint32_t r = (uint32_t)((wrow + c) * qsn * 2);
#pragma unroll
    for (int t = 0; t < C::TQ; ++t) qf[t] = __builtin_bit_cast(bf16x8, bload16(rq, r + 32 * t + 16 * hh));
    __builtin_amdgcn_s_waitcnt(0);  // settle Q before the asm tile DMA starts
  }

  const int kv_end = p.causal ? min(N, row0 + BM) : N;
  const int ntiles = (kv_end + kSBN - 1) / kSBN;
  // sliding window: the block's first row sees keys from row0 - window + 1 on
  const int t_begin = p.window > 0 ? max(0, row0 - p.window + 1) / kSBN : 0;
  // tiles this wave computes: from the tile holding its first row's first visible key up to its
  // last visible key
  const bool wave_has_rows = wrow < N;
  const int last_key = p.causal ? min(N, wrow + 32) : N;
  const int nt_wave = wave_has_rows ? min(ntiles, (last_key + kSBN - 1) / kSBN) : 0;
  const int t0_wave = p.window > 0 ? max(t_begin, max(0, wrow - p.window + 1) / kSBN) : 0;

  const uint32_t k1_row = (uint32_t)(p.sk1.sn * 2), k2_row = (uint32_t)(p.sk2.sn * 2);
  const uint32_t v_row = (uint32_t)(p.sv.sn * 2);
  const char* k1_base = static_cast<const char*>(p.k1) + 2 * (b * p.sk1.sb + qh * p.sk1.sh);
  const char* k2_base = static_cast<const char*>(p.k2) + 2 * (b * p.sk2.sb + qh * p.sk2.sh);
  const char* v_base = static_cast<const char*>(p.v) + 2 * (b * p.sv.sb + qh * p.sv.sh);

  // ---- tile loads.  Wave w issues the 1 KB DMA loads j = w + 4i of a K buffer (K1 then K2 in
  // V1) and of a V buffer.  Lane offsets are relative to the tile's first row, which moves into
  // the scalar buffer base.
  constexpr int KPW = C::K_LOADS / 4;  // per wave per K tensor
  constexpr int VPW = C::V_LOADS / 4;  // per wave, V
  uint32_t k_lane[C::NK][KPW];
  uint32_t v_lane[VPW];
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

  auto issue_k = [&](int kt, int buf) {
    bf16* kb = smem + buf * C::KBUF;
    const int rows_left = N - kt;
#pragma unroll
    for (int nk = 0; nk < C::NK; ++nk) {
      const uint32_t krow = nk == 0 ? k1_row : k2_row;
      const __amdgpu_buffer_rsrc_t rk =
          make_rsrc((nk == 0 ? k1_base : k2_base) + (size_t)kt * krow, (uint32_t)rows_left * krow);
#pragma unroll
      for (int i = 0; i < KPW; ++i) dma16(rk, kb + nk * C::K_ELEMS + 512 * (w + 4 * i), k_lane[nk][i]);
    }
  };
  auto issue_v = [&](int kt, int buf) {
    const int rows_left = N - kt;
    const __amdgpu_buffer_rsrc_t rvt = make_rsrc(v_base + (size_t)kt * v_row, (uint32_t)rows_left * v_row);
    bf16* vb = smem + NS * C::KBUF + buf * C::VBUF;
#pragma unroll
    for (int i = 0; i < VPW; ++i) dma16(rvt, vb + 512 * (w + 4 * i), v_lane[i]);
  };
  auto issue_tile = [&](int i) {
    issue_k(i * kSBN, i % NS);
    issue_v(i * kSBN, i % NS);
  };

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float mrun = kNegBig, lrun = 0.f;
  const float sl2 = p.scale_log2;
  float nmrun = -mrun * sl2;  // -m log2(e)/sqrt(d), updated whenever m moves

  // Per-lane LDS byte addresses of the MFMA operands, one register each; they flip to the other
  // buffer after use (one XOR).  Both swizzles act on address bits that the operand index only
  // XORs into, so operand t (or db) sits at base ^ (constant * t):
  //  K operand t of S^T: row c, 16-byte chunk (2t + hh) ^ swz(c), i.e. k_ad ^ 32 t.
  //  V^T operand db: two transposing reads; in each 16-lane group lane j addresses row
  //  4 hh + j / 4 (plus 16 u, and 8 for the upper read), channels 32 db + 16 dh + 4 (j % 4),
  //  whose 32-byte chunk db ^ (row & 3) puts it at v_ad ^ 64 db.
  uint32_t k_ad = 2u * (br * C::K_ELEMS + k_off<DQK>(c, 8 * hh));
  uint32_t v_ad;
  {
    const int j = lane & 15, dh = (lane >> 4) & 1;
    const int row = 4 * hh + (j >> 2);
    v_ad = 2u * (NS * C::KBUF + v_off(row, dh * 16 + 4 * (j & 3)));
  }
  const char* sb = reinterpret_cast<const char*>(smem);
  // max over the lane pair (l, l ^ 32) through ds_bpermute with a loop-invariant address
  const int bp_pair = (lane ^ 32) << 2;
  auto pmax = [&](float x) {
    return fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(bp_pair, __builtin_bit_cast(int, x))));
  };

  // K operand t of the next score tile; V^T operand db, lower or upper read, 16-key group u
  auto k_operand = [&](uint32_t kb, int t) { return *reinterpret_cast<const bf16x8*>(sb + (kb ^ (32u * t))); };
  auto v_read = [&](uint32_t vb, int db, int u, int upper) {
    return lds_read_tr(reinterpret_cast<const bf16*>(sb + (vb ^ (64u * db))) + (16 * u + 8 * upper) * kDV);
  };

  auto scores = [&](uint32_t kb) {
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int t = 0; t < C::TQ; ++t) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_operand(kb, t), qf[t], s, 0, 0, 0);
    return s;
  };
  // causal diagonal and ragged end only
  auto mask = [&](f32x16& s, int kt) {
    const bool below = p.window > 0 && kt <= wrow + 31 - p.window;  // tile reaches below a window
    if ((p.causal && kt + 31 > wrow) || kt + kSBN > N || below) {
      const int qrow = wrow + c;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kt + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key >= N || (p.causal && key > qrow) || (p.window > 0 && key <= qrow - p.window))
          s[r] = -INFINITY;
      }
    }
  };
  // weights exp2((s - m) log2(e) / sqrt(d)) for the reference max m, rounded to the two packed
  // P operands (16 keys each); tl gets the lane's sum of the rounded weights
  // (s is overwritten by the weights; the rare slow path forms the scores again from LDS)
  auto weights = [&](f32x16& e, bf16x8& p0, bf16x8& p1, float& tl) {
    const float nm = nmrun;
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(fmaf(e[r], sl2, nm));
    tl = 0.f;
    p0 = cvt8_sum(e, 0, tl);
    p1 = cvt8_sum(e, 8, tl);
  };

  // One tile of this wave's branch.  The softmax keeps a reference max m per row that moves only
  // when needed: the weights of a tile are formed against the current m, and only if some lane's
  // weight sum exceeds 2^kCap (a score beyond m + kCap in exp2 units, or the very first tile,
  // whose m is still -1e30) does the tile's exact row max get taken, the accumulators rescaled and
  // the weights formed again.  softmax(s) does not depend on m, so the result is the same as
  // with an exact running max.  kFirst: the wave's first tile, whose m starts at this tile's
  // exact row max straight from its scores (nothing is accumulated yet, so nothing rescales, and
  // every weight is at most 1).
  auto compute_tile = [&](int i, auto first_tag) {
    constexpr bool kFirst = decltype(first_tag)::value;
    const int kt = i * kSBN;
    const int buf = i % NS;
    const uint32_t kb = k_ad + buf * kKB;  // this tile's buffers (the swizzle XORs touch bits < 13)
    const uint32_t vb = v_ad + buf * kVB;
    __builtin_amdgcn_s_setprio(1);
    f32x16 s = scores(kb);
    __builtin_amdgcn_s_setprio(0);
    mask(s, kt);
    if constexpr (kFirst) {
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mrun = fmaxf(mrun, pmax(mx));
      nmrun = -mrun * sl2;
    }
    bf16x8 p0, p1;
    float tl;
    weights(s, p0, p1, tl);
    if (!kFirst && __any(!(tl <= kCapSum))) {
      // the K tile of this step is still in its buffer: form the scores again
      __builtin_amdgcn_s_setprio(1);
      s = scores(kb);
      __builtin_amdgcn_s_setprio(0);
      mask(s, kt);
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = pmax(mx);
      const float mnew = fmaxf(mrun, mx);
      const float alpha = exp2f((mrun - mnew) * sl2);
      mrun = mnew;
      nmrun = -mrun * sl2;
      lrun *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] *= alpha;
      weights(s, p0, p1, tl);
    }
    lrun += tl;

    // O^T += V^T P^T, 16 keys per MFMA
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bf16x8 pp = u == 0 ? p0 : p1;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const u32x2 lo = v_read(vb, db, u, 0);
        const u32x2 hi = v_read(vb, db, u, 1);
        const u32x4 a4 = {lo[0], lo[1], hi[0], hi[1]};
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4), pp, acc[db], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- main loop: loads of tile t+1 are in flight during the MFMAs of tile t.  A wave computes
  // the tiles up to its last visible key, then only helps load and meets the barriers, so that
  // the loop that carries the accumulators has no path around them.
  // Iteration i loads tile i + NS - 1 into the buffer tile i - 1 used, computes tile i, and waits
  // until tile i + 1 has landed: with NS > 2 the loads of the tiles after it stay in flight
  // (vmcnt counts this wave's outstanding buffer loads, which complete in order).
  constexpr int kLoadsPerTile = C::NK * KPW + VPW;  // DMA instructions per wave per tile
  auto wait_next = [&](int i) {
    if constexpr (NS == 2) {
      __builtin_amdgcn_s_waitcnt(0);
    } else {
      static_assert(NS == 3, "vmcnt for one younger tile in flight");
      if (i + 2 < ntiles) __builtin_amdgcn_s_waitcnt(kLoadsPerTile | (7 << 4) | (15 << 8));
      else __builtin_amdgcn_s_waitcnt(0);
    }
  };
  auto step = [&](int i, auto first_tag) {
    if (i + NS - 1 < ntiles) issue_tile(i + NS - 1);
    compute_tile(i, first_tag);
    wait_next(i);
    __syncthreads();
  };
#pragma unroll
  for (int i = 0; i < NS - 1; ++i) {
    if (t_begin + i < ntiles) issue_tile(t_begin + i);
  }
  if constexpr (NS == 2) {
    __builtin_amdgcn_s_waitcnt(0);
  } else {
    if (t_begin + 1 < ntiles) __builtin_amdgcn_s_waitcnt(kLoadsPerTile | (7 << 4) | (15 << 8));
    else __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
  // tiles before this wave's window only need its share of the loads and the barriers
  auto help = [&](int i) {
    if (i + NS - 1 < ntiles) issue_tile(i + NS - 1);
    wait_next(i);
    __syncthreads();
  };
  int it = t_begin;
  for (; it < t0_wave; ++it) help(it);
  if (it < nt_wave) step(it++, std::true_type{});
  for (; it < nt_wave; ++it) step(it, std::false_type{});
  for (; it < ntiles; ++it) help(it);

  // ---- epilogue: branch-2 waves publish lambda acc_2 / l_2; branch-1 waves finish the rows
  const float lam = head_lambda(p.lam, qh, lane);
  if (p.lam.out != nullptr && b == 0 && rb == 0 && w == 0 && lane == 0) p.lam.out[qh] = lam;
  // training forward: this branch's normalised output and log-sum-exp (base 2) per row
  if (p.stash_o != nullptr && wave_has_rows && wrow + c < N) {
    const float l = pair_sum(lrun);
    const float inv = 1.f / l;
    const int64_t row = (((int64_t)br * p.B + b) * p.heads + qh) * N + wrow + c;
    float* o = p.stash_o + row * kDV;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 x = {acc[db][4 * j] * inv, acc[db][4 * j + 1] * inv, acc[db][4 * j + 2] * inv,
                         acc[db][4 * j + 3] * inv};
        *reinterpret_cast<f32x4*>(o + db * 32 + 8 * j + 4 * hh) = x;
      }
    if (hh == 0) p.stash_lse[row] = mrun * sl2 + __log2f(l);
  }
  float* xb = reinterpret_cast<float*>(smem) + rh * (64 * 64);
  if (br == 1 && wave_has_rows) {
    const float i2 = lam / pair_sum(lrun);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) xb[(db * 16 + r) * 64 + lane] = acc[db][r] * i2;
  }
  __syncthreads();
  if (br == 1 || !wave_has_rows) return;
  const float i1 = 1.f / pair_sum(lrun);
  float o[4][16];
  float ss = 0.f;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float x = acc[db][r] * i1 - xb[(db * 16 + r) * 64 + lane];
      o[db][r] = x;
      ss = fmaf(x, x, ss);
    }
  float rs = 1.f;
  if (p.norm) {
    ss = pair_sum(ss);
    rs = p.out_scale * rsqrtf(ss * (1.f / kDV) + p.eps);
  }
  const int qrow = wrow + c;
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
  q.n_row_blocks = (p.N + 63) / 64;
  q.head_chunk = head_chunk((int64_t)p.B * p.heads, (int64_t)p.N * (2 * 64 + kDV) * 2);  // K1, K2, V
  const dim3 grid(p.B * p.heads, q.n_row_blocks);
  hipLaunchKernelGGL((prefill_kernel<64, kStagesV1>), grid, dim3(kThreads), 0, stream, q);
  return hipGetLastError();
}

}  // namespace da
