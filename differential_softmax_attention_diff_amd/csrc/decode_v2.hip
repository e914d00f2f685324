// One V2 decode step for gfx950: every sequence's new query token attends to its whole KV cache.
//
// What is computed (ai-engineering.academy "Atención Diferencial (V2)", section "V1 vs V2: la
// diferencia"): the two query heads (2p, 2p+1) of pair p read the same KV head
// g = p * Hkv / P; out_p = softmax(q_2p K^T / sqrt(D)) V - lambda_p softmax(q_2p+1 K^T / sqrt(D)) V.
// The page's point about V2 decode is that the KV cache is read once per step; here every K and V
// byte is read exactly once per step, serving all 2P/Hkv query heads of its KV head.
//
// Bandwidth-bound design (split-K over the cache, then a log-sum-exp merge):
//  * decode_partial: one 256-thread workgroup per (split s, KV head g, batch b) streams keys
//    [s*chunk, min(L, (s+1)*chunk)) in blocks of 256 (64 per wavefront):
//      - scores S = Q K^T with v_mfma_f32_16x16x32_bf16: the A operand holds the G query heads of
//        the KV head (rows G..15 zero), the B operand takes K rows straight from global memory;
//      - per-head block max / exp2 / sum by one wavefront per head over the 256 scores in LDS;
//      - P.V on the vector ALUs: 16 lanes cover one 256-byte V row (8 channels each) and read the
//        G weights of that key as an LDS broadcast;
//    it writes the split's (running max, running sum, un-normalised accumulator) per query head.
//  * decode_paged_balanced: the paged cache's sequences have their own lengths, so instead of
//    splitting each sequence, the blocks of all sequences are dealt in equal contiguous runs to as
//    many workgroups per KV head as the chip holds at once; a run covers pieces of one or more
//    sequences, each processed as above and written as its own partial.
//  * decode_combine: per (pair, batch) merges the splits of both heads by log-sum-exp, normalises,
//    and stores out = O_2p - lambda_p O_2p+1 in bf16.
#include <algorithm>
#include <mutex>

#include "device_common.hpp"
#include "launch.hpp"

namespace da {
namespace {

constexpr int kD = 128;
constexpr int kKB = 256;  // keys per block (64 per wavefront)
constexpr int kThreads = 256;
constexpr float kNegBig = -1.0e30f;
constexpr int kPagedRounds = 1;  // balanced paged pass: workgroups per resident slot
constexpr int kCombineBatch = 8;  // partial slots per head that the combine loads at once

// G = query heads per KV head (2P / Hkv): 2, 4, 8 or 16.  PAGED: the cache is a pool of pages
// [num_pages, Hkv, page_size, D] addressed through a per-sequence block table, and every sequence
// has its own length (the serving layout); otherwise [B, Hkv, L, D] with strides and one length.
template <int G, bool PAGED>
struct PartialLds {
  float sc[G][kKB];                             // scores of the block, per head
  __attribute__((aligned(16))) float pw[kKB][G];  // exp-weights, per key
  float alpha[G];
  float red[4][G][kD];
  int tab[PAGED ? 2 : 1][PAGED ? kKB : 1];      // page of each page-sized run of a block
};

// keys of paged sequence b: its length clamped to [0, L] and to the table's extent
__device__ __forceinline__ int paged_len(const DecodeParams& p, int b) {
  return (int)min((int64_t)max(p.seq_lens[b], 0), min((int64_t)p.L, (int64_t)p.max_blocks << p.page_shift));
}
__device__ __forceinline__ int n_blocks(int keys) { return (keys + kKB - 1) / kKB; }

// One piece of the cache of sequence b and KV head g: keys [k_begin, k_end) (k_begin a multiple
// of the block size) in blocks of 256.  Each query head hq of the KV head gets its (running max,
// running sum, un-normalised accumulator) at workspace row hq * ws_stride + ws_off.  Every thread
// of the workgroup calls it with the same arguments; it ends on a barrier, so that it can be
// called again for another piece.
template <int G, bool PAGED>
__device__ __forceinline__ void partial_range(const DecodeParams& p, PartialLds<G, PAGED>& sm, int b,
                                              int g, int k_begin, int k_end, int64_t ws_stride,
                                              int64_t ws_off) {
  constexpr int SLOTS = (G + 3) / 4;  // heads whose softmax state one wavefront owns
  auto& sc_lds = sm.sc;
  auto& pw_lds = sm.pw;
  auto& alpha_lds = sm.alpha;
  auto& red_lds = sm.red;
  auto& tab_lds = sm.tab;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l16 = lane & 15;
  const int grp = lane >> 4;
  const float c2 = p.scale_log2;

  const bf16* kbase = static_cast<const bf16*>(p.k) + b * p.sk.sb + g * p.sk.sh;
  const bf16* vbase = static_cast<const bf16*>(p.v) + b * p.sv.sb + g * p.sv.sh;
  // Paged: the page indices of a block's keys are staged in LDS one block ahead (a block of 256
  // keys starts on a multiple of 256, so it spans 256 / page_size pages, or lies inside one).
  // A page index outside the pool is clamped, so that a bad table entry cannot address memory
  // beyond it.
  const int32_t* btab = PAGED ? p.block_table + (int64_t)b * p.max_blocks : nullptr;
  const int page_mask = (1 << p.page_shift) - 1;
  const int tab_n = p.page_shift >= 8 ? 1 : kKB >> p.page_shift;  // pages per block
  auto fetch_tab = [&](int blk) -> int {  // this thread's entry for the block starting at blk
    const int e = (blk >> p.page_shift) + tid;
    return (tid < tab_n && e < p.max_blocks) ? min(max(btab[e], 0), p.num_pages - 1) : 0;
  };
  int cur = 0;
  auto row = [&](int key, int blk, int64_t sn, int tb) -> int64_t {  // tb: the table buffer
    if constexpr (PAGED) {
      const int pg = tab_lds[tb][(key >> p.page_shift) - (blk >> p.page_shift)];
      return (((int64_t)pg * p.Hkv + g) << p.page_shift | (key & page_mask)) * kD;
    } else {
      return (int64_t)key * sn;
    }
  };
  if constexpr (PAGED) {
    if (k_begin < k_end) tab_lds[0][tid] = fetch_tab(k_begin);
    __syncthreads();
  }

  // A operand: row m = l16 is query head g*G + l16 (zero rows beyond G); k = 32t + 8*grp + i
  bf16x8 qa[4];
  {
    u32x4 z = {0u, 0u, 0u, 0u};
    const int hq = g * G + l16;
    const int pair = hq >> 1;
    const bf16* qp = (hq & 1) ? static_cast<const bf16*>(p.q2) + b * p.sq2.sb + pair * p.sq2.sh
                              : static_cast<const bf16*>(p.q1) + b * p.sq1.sb + pair * p.sq1.sh;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const u32x4 x = l16 < G ? load16(qp + 32 * t + 8 * grp) : z;
      qa[t] = __builtin_bit_cast(bf16x8, x);
    }
  }

  float mrun[SLOTS], lrun[SLOTS];
#pragma unroll
  for (int j = 0; j < SLOTS; ++j) {
    mrun[j] = kNegBig;
    lrun[j] = 0.f;
  }
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  // A block's K rows are loaded while the block before it finishes: into the registers its score
  // products are done with, as soon as they are (3.5 % faster at the 32K workload); V at the
  // block's start.  Where that would take more than 256 registers (one wave per SIMD) -- G = 8
  // with a paged cache, G = 16 -- K is loaded at the block's start instead.
  constexpr bool kEarlyK = G <= 4 || (G == 8 && !PAGED);
  u32x4 kf[4][4];
  auto load_k = [&](int blk, int tb) {
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      const int key = blk + 64 * w + 16 * sb + l16;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        kf[sb][t] = key < k_end ? load16_nt(kbase + row(key, blk, p.sk.sn, tb) + 32 * t + 8 * grp)
                                : u32x4{0u, 0u, 0u, 0u};
    }
  };
  if (kEarlyK && k_begin < k_end) load_k(k_begin, 0);
  for (int blk = k_begin; blk < k_end; blk += kKB) {
    // paged: the next block's page indices are loaded now and published once this block's scores
    // are formed (the previous block's table, in that buffer, is no longer read by then)
    int tab_next = 0;
    if constexpr (PAGED) {
      if (blk + kKB < k_end) tab_next = fetch_tab(blk + kKB);
    }
    if constexpr (!kEarlyK) load_k(blk, cur);
    u32x4 vf[16];
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int key = blk + 64 * w + 4 * st + grp;
      vf[st] = key < k_end ? load16_nt(vbase + row(key, blk, p.sv.sn, cur) + 8 * l16) : u32x4{0u, 0u, 0u, 0u};
    }

    // scores: D[m = head 4*grp + r][n = key l16] for 16 keys per MFMA group
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[t], __builtin_bit_cast(bf16x8, kf[sb][t]), s, 0, 0, 0);
      const int kl = 64 * w + 16 * sb + l16;
      const bool valid = blk + kl < k_end;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * grp + r;
        if (h < G) sc_lds[h][kl] = valid ? s[r] : -INFINITY;
      }
    }
    if constexpr (PAGED) {
      tab_lds[cur ^ 1][tid] = tab_next;
    } else if constexpr (kEarlyK) {
      if (blk + kKB < k_end) load_k(blk + kKB, 0);
    }
    __syncthreads();
    if constexpr (PAGED && kEarlyK) {
      if (blk + kKB < k_end) load_k(blk + kKB, cur ^ 1);
    }

    // per-head block softmax statistics (wavefront w owns heads w, w+4, ...)
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
      const int h = w + 4 * j;
      if (h < G) {
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = sc_lds[h][lane + 64 * i];
        const float mx = wave_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
        const float mnew = fmaxf(mrun[j], mx);
        const float alpha = exp2f((mrun[j] - mnew) * c2);
        mrun[j] = mnew;
        const float nm = -mnew * c2;
        float ls = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(fmaf(x[i], c2, nm));
          pw_lds[lane + 64 * i][h] = e;
          ls += e;
        }
        lrun[j] = lrun[j] * alpha + wave_sum(ls);
        if (lane == 0) alpha_lds[h] = alpha;
      }
    }
    __syncthreads();

    // P.V: lane covers channels 8*l16 .. +7 of keys 64w + 4st + grp
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float a = alpha_lds[h];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= a;
    }
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int kl = 64 * w + 4 * st + grp;
      float vv[8];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        vv[2 * m] = bf16_lo(vf[st][m]);
        vv[2 * m + 1] = bf16_hi(vf[st][m]);
      }
      if constexpr (G >= 4) {
#pragma unroll
        for (int h4 = 0; h4 < G; h4 += 4) {
          const f32x4 pw = *reinterpret_cast<const f32x4*>(&pw_lds[kl][h4]);
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h4 + r][e] = fmaf(pw[r], vv[e], acc[h4 + r][e]);
        }
      } else {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        const f32x2 pw = *reinterpret_cast<const f32x2*>(&pw_lds[kl][0]);
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(pw[r], vv[e], acc[r][e]);
      }
    }
    if constexpr (PAGED) cur ^= 1;
    __syncthreads();
  }

  // reduce the four key groups of each wavefront, then the four wavefronts
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[h][e];
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc[h][e] = x;
    }
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) red_lds[w][h][8 * l16 + e] = acc[h][e];
  }
  // softmax statistics of the piece
#pragma unroll
  for (int j = 0; j < SLOTS; ++j) {
    const int h = w + 4 * j;
    if (h < G && lane == 0) {
      const int hq = g * G + h;
      float* ml = p.ws_ml + ((int64_t)hq * ws_stride + ws_off) * 2;
      ml[0] = mrun[j];
      ml[1] = lrun[j];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * kD; idx += kThreads) {
    const int h = idx / kD;
    const int ch = idx % kD;
    const float s = red_lds[0][h][ch] + red_lds[1][h][ch] + red_lds[2][h][ch] + red_lds[3][h][ch];
    const int hq = g * G + h;
    p.ws_acc[((int64_t)hq * ws_stride + ws_off) * kD + ch] = s;
  }
  __syncthreads();  // the LDS is free for the next piece
}

// Per-sequence splits: workgroup (split, g, b) takes an equal share of sequence b's blocks.
template <int G, bool PAGED>
__global__ __launch_bounds__(kThreads) void decode_partial_kernel(const DecodeParams p) {
  __shared__ PartialLds<G, PAGED> sm;
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int seq_len = PAGED ? paged_len(p, b) : p.L;
  // the sequence's 256-key blocks are dealt evenly to the splits, so that with per-sequence
  // lengths every split of a sequence gets the same share (empty only when it has fewer blocks
  // than splits)
  const int nblk = n_blocks(seq_len);
  const int k_begin = (int)(((int64_t)split * nblk) / p.splits) * kKB;
  const int k_end = min(seq_len, (int)(((int64_t)(split + 1) * nblk) / p.splits) * kKB);
  partial_range<G, PAGED>(p, sm, b, g, k_begin, k_end, p.splits, (int64_t)b * 2 * p.P * p.splits + split);
}

// inclusive prefix sum over the wavefront
__device__ __forceinline__ int64_t wave_incl_scan(int64_t x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}
__device__ __forceinline__ int64_t wave_sum64(int64_t x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

// Paged cache, balanced over uneven lengths: the blocks of all sequences, taken in sequence
// order (TB in all), are dealt to the NW = gridDim.y workgroups of a KV head in equal contiguous
// runs (grid x = KV head, so that the KV heads of a run, which read the same pages, start
// together: 1.4 % faster than the other way round); workgroup w takes global blocks [w TB / NW, (w + 1) TB / NW).  A run may start or end
// inside a sequence and may cover several; each (workgroup w, sequence b) piece writes its
// partial at slot w + b of the query head's NW + B slots.  Slots are unique: along the runs both
// w and b only grow, and each step moves at least one of them.
template <int G>
__global__ __launch_bounds__(kThreads) void decode_paged_balanced_kernel(const DecodeParams p) {
  __shared__ PartialLds<G, true> sm;
  __shared__ int64_t red64[kThreads / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int wg = blockIdx.y;
  const int g = blockIdx.x;  // the KV heads of one run are dispatched together
  const int64_t nw = gridDim.y;
  int64_t part = 0;
  for (int b = tid; b < p.B; b += kThreads) part += n_blocks(paged_len(p, b));
  part = wave_sum64(part);
  if (lane == 0) red64[wv] = part;
  __syncthreads();
  int64_t tb = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) tb += red64[i];
  const int64_t x0 = wg * tb / nw;
  const int64_t x1 = (wg + 1) * tb / nw;
  if (x0 >= x1) return;  // the same for every thread
  // first sequence of the run: the first b whose blocks end past x0 (each wavefront finds it)
  int64_t base = 0;  // global index of sequence b's first block
  int b = p.B;
  for (int c = 0; c < p.B; c += 64) {
    const int bb = c + lane;
    const int64_t n = bb < p.B ? n_blocks(paged_len(p, bb)) : 0;
    const int64_t incl = wave_incl_scan(n, lane);
    const uint64_t hit = __ballot(base + incl > x0);
    if (hit != 0) {
      const int l = __ffsll((unsigned long long)hit) - 1;
      b = c + l;
      base += __shfl(incl - n, l);
      break;
    }
    base += __shfl(incl, 63);
  }
  for (; b < p.B && base < x1; ++b) {
    const int len = paged_len(p, b);
    const int nb = n_blocks(len);
    const int64_t lo = max(x0, base) - base;
    const int64_t hi = min(x1, base + nb) - base;
    if (lo < hi)
      partial_range<G, true>(p, sm, b, g, (int)lo * kKB, min(len, (int)hi * kKB), nw + p.B, wg + b);
    base += nb;
  }
}

__global__ __launch_bounds__(kD) void decode_combine_kernel(const DecodeParams p) {
  __shared__ int64_t red64[2][kD / 64];
  const int pair = blockIdx.x;
  const int b = blockIdx.y;
  const int ch = threadIdx.x;
  const int lane = ch & 63;
  const float lam = head_lambda(p.lam, pair, lane);
  if (p.lam.out != nullptr && b == 0 && ch == 0) p.lam.out[pair] = lam;
  const int two_p = 2 * p.P;
  // this sequence's partials: rows hq * stride + first .. + last of the query head hq
  int64_t stride = p.splits, first = (int64_t)b * two_p * p.splits, last = first + p.splits - 1;
  int64_t tot_blocks = 0;
  if (p.stream_wgs > 0) {
    // the balanced paged pass: the workgroups whose runs of blocks meet this sequence's
    int64_t tot = 0, pre = 0;
    for (int i = ch; i < p.B; i += kD) {
      const int64_t n = n_blocks(paged_len(p, i));
      tot += n;
      if (i < b) pre += n;
    }
    tot = wave_sum64(tot);
    pre = wave_sum64(pre);
    if (lane == 0) {
      red64[0][ch >> 6] = tot;
      red64[1][ch >> 6] = pre;
    }
    __syncthreads();
    tot = red64[0][0] + red64[0][1];
    pre = red64[1][0] + red64[1][1];
    const int64_t nw = p.stream_wgs;
    const int64_t nb = n_blocks(paged_len(p, b));
    // the workgroup whose run [w tot / nw, (w + 1) tot / nw) holds global block x
    auto owner = [&](int64_t x) { return ((x + 1) * nw + tot - 1) / tot - 1; };
    stride = nw + p.B;
    first = nb > 0 ? owner(pre) + b : 0;
    last = nb > 0 ? owner(pre + nb - 1) + b : -1;
    tot_blocks = tot;
  }
  // with more workgroups than blocks some runs are empty, and their slots hold nothing
  auto skip = [&](int64_t s) {
    if (p.stream_wgs == 0) return false;
    const int64_t w = s - b;
    return w * tot_blocks / p.stream_wgs == (w + 1) * tot_blocks / p.stream_wgs;
  };
  float o[2];
  if (last - first < kCombineBatch) {
    // every partial of both heads loaded at once (their loads in flight together), then merged
    // in slot order
    bool use[kCombineBatch];
    float mv[2][kCombineBatch], lv[2][kCombineBatch], av[2][kCombineBatch];
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) use[i] = first + i <= last && !skip(first + i);
#pragma unroll
    for (int br = 0; br < 2; ++br) {
      const int hq = 2 * pair + br;
      const float* ml = p.ws_ml + (hq * stride) * 2;
      const float* ac = p.ws_acc + (hq * stride) * kD;
#pragma unroll
      for (int i = 0; i < kCombineBatch; ++i) {
        const int64_t s = first + i;
        mv[br][i] = kNegBig;
        lv[br][i] = av[br][i] = 0.f;
        if (use[i]) {
          mv[br][i] = ml[2 * s];
          lv[br][i] = ml[2 * s + 1];
          av[br][i] = ac[s * kD + ch];
        }
      }
    }
#pragma unroll
    for (int br = 0; br < 2; ++br) {
      float m = kNegBig;
#pragma unroll
      for (int i = 0; i < kCombineBatch; ++i) m = fmaxf(m, mv[br][i]);
      float l = 0.f, x = 0.f;
#pragma unroll
      for (int i = 0; i < kCombineBatch; ++i) {
        if (use[i]) {
          const float wgt = exp2f((mv[br][i] - m) * p.scale_log2);
          l = fmaf(lv[br][i], wgt, l);
          x = fmaf(av[br][i], wgt, x);
        }
      }
      o[br] = x / l;
    }
  } else {
#pragma unroll
    for (int br = 0; br < 2; ++br) {
      const int hq = 2 * pair + br;
      const float* ml = p.ws_ml + (hq * stride) * 2;
      const float* ac = p.ws_acc + (hq * stride) * kD;
      float m = kNegBig;
      for (int64_t s = first; s <= last; ++s)
        if (!skip(s)) m = fmaxf(m, ml[2 * s]);
      float l = 0.f, x = 0.f;
      for (int64_t s = first; s <= last; ++s) {
        if (skip(s)) continue;
        const float wgt = exp2f((ml[2 * s] - m) * p.scale_log2);
        l = fmaf(ml[2 * s + 1], wgt, l);
        x = fmaf(ac[s * kD + ch], wgt, x);
      }
      o[br] = x / l;
    }
  }
  bf16* out = static_cast<bf16*>(p.out) + b * p.so.sb + pair * p.so.sh;
  out[ch] = (bf16)(o[0] - lam * o[1]);
}

template <int G, bool PAGED>
hipError_t launch_partial(const DecodeParams& p, hipStream_t stream) {
  if (PAGED && p.stream_wgs > 0) {
    hipLaunchKernelGGL((decode_paged_balanced_kernel<G>), dim3(p.Hkv, p.stream_wgs), dim3(kThreads), 0,
                       stream, p);
  } else {
    hipLaunchKernelGGL((decode_partial_kernel<G, PAGED>), dim3(p.splits, p.Hkv, p.B), dim3(kThreads), 0,
                       stream, p);
  }
  return hipGetLastError();
}

template <bool PAGED>
hipError_t launch_step(const DecodeParams& p, hipStream_t stream) {
  const int G = 2 * p.P / p.Hkv;
  hipError_t e;
  switch (G) {
    case 2: e = launch_partial<2, PAGED>(p, stream); break;
    case 4: e = launch_partial<4, PAGED>(p, stream); break;
    case 8: e = launch_partial<8, PAGED>(p, stream); break;
    case 16: e = launch_partial<16, PAGED>(p, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(p.P, p.B), dim3(kD), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_v2(const DecodeParams& p, hipStream_t stream) {
  return launch_step<false>(p, stream);
}

// ---------------------------------------------------------------------------------------------
// Scratch of the allocation-free decode entry point: the split partials live in this fixed
// device array instead of a caller workspace.  Each GPU the library runs on holds its own copy
// (until the process ends).  In host code `scratch` names a host-side stand-in, not device
// memory, so its device address is looked up once per device (with that device current) and
// only that address is handed to the kernels.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

void* noalloc_scratch() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    addr[dev] = ptr;
  }
  return addr[dev];
}

hipError_t launch_decode_v2_paged(const DecodeParams& p, hipStream_t stream) {
  // Uneven lengths would leave the per-sequence splits uneven too (the longest sequences' pieces
  // forming the tail), so the blocks of all sequences are dealt evenly to as many workgroups as
  // the chip holds at once (2 per CU, 1 for G = 16, whose registers allow one wave per SIMD),
  // within the partial rows the workspace has: 2P (NW + B) <= 2P B splits.
  DecodeParams q = p;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipErrorInvalidDevice;
  const int G = 2 * p.P / p.Hkv;
  const int64_t resident = (int64_t)cus * (G == 16 ? 1 : 2) * kPagedRounds;
  const int64_t nw = (resident + p.Hkv - 1) / p.Hkv;
  const int64_t cap = (int64_t)p.B * (p.splits - 1);
  q.stream_wgs = (int)std::min<int64_t>(std::min<int64_t>(nw, cap), 65535);  // grid y
  // For G = 8 the balanced kernel needs more than 256 registers (one wave per SIMD) where the
  // per-sequence one fits in 248 (two), which is worth more than the balance.
  if (G == 8) q.stream_wgs = 0;
  return launch_step<true>(q, stream);
}

}  // namespace da
