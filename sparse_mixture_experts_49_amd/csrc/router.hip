// Router of the MoE layer on gfx950: logits on MFMA, then softmax, top-k and the
// routing weights in registers, plus the per-block partial sums of the aux loss.
//
// Web page "Mixture of Experts: Scaling Parameters Without Scaling Compute",
// section "The MoE layer": logits g = W_r x, p = softmax(g), keep the top-k
// experts, renormalise the chosen probabilities.  Section "The central
// problem: load balancing": aux = E * sum_i f_i P_i with f_i the fraction of
// tokens whose first choice is i and P_i the mean router probability.
//
// Ranking is by logit (softmax is monotone), descending; equal logits go to
// the lower expert index, the order a stable descending sort gives.  An
// optional per-expert selection bias is added to the ranking scores only
// (same page and section: auxiliary-loss-free balancing); the weights stay the
// unbiased probabilities.  The router z-loss is the mean over tokens of the
// squared log-sum-exp of the logits (same section: router z-loss).
#include "device_common.h"
#include "kernels.h"
#include "aux_reduce.h"
#include "perm_small.h"

namespace moe {

constexpr int kRouterTile = 16;     // tokens per MFMA row tile
constexpr int kAuxThreads = 1024;   // threads of the single aux-reduction block
constexpr int kRouterWaves = 8;     // the block's waves split d between them

// LDS of a block of MT token tiles: the waves' partial logits, then each
// token's probabilities, first choice and log-sum-exp for the aux and z-loss
// sums, and (reroute policy) its ranking keys and weights.
// A token's ranking as one unsigned compare: the score's bits mapped to an
// integer of the same order (-0 taken as +0, as the float compare does) above,
// 63 - e below, so the larger key is the higher score, or the lower index on
// equal scores.  Valid keys are > 0.
__device__ __forceinline__ uint64_t rank_key(float s, int e) {
  const uint32_t b = __float_as_uint(s == 0.f ? 0.f : s);
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)(63 - e);
}

template <int WAVES, int MT>
struct RouterTileLds {
  float red[WAVES][kRouterTile * MT][65];
  float prob[kRouterTile * MT][64];
  uint64_t rkey[kRouterTile * MT][64];
  float rwt[kRouterTile * MT][64];
  int top1[kRouterTile * MT];
  int sel[kRouterTile * MT][8];
  float lse[kRouterTile * MT];
  double wps[MT][64];      // WSUM: per finishing wave, sum of p over its tokens per expert
  int wcnt[MT][64];        //   its first-choice count per expert
  double wz[MT];           //   its sum of squared log-sum-exp
};

// Tokens t0 .. t0 + 16*MT - 1 of the router: logits on MFMA (the WAVES waves
// split d), softmax, top-k and the routing weights; fills sm.prob / top1 / lse
// (and, with `rr`, sm.rkey / rwt).  Ends with a barrier.  Wave w accumulates
// the k-chunks w, w+WAVES, ... of the d-long dot products; the partial logit
// tiles are summed in wave order through LDS, so the result does not depend on
// scheduling.
//
// Lane layout of the loads: lane l reads row (l % 16) -- a token of x, or an
// expert row of W_r -- and in load q of a chunk the 16 bytes at offset
// q * 64 + (l / 16) * 16 of the row's 256-byte chunk, so the four lanes of a
// row cover 64 contiguous bytes (half a cache line) per instruction.  MFMA q of
// the chunk consumes load q; A and B use the same map, so each MFMA sums 32
// (bf16) or 16 (fp32, four MFMAs) consecutive k.
template <int WAVES, int MT, int MAXPER = 16, int KMAX = 8, bool WSUM = false>
__device__ __forceinline__ void route_finish(
    const float* __restrict__ br, const float* __restrict__ bsel, int T_, int E, int k, int renorm,
    int t0, bool rr, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    RouterTileLds<WAVES, MT>& sm);

template <typename T, int NT, int WAVES, int MT, int MAXPER = 16, int KMAX = 8>
__device__ __forceinline__ void route_tile(
    const T* __restrict__ x, const T* __restrict__ wr, const float* __restrict__ br,
    const float* __restrict__ bsel, int T_, int d, int E, int k, int renorm, int t0, bool rr,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, RouterTileLds<WAVES, MT>& sm) {
  constexpr int kPerVec = 16 / sizeof(T);           // elements per 16-byte piece
  constexpr int kChunk = 16 * kPerVec;              // 128 bf16 or 64 fp32 = 256 bytes
  auto& red = sm.red;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, c = lane >> 4;
  const T* xrow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
    xrow[m] = x + (size_t)min(t0 + 16 * m + r, T_ - 1) * d + c * kPerVec;
  const T* wrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) wrow[nt] = wr + (size_t)min(nt * 16 + r, E - 1) * d + c * kPerVec;

  f32x4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[m][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nch = d / kChunk;
  auto load_chunk = [&](int ch, u32x4 (&a)[MT][4], u32x4 (&b)[NT][4]) {
    const int kk = ch * kChunk;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q) a[m][q] = ld16(xrow[m] + kk + q * 4 * kPerVec);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q) b[nt][q] = ld16(wrow[nt] + kk + q * 4 * kPerVec);
  };
  auto mma_chunk = [&](const u32x4 (&a)[MT][4], const u32x4 (&b)[NT][4]) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[m][nt] = mfma_bf16(a[m][q], b[nt][q], acc[m][nt]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[m][nt] = mfma_f32(__uint_as_float(a[m][q][i]), __uint_as_float(b[nt][q][i]), acc[m][nt]);
        }
      }
  };
  // Two chunks per iteration, both loaded before either is multiplied: with
  // few tokens (decode) the loop is bound by load latency.  The chunks are
  // accumulated in order ch = wave, wave + WAVES, ... either way.
  int ch = wave;
  for (; ch + WAVES < nch; ch += 2 * WAVES) {
    u32x4 a0[MT][4], b0[NT][4], a1[MT][4], b1[NT][4];
    load_chunk(ch, a0, b0);
    load_chunk(ch + WAVES, a1, b1);
    mma_chunk(a0, b0);
    mma_chunk(a1, b1);
  }
  if (ch < nch) {
    u32x4 a0[MT][4], b0[NT][4];
    load_chunk(ch, a0, b0);
    mma_chunk(a0, b0);
  }
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][16 * m + 4 * c + i][nt * 16 + r] = acc[m][nt][i];

  route_finish<WAVES, MT, MAXPER, KMAX>(br, bsel, T_, E, k, renorm, t0, rr, topk_idx, topk_w, sm);
}

// The rest of a token tile once the partial logit tiles sit in sm.red[0 ..
// WAVES-1] (summed here in that order): softmax, top-k, the routing weights,
// sm.prob / top1 / lse / sel (and, with `rr`, sm.rkey / rwt).  Wave m < MT
// finishes tile m.  Starts and ends with a barrier.  MAXPER >= ceil(E / 4)
// (experts per lane) and KMAX >= k bound the unrolled loops: the code runs
// once per launch from a cold instruction cache, so its size is its latency.
// WSUM: each finishing wave also sums, over its tokens below T_, p per expert,
// first choices per expert and the squared log-sum-exp (fixed xor trees over
// the quads) into sm.wps / wcnt / wz.
template <int WAVES, int MT, int MAXPER, int KMAX, bool WSUM>
__device__ __forceinline__ void route_finish(
    const float* __restrict__ br, const float* __restrict__ bsel, int T_, int E, int k, int renorm,
    int t0, bool rr, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    RouterTileLds<WAVES, MT>& sm) {
  auto& red = sm.red;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // The bias words of the lane's experts (quarter q of a quad holds experts q, q+4,
  // ...), all issued before the barrier so that their latency overlaps it rather
  // than adding one round trip per expert to the epilogue.
  constexpr int kMaxPer = MAXPER;
  float bb[kMaxPer], bs[kMaxPer];
  {
    const int q = lane & 3;
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      bb[j] = 0.f;
      bs[j] = 0.f;
    }
    if (wave < MT) {
      if (br) {
#pragma unroll
        for (int j = 0; j < kMaxPer; ++j)
          if (4 * j < E) bb[j] = br[min(q + 4 * j, E - 1)];
      }
      if (bsel) {
#pragma unroll
        for (int j = 0; j < kMaxPer; ++j)
          if (4 * j < E) bs[j] = bsel[min(q + 4 * j, E - 1)];
      }
    }
  }
  __syncthreads();

  if (wave < MT) {
    // Wave w finishes token tile w.  Four lanes per token: lane quarter q holds
    // experts q, q+4, q+8, ...
    const int tq = lane >> 2, q = lane & 3;
    const int tr = 16 * wave + tq;                   // token row of the block
    const int t = t0 + tr;
    float g[kMaxPer], p[kMaxPer], sc[kMaxPer];
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      const int e = q + 4 * j;
      g[j] = -INFINITY;
      if (e < E) {
        g[j] = red[0][tr][e];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) g[j] += red[w][tr][e];   // in wave order
        if (br) g[j] += bb[j];
        m = fmaxf(m, g[j]);
      }
    }
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      p[j] = (q + 4 * j < E) ? expf(g[j] - m) : 0.f;
      s += p[j];
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    const float inv = 1.0f / s;
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      p[j] *= inv;
      const int e = q + 4 * j;
      sc[j] = (bsel && e < E) ? g[j] + bs[j] : g[j];     // ranking scores
    }
    const float lse_t = m + logf(s);
    if (q == 0) sm.lse[tr] = lse_t;

    // top-k: k rounds of a quad-wide argmax over the unselected logits.
    uint32_t taken = 0;
    int sel_e[KMAX];
    float sel_p[KMAX];
#pragma unroll
    for (int sl = 0; sl < KMAX; ++sl) {
      sel_e[sl] = 0;
      sel_p[sl] = 0.f;
      if (sl < k) {
        float bv = -INFINITY, bp = 0.f;
        int be = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < kMaxPer; ++j) {
          const int e = q + 4 * j;
          if (e < E && !((taken >> j) & 1u) && (sc[j] > bv || be == 0x7fffffff)) {
            bv = sc[j];
            be = e;
            bp = p[j];
          }
        }
#pragma unroll
        for (int off = 1; off <= 2; off <<= 1) {
          const float ov = __shfl_xor(bv, off);
          const int oe = __shfl_xor(be, off);
          const float op = __shfl_xor(bp, off);
          if (ov > bv || (ov == bv && oe < be)) {
            bv = ov;
            be = oe;
            bp = op;
          }
        }
        if ((be & 3) == q) taken |= 1u << (be >> 2);
        sel_e[sl] = be;
        sel_p[sl] = bp;
      }
    }
    float wsum = 0.f;
#pragma unroll
    for (int sl = 0; sl < KMAX; ++sl)
      if (sl < k) wsum += sel_p[sl];
    const float winv = renorm ? 1.0f / wsum : 1.0f;
    if (t < T_ && q == 0) {
#pragma unroll
      for (int sl = 0; sl < KMAX; ++sl) {
        if (sl < k) {
          topk_idx[(size_t)t * k + sl] = sel_e[sl];
          topk_w[(size_t)t * k + sl] = renorm ? sel_p[sl] * winv : sel_p[sl];
        }
      }
    }
    if (rr) {                                        // inputs of the expert ranking (all 64 keys)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int e = q + 4 * j;                     // rows of 64, key 0 past E
        if (j < kMaxPer) {
          sm.rkey[tr][e] = e < E ? rank_key(sc[j], e) : 0ull;
          sm.rwt[tr][e] = renorm ? p[j] * winv : p[j];
        } else {
          sm.rkey[tr][e] = 0ull;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      const int e = q + 4 * j;
      if (e < E) sm.prob[tr][e] = (t < T_) ? p[j] : 0.f;
    }
    if (q == 0) sm.top1[tr] = (t < T_) ? sel_e[0] : -1;
    if (q == 0) {
#pragma unroll
      for (int sl = 0; sl < KMAX; ++sl)
        if (sl < k) sm.sel[tr][sl] = (t < T_) ? sel_e[sl] : -1;
    }
    if constexpr (WSUM) {
      const bool valid = t < T_;
#pragma unroll
      for (int j = 0; j < kMaxPer; ++j) {
        const int e = q + 4 * j;
        double v = valid ? (double)p[j] : 0.0;
        int c = (valid && sel_e[0] == e) ? 1 : 0;
#pragma unroll
        for (int off = 4; off < 64; off <<= 1) {
          v += __shfl_xor(v, off);
          c += __shfl_xor(c, off);
        }
        if (tq == 0 && e < E) {
          sm.wps[wave][e] = v;
          sm.wcnt[wave][e] = c;
        }
      }
      double z = (q == 0 && valid) ? (double)lse_t * (double)lse_t : 0.0;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) z += __shfl_xor(z, off);
      if (lane == 0) sm.wz[wave] = z;
    }
  }
  __syncthreads();
}

// One block = 16*MT tokens x all experts, W waves splitting d.  The block then
// writes its partial sums of the aux loss and z-loss for aux_finalize_kernel
// and, for the reroute policy, every token's experts in ranking order.
// MAXPER and KMAX as in route_finish: instantiated for the layer's expert and
// slot counts (measured on MI355X: the finish took 10.4 us per 32-token block
// of the Switch-style layer and 5.5 us per 16-token block of the prefill layer
// with the 64-expert, 8-slot code).
template <typename T, int NT, int MT, int W, int MAXPER, int KMAX>
__global__ __launch_bounds__(W * 64) void router_kernel(
    const T* __restrict__ x, const T* __restrict__ wr, const float* __restrict__ br,
    const float* __restrict__ bsel, int T_, int d, int E, int k, int renorm,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    double* __restrict__ part_psum, int32_t* __restrict__ part_top1, double* __restrict__ part_z,
    int32_t* __restrict__ rr_rank) {
  __shared__ RouterTileLds<W, MT> sm;
  constexpr int kTok = kRouterTile * MT;
  const int t0 = blockIdx.x * kTok;
  route_tile<T, NT, W, MT, MAXPER, KMAX>(x, wr, br, bsel, T_, d, E, k, renorm, t0, rr_rank != nullptr,
                                         topk_idx, topk_w, sm);
  auto& prob = sm.prob;
  auto& top1 = sm.top1;
  auto& lse = sm.lse;
  // Per-block partials of the aux loss, summed in token order.
  if (threadIdx.x < E) {
    const int e = threadIdx.x;
    double ps = 0.0;
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < kTok; ++i) {
      ps += (double)prob[i][e];
      cnt += (top1[i] == e);
    }
    part_psum[(size_t)blockIdx.x * E + e] = ps;
    part_top1[(size_t)blockIdx.x * E + e] = cnt;
  }
  if (threadIdx.x == 64) {                           // z-loss partial, token order
    double z = 0.0;
    for (int i = 0; i < kTok && t0 + i < T_; ++i) z += (double)lse[i] * (double)lse[i];
    part_z[blockIdx.x] = z;
  }
  if (rr_rank) {
    // The token's experts in ranking order (higher score first, equal scores
    // by lower index): expert e goes to position = the number of experts
    // ranked above it, as {e, weight bits}.  Lanes of a wave take the 64
    // experts of one token, so the score reads are LDS broadcasts.
#pragma unroll 1
    for (int idx = threadIdx.x; idx < kTok * 64; idx += W * 64) {
      const int tr = idx >> 6, e = idx & 63, t = t0 + tr;
      if (e >= E || t >= T_) continue;
      const uint64_t key = sm.rkey[tr][e];
      int pos = 0;
#pragma unroll
      for (int j = 0; j < 64; ++j) pos += (int)(sm.rkey[tr][j] > key);
      typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
      *reinterpret_cast<i32x2*>(rr_rank + ((size_t)t * 64 + pos) * 2) =
          i32x2{e, (int32_t)__float_as_uint(sm.rwt[tr][e])};
    }
  }
}

// The router partials reduced in a fixed order (aux_reduce), then the small
// layers' dispatch layout.
__global__ __launch_bounds__(kAuxThreads) void aux_finalize_kernel(
    const double* __restrict__ part_psum, const int32_t* __restrict__ part_top1,
    const double* __restrict__ part_z, int nblk, int T_, int E, int32_t* __restrict__ top1_count,
    float* __restrict__ prob_mean, float* __restrict__ aux, float* __restrict__ z_loss,
    int32_t* __restrict__ rounds_zero, const int32_t* __restrict__ topk_idx, int k, bool perm,
    int capacity, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ dest, int32_t* __restrict__ src) {
  __shared__ AuxLds<kAuxThreads> ared;
  constexpr int kBatches = kPermWide / kAuxThreads;
  __shared__ PermLayoutLds<kAuxThreads / 64, kBatches, false> psm;
  // Small layers: the dispatch layout too, saving the permute's own launch.  Its
  // loads are issued first, so that their latency overlaps the reduction's.
  int ex[kBatches];
  if (perm) perm_load<kAuxThreads / 64, kBatches>(topk_idx, T_ * k, ex);
  aux_reduce<kAuxThreads>(part_psum, part_top1, part_z, nblk, T_, E, top1_count, prob_mean, aux,
                          z_loss, ared);
  if (threadIdx.x == 128 && rounds_zero) *rounds_zero = 0;
  if (perm)
    perm_layout<kAuxThreads / 64, kBatches, false>(ex, T_, k, E, capacity, true, counts, offsets,
                                                   dest, src, psm);
}

// ---------------------------------------------------------------------------
// Small batches (at most kSmallTokens tokens, drop policy).  The tile router
// above gives a decode batch of 32 tokens two blocks, and each spends most of
// its time pulling its ~190 KB of x and W_r into one CU (measured: ~6.8 us of
// loads at d = 4096, the same with 16 waves as with 8).  Here the dot products
// are split along d instead: one wave per (d-range, token tile) computes a
// partial logit tile from a few 256-byte chunks of each row, so every load
// of the layer is in flight at once across the chip; then a single block sums
// the partial tiles in d order, finishes the tokens (route_finish), reduces the
// aux loss and z-loss directly from its own LDS, and lays out the dispatch --
// the same two launches as router + aux block, with the long load phase spread
// over many CUs.
// ---------------------------------------------------------------------------
constexpr int kSmallTokens = 64;        // 4 token tiles: the finishing block's waves 0..3
constexpr int kSmallSlices = 32;        // d-ranges (partial logit tiles per token tile), at most

// Partial logit tile of token tile blockIdx.y over chunks [blockIdx.x * cpc,
// (blockIdx.x + 1) * cpc) of d, lane layout and chunk order as in route_tile;
// written as part[token row][expert column][slice] with ldp = 16 * NT columns
// and kSmallSlices slices per logit, so that one logit's slices are contiguous.
template <typename T, int NT>
__global__ __launch_bounds__(64) void router_part_kernel(
    const T* __restrict__ x, const T* __restrict__ wr, int T_, int d, int E, int cpc,
    float* __restrict__ part) {
  constexpr int kPerVec = 16 / sizeof(T);
  constexpr int kChunk = 16 * kPerVec;
  const int lane = threadIdx.x, r = lane & 15, c = lane >> 4;
  const int tile = blockIdx.y, slice = blockIdx.x;
  const int nch = d / kChunk;
  const int ch0 = slice * cpc, ch1 = min(nch, ch0 + cpc);
  const T* xrow = x + (size_t)min(tile * 16 + r, T_ - 1) * d + c * kPerVec;
  const T* wrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) wrow[nt] = wr + (size_t)min(nt * 16 + r, E - 1) * d + c * kPerVec;
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto load = [&](int ch, u32x4 (&a)[4], u32x4 (&b)[NT][4]) {
    const int kk = ch * kChunk;
#pragma unroll
    for (int q = 0; q < 4; ++q) a[q] = ld16(xrow + kk + q * 4 * kPerVec);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q) b[nt][q] = ld16(wrow[nt] + kk + q * 4 * kPerVec);
  };
  auto mma = [&](const u32x4 (&a)[4], const u32x4 (&b)[NT][4]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[nt] = mfma_bf16(a[q], b[nt][q], acc[nt]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[nt] = mfma_f32(__uint_as_float(a[q][i]), __uint_as_float(b[nt][q][i]), acc[nt]);
      }
    }
  };
  // Two chunks per step, both loaded before either is multiplied; chunks are
  // accumulated in increasing order.
  int ch = ch0;
  for (; ch + 1 < ch1; ch += 2) {
    u32x4 a0[4], b0[NT][4], a1[4], b1[NT][4];
    load(ch, a0, b0);
    load(ch + 1, a1, b1);
    mma(a0, b0);
    mma(a1, b1);
  }
  if (ch < ch1) {
    u32x4 a0[4], b0[NT][4];
    load(ch, a0, b0);
    mma(a0, b0);
  }
  const int ldp = 16 * NT;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      part[((size_t)(tile * 16 + 4 * c + i) * ldp + nt * 16 + r) * kSmallSlices + slice] = acc[nt][i];
}

// One block of kAuxThreads threads: the partial tiles summed in slice order,
// route_finish for every token, then f, P, aux and z-loss from the block's own
// LDS (no partial buffers), and (perm) the dispatch layout from the selections
// in LDS.  Every aux output may be null.  MAXPER and KMAX as in route_finish;
// the layout takes 8 waves of one batch (64 tokens x 8 slots at most).
constexpr int kSmallPermWaves = kSmallTokens * 8 / 64;
template <int MAXPER, int KMAX>
__global__ __launch_bounds__(kAuxThreads) void router_small_finish_kernel(
    const float* __restrict__ part, int slices, int ldp, const float* __restrict__ br,
    const float* __restrict__ bsel, int T_, int E, int k, int renorm,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int32_t* __restrict__ top1_count,
    float* __restrict__ prob_mean, float* __restrict__ aux, float* __restrict__ z_loss,
    int32_t* __restrict__ rounds_zero, bool perm, int capacity, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ dest, int32_t* __restrict__ src) {
  constexpr int kMT = kSmallTokens / kRouterTile;
  __shared__ RouterTileLds<1, kMT> sm;
  __shared__ PermLayoutLds<kSmallPermWaves, 1, false> psm;
  const int rows = ((T_ + 15) / 16) * 16;          // rows of the partial tiles
  // Logit (t, e) = sum over slices in order; token rows past T_ get 0.  The
  // slices of one logit are contiguous: 8 loads of 16 B, all issued before any
  // add (a load under a branch would make the compiler wait at the merge;
  // entries past `slices` are read but not added).
  for (int idx = threadIdx.x; idx < kSmallTokens * E; idx += kAuxThreads) {
    const int t = idx / E, e = idx - t * E;
    float g = 0.f;
    if (t < rows) {
      const f32x4* p = reinterpret_cast<const f32x4*>(part + ((size_t)t * ldp + e) * kSmallSlices);
      f32x4 v[kSmallSlices / 4];
#pragma unroll
      for (int i = 0; i < kSmallSlices / 4; ++i) v[i] = p[i];
      g = v[0][0];
#pragma unroll
      for (int s = 1; s < kSmallSlices; ++s)
        if (s < slices) g += v[s / 4][s % 4];
    }
    sm.red[0][t][e] = g;
  }
  route_finish<1, kMT, MAXPER, KMAX, true>(br, bsel, T_, E, k, renorm, 0, false, topk_idx, topk_w,
                                           sm);
  if (threadIdx.x < 64) {
    // f, P and the z-loss from the finishing waves' sums, added in wave order;
    // sum f_e P_e over lanes by a fixed xor tree.
    const int e = threadIdx.x;
    double ps = 0.0, z = 0.0;
    int cnt = 0;
#pragma unroll
    for (int w = 0; w < kMT; ++w) {
      if (e < E) {
        ps += sm.wps[w][e];
        cnt += sm.wcnt[w][e];
      }
      z += sm.wz[w];
    }
    const double P = ps / (double)T_, f = (double)cnt / (double)T_;
    double fP = e < E ? f * P : 0.0;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) fP += __shfl_xor(fP, off);
    if (e < E) {
      if (top1_count) top1_count[e] = cnt;
      if (prob_mean) prob_mean[e] = (float)P;
    }
    if (e == 0 && aux) *aux = (float)((double)E * fP);
    if (e == 1 && z_loss) *z_loss = (float)(z / (double)T_);
    if (e == 2 && rounds_zero) *rounds_zero = 0;
  }
  if (perm) {
    int ex[1];
    const int a = threadIdx.x;
    ex[0] = a < T_ * k ? sm.sel[a / k][a % k] : -1;
    perm_layout<kSmallPermWaves, 1, false>(ex, T_, k, E, capacity, true, counts, offsets, dest,
                                           src, psm);
  }
}

// Whether a router launch takes the small-batch path above.
static bool router_small(int T, bool rr) { return T <= kSmallTokens && !rr; }

// Slices of d and chunks per slice for the small-batch path.
static void small_split(int d, bool bf16, int& slices, int& cpc) {
  const int nch = d / (bf16 ? 128 : 64);
  cpc = (nch + kSmallSlices - 1) / kSmallSlices;
  slices = (nch + cpc - 1) / cpc;
}

size_t router_small_part_bytes(int T, int E, bool rr) {
  if (!router_small(T, rr)) return 0;
  return (size_t)kSmallSlices * ((T + 15) / 16) * 16 * ((E + 15) / 16) * 16 * sizeof(float);
}

bool router_can_permute(int assignments) { return assignments <= kPermWide; }

// Two token tiles per block when the expert rows are many (E > 16) and the
// tokens fill the chip with one block per CU: each W_r fragment loaded then
// serves 32 tokens, halving the re-reads of W_r.
static int router_tiles(int T, int E) { return (E > 16 && T >= 256 * 2 * kRouterTile) ? 2 : 1; }

int router_launch_blocks(int T, int E) {
  const int mt = router_tiles(T, E);
  return (T + kRouterTile * mt - 1) / (kRouterTile * mt);
}

template <typename T>
static hipError_t launch_router_t(const RouterArgs& a, hipStream_t s) {
  const int nt = (a.E + 15) / 16;
  const int mt = router_tiles(a.T, a.E);
  const int nblk = router_launch_blocks(a.T, a.E);
  const T* x = static_cast<const T*>(a.x);
  const T* wr = static_cast<const T*>(a.w_router);
  if (a.perm && !router_can_permute(a.T * a.k)) return hipErrorInvalidValue;
  if (router_small(a.T, a.rr_rank != nullptr)) {
    if (!a.part_logit) return hipErrorInvalidValue;
    int slices, cpc;
    small_split(a.d, sizeof(T) == 2, slices, cpc);
    const dim3 grid(slices, (a.T + 15) / 16);
    switch (nt) {
      case 1: router_part_kernel<T, 1><<<grid, 64, 0, s>>>(x, wr, a.T, a.d, a.E, cpc, a.part_logit); break;
      case 2: router_part_kernel<T, 2><<<grid, 64, 0, s>>>(x, wr, a.T, a.d, a.E, cpc, a.part_logit); break;
      case 3: router_part_kernel<T, 3><<<grid, 64, 0, s>>>(x, wr, a.T, a.d, a.E, cpc, a.part_logit); break;
      case 4: router_part_kernel<T, 4><<<grid, 64, 0, s>>>(x, wr, a.T, a.d, a.E, cpc, a.part_logit); break;
      default: return hipErrorInvalidValue;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
#define MOE_SMALL_FINISH(MAXPER, KMAX)                                                        \
  router_small_finish_kernel<MAXPER, KMAX><<<1, kAuxThreads, 0, s>>>(                          \
      a.part_logit, slices, 16 * nt, a.b_router, a.b_select, a.T, a.E, a.k, a.renorm, a.topk_idx, \
      a.topk_w, a.top1_count, a.prob_mean, a.aux, a.z_loss, a.rounds_zero, a.perm, a.capacity,    \
      a.counts, a.offsets, a.dest, a.src)
    const int per = a.E <= 8 ? 2 : a.E <= 16 ? 4 : 16;
    if (a.k <= 2) {
      if (per == 2) MOE_SMALL_FINISH(2, 2);
      else if (per == 4) MOE_SMALL_FINISH(4, 2);
      else MOE_SMALL_FINISH(16, 2);
    } else {
      if (per == 2) MOE_SMALL_FINISH(2, 8);
      else if (per == 4) MOE_SMALL_FINISH(4, 8);
      else MOE_SMALL_FINISH(16, 8);
    }
#undef MOE_SMALL_FINISH
    return hipGetLastError();
  }
  // Experts per lane: 2 up to 8 experts, else 4 per 16-expert tile; slots: 2 or 8.
  const bool k2 = a.k <= 2;
#define MOE_ROUTER_LAUNCH(NT, MT, PER, KM)                                                    \
  router_kernel<T, NT, MT, kRouterWaves, PER, KM><<<nblk, kRouterWaves * 64, 0, s>>>(         \
      x, wr, a.b_router, a.b_select, a.T, a.d, a.E, a.k, a.renorm, a.topk_idx, a.topk_w,     \
      a.part_psum, a.part_top1, a.part_z, a.rr_rank)
#define MOE_ROUTER_CASE(NT, MT)                                                               \
  case NT * 4 + MT:                                                                         \
    if (k2) MOE_ROUTER_LAUNCH(NT, MT, 4 * NT, 2);                                             \
    else MOE_ROUTER_LAUNCH(NT, MT, 4 * NT, 8);                                                \
    break;
  if (nt == 1 && mt == 1 && a.E <= 8) {
    if (k2) MOE_ROUTER_LAUNCH(1, 1, 2, 2);
    else MOE_ROUTER_LAUNCH(1, 1, 2, 8);
  } else {
    switch (nt * 4 + mt) {
      MOE_ROUTER_CASE(1, 1)
      MOE_ROUTER_CASE(2, 1)
      MOE_ROUTER_CASE(3, 1)
      MOE_ROUTER_CASE(4, 1)
      MOE_ROUTER_CASE(2, 2)
      MOE_ROUTER_CASE(3, 2)
      MOE_ROUTER_CASE(4, 2)
      default: return hipErrorInvalidValue;
    }
  }
#undef MOE_ROUTER_CASE
#undef MOE_ROUTER_LAUNCH
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (a.rr_rank) return hipSuccess;                   // reduced by the reroute launch
  aux_finalize_kernel<<<1, kAuxThreads, 0, s>>>(a.part_psum, a.part_top1, a.part_z, nblk, a.T, a.E,
                                                a.top1_count, a.prob_mean, a.aux, a.z_loss,
                                                a.rounds_zero, a.topk_idx, a.k, a.perm, a.capacity,
                                                a.counts, a.offsets, a.dest, a.src);
  return hipGetLastError();
}

// Upper bound of the blocks a router launch uses (sizes the partial-sum buffers).
int router_blocks(int T) { return (T + kRouterTile - 1) / kRouterTile; }

hipError_t launch_router(const RouterArgs& a, hipStream_t s) {
  return a.bf16 ? launch_router_t<uint16_t>(a, s) : launch_router_t<float>(a, s);
}

}  // namespace moe
