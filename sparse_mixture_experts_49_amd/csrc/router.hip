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
  float lse[kRouterTile * MT];
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
template <typename T, int NT, int WAVES, int MT>
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

  // The bias words of the lane's experts (quarter q of a quad holds experts q, q+4,
  // ...), all issued before the barrier so that their latency overlaps it rather
  // than adding one round trip per expert to the epilogue.
  constexpr int kMaxPer = 16;
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
    if (q == 0) sm.lse[tr] = m + logf(s);

    // top-k: k rounds of a quad-wide argmax over the unselected logits.
    uint32_t taken = 0;
    int sel_e[8];
    float sel_p[8];
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
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
    for (int sl = 0; sl < 8; ++sl)
      if (sl < k) wsum += sel_p[sl];
    const float winv = renorm ? 1.0f / wsum : 1.0f;
    if (t < T_ && q == 0) {
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) {
        if (sl < k) {
          topk_idx[(size_t)t * k + sl] = sel_e[sl];
          topk_w[(size_t)t * k + sl] = renorm ? sel_p[sl] * winv : sel_p[sl];
        }
      }
    }
    if (rr) {                                        // inputs of the expert ranking
#pragma unroll
      for (int j = 0; j < kMaxPer; ++j) {
        const int e = q + 4 * j;                     // rows of 64, key 0 past E
        sm.rkey[tr][e] = e < E ? rank_key(sc[j], e) : 0ull;
        sm.rwt[tr][e] = renorm ? p[j] * winv : p[j];
      }
    }
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      const int e = q + 4 * j;
      if (e < E) sm.prob[tr][e] = (t < T_) ? p[j] : 0.f;
    }
    if (q == 0) sm.top1[tr] = (t < T_) ? sel_e[0] : -1;
  }
  __syncthreads();
}

// One block = 16*MT tokens x all experts, W waves splitting d.  The block then
// writes its partial sums of the aux loss and z-loss for aux_finalize_kernel
// and, for the reroute policy, every token's experts in ranking order.
template <typename T, int NT, int MT, int W>
__global__ __launch_bounds__(W * 64) void router_kernel(
    const T* __restrict__ x, const T* __restrict__ wr, const float* __restrict__ br,
    const float* __restrict__ bsel, int T_, int d, int E, int k, int renorm,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    double* __restrict__ part_psum, int32_t* __restrict__ part_top1, double* __restrict__ part_z,
    int32_t* __restrict__ rr_rank) {
  __shared__ RouterTileLds<W, MT> sm;
  constexpr int kTok = kRouterTile * MT;
  const int t0 = blockIdx.x * kTok;
  route_tile<T, NT, W, MT>(x, wr, br, bsel, T_, d, E, k, renorm, t0, rr_rank != nullptr, topk_idx,
                           topk_w, sm);
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
#define MOE_ROUTER_CASE(NT, MT)                                                               \
  case NT * 4 + MT:                                                                         \
    router_kernel<T, NT, MT, kRouterWaves><<<nblk, kRouterWaves * 64, 0, s>>>(                \
        x, wr, a.b_router, a.b_select, a.T, a.d, a.E, a.k, a.renorm, a.topk_idx, a.topk_w,   \
        a.part_psum, a.part_top1, a.part_z, a.rr_rank);                                       \
    break;
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
#undef MOE_ROUTER_CASE
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (a.rr_rank) return hipSuccess;                   // reduced by the reroute launch
  if (a.perm && !router_can_permute(a.T * a.k)) return hipErrorInvalidValue;
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
