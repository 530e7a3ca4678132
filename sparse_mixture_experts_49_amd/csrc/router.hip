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
#include "perm_small.h"

namespace moe {

constexpr int kRouterTokens = 16;   // tokens per block (one MFMA row tile)
constexpr int kAuxThreads = 1024;   // threads of the single aux-reduction block
constexpr int kRouterWaves = 8;     // the block's waves split d between them

// LDS of one token tile: the waves' partial logits, then each token's
// probabilities, first choice and log-sum-exp for the aux and z-loss sums.
template <int WAVES>
struct RouterTileLds {
  float red[WAVES][kRouterTokens][65];
  float prob[kRouterTokens][64];
  int top1[kRouterTokens];
  float lse[kRouterTokens];
};

// Tokens t0 .. t0+15 of the router: logits on MFMA (the WAVES waves split d),
// softmax, top-k and the routing weights; fills sm.prob / top1 / lse.  Ends
// with a barrier.  Wave w accumulates the k-chunks w, w+WAVES, ... of the
// d-long dot products; the partial logit tiles are summed in wave order
// through LDS, so the result does not depend on scheduling.
//
// Lane layout of the loads: lane l reads row (l % 16) -- a token of x, or an
// expert row of W_r -- and 64 contiguous bytes starting at k-chunk offset
// (l / 16) * 64 B, so each row's 256 B per chunk come from 4 lanes.  MFMA j of
// the chunk consumes the lane's j-th 16-byte piece; A and B use the same map.
template <typename T, int NT, int WAVES>
__device__ __forceinline__ void route_tile(
    const T* __restrict__ x, const T* __restrict__ wr, const float* __restrict__ br,
    const float* __restrict__ bsel, int T_, int d, int E, int k, int renorm, int t0,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, float* __restrict__ rr_score,
    float* __restrict__ rr_wt, RouterTileLds<WAVES>& sm) {
  constexpr int kPerLane = 64 / sizeof(T);          // elements per lane per chunk
  constexpr int kChunk = 4 * kPerLane;              // 128 bf16 or 64 fp32
  constexpr int kPerVec = 16 / sizeof(T);
  auto& red = sm.red;
  auto& prob = sm.prob;
  auto& top1 = sm.top1;
  auto& lse = sm.lse;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, c = lane >> 4;
  const T* xrow = x + (size_t)min(t0 + r, T_ - 1) * d + c * kPerLane;
  const T* wrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) wrow[nt] = wr + (size_t)min(nt * 16 + r, E - 1) * d + c * kPerLane;

  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nch = d / kChunk;
  auto load_chunk = [&](int ch, u32x4 (&a)[4], u32x4 (&b)[NT][4]) {
    const int kk = ch * kChunk;
#pragma unroll
    for (int q = 0; q < 4; ++q) a[q] = ld16(xrow + kk + q * kPerVec);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q) b[nt][q] = ld16(wrow[nt] + kk + q * kPerVec);
  };
  auto mma_chunk = [&](const u32x4 (&a)[4], const u32x4 (&b)[NT][4]) {
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
  // Two chunks per iteration, both loaded before either is multiplied: with
  // few tokens (decode) the loop is bound by load latency.  The chunks are
  // accumulated in order ch = wave, wave + WAVES, ... either way.
  int ch = wave;
  for (; ch + WAVES < nch; ch += 2 * WAVES) {
    u32x4 a0[4], b0[NT][4], a1[4], b1[NT][4];
    load_chunk(ch, a0, b0);
    load_chunk(ch + WAVES, a1, b1);
    mma_chunk(a0, b0);
    mma_chunk(a1, b1);
  }
  if (ch < nch) {
    u32x4 a0[4], b0[NT][4];
    load_chunk(ch, a0, b0);
    mma_chunk(a0, b0);
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * c + i][nt * 16 + r] = acc[nt][i];
  __syncthreads();

  if (wave == 0) {
    // Four lanes per token: lane quarter q holds experts q, q+4, q+8, ...
    const int tq = lane >> 2, q = lane & 3;
    const int t = t0 + tq;
    constexpr int kMaxPer = 16;
    float g[kMaxPer], p[kMaxPer], sc[kMaxPer];
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      const int e = q + 4 * j;
      g[j] = -INFINITY;
      if (e < E) {
        g[j] = red[0][tq][e];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) g[j] += red[w][tq][e];   // in wave order
        if (br) g[j] += br[e];
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
      sc[j] = (bsel && e < E) ? g[j] + bsel[e] : g[j];   // ranking scores
    }
    if (q == 0) lse[tq] = m + logf(s);

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
    if (rr_score && t < T_) {                       // inputs of the reroute policy
#pragma unroll
      for (int j = 0; j < kMaxPer; ++j) {
        const int e = q + 4 * j;                     // rows of 64 scores, -inf past E
        rr_score[(size_t)t * 64 + e] = e < E ? sc[j] : -INFINITY;
        if (e < E) rr_wt[(size_t)t * E + e] = renorm ? p[j] * winv : p[j];
      }
    }
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      const int e = q + 4 * j;
      if (e < E) prob[tq][e] = (t < T_) ? p[j] : 0.f;
    }
    if (q == 0) top1[tq] = (t < T_) ? sel_e[0] : -1;
  }
  __syncthreads();
}

// One block = 16 tokens x all experts, 8 waves splitting d.  The block then
// writes its partial sums of the aux loss and z-loss for aux_finalize_kernel.
template <typename T, int NT>
__global__ __launch_bounds__(kRouterWaves * 64) void router_kernel(
    const T* __restrict__ x, const T* __restrict__ wr, const float* __restrict__ br,
    const float* __restrict__ bsel, int T_, int d, int E, int k, int renorm,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    double* __restrict__ part_psum, int32_t* __restrict__ part_top1, double* __restrict__ part_z,
    float* __restrict__ rr_score, float* __restrict__ rr_wt) {
  __shared__ RouterTileLds<kRouterWaves> sm;
  const int t0 = blockIdx.x * kRouterTokens;
  route_tile<T, NT, kRouterWaves>(x, wr, br, bsel, T_, d, E, k, renorm, t0, topk_idx, topk_w,
                                  rr_score, rr_wt, sm);
  auto& prob = sm.prob;
  auto& top1 = sm.top1;
  auto& lse = sm.lse;
  // Per-block partials of the aux loss, summed in token order.
  if (threadIdx.x < E) {
    const int e = threadIdx.x;
    double ps = 0.0;
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < kRouterTokens; ++i) {
      ps += (double)prob[i][e];
      cnt += (top1[i] == e);
    }
    part_psum[(size_t)blockIdx.x * E + e] = ps;
    part_top1[(size_t)blockIdx.x * E + e] = cnt;
  }
  if (threadIdx.x == 64) {                           // z-loss partial, token order
    double z = 0.0;
    for (int i = 0; i < kRouterTokens && t0 + i < T_; ++i) z += (double)lse[i] * (double)lse[i];
    part_z[blockIdx.x] = z;
  }
}

// Fixed-order reduction of the router partials: f, P and aux (web page
// "Mixture of Experts: Scaling Parameters Without Scaling Compute", section
// "The central problem: load balancing").
__global__ __launch_bounds__(kAuxThreads) void aux_finalize_kernel(
    const double* __restrict__ part_psum, const int32_t* __restrict__ part_top1,
    const double* __restrict__ part_z, int nblk, int T_, int E, int32_t* __restrict__ top1_count,
    float* __restrict__ prob_mean, float* __restrict__ aux, float* __restrict__ z_loss,
    int32_t* __restrict__ rounds_zero, const int32_t* __restrict__ topk_idx, int k, bool perm,
    int capacity, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ dest, int32_t* __restrict__ src) {
  // The partials are [nblk][E] laid out flat.  Thread t < stride (a multiple of
  // E) sums entries t, t + stride, ... (all of expert t % E, coalesced across
  // the block); expert e's per-thread sums are then added in thread order.
  // The grouping depends only on (nblk, E), so the result is deterministic.
  __shared__ double ps[kAuxThreads];
  __shared__ long long pc[kAuxThreads];
  __shared__ double fP[64];
  __shared__ double wz[kAuxThreads / 64];
  __shared__ PermSmallLds psm;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int stride = (kAuxThreads / E) * E;
  const long n = (long)nblk * E;
  double sum = 0.0;
  long long cnt = 0;
  if (t < stride) {
    // Unrolled so that several loads are in flight; the sum still runs in i order.
#pragma unroll 8
    for (long i = t; i < n; i += stride) {
      sum += part_psum[i];
      cnt += part_top1[i];
    }
  }
  ps[t] = sum;
  pc[t] = cnt;
  double zs = 0.0;                                   // z-loss: block partials t, t + threads, ...
#pragma unroll 4
  for (int b = t; b < nblk; b += kAuxThreads) zs += part_z[b];
  // Fixed shuffle tree per wave, then the waves in order.
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) zs += __shfl_down(zs, off);
  if (lane == 0) wz[wave] = zs;
  __syncthreads();
  if (t < E) {
    double S = 0.0;
    long long C = 0;
    for (int u = t; u < stride; u += E) {
      S += ps[u];
      C += pc[u];
    }
    const double P = S / (double)T_, f = (double)C / (double)T_;
    fP[t] = f * P;
    if (top1_count) top1_count[t] = (int32_t)C;
    if (prob_mean) prob_mean[t] = (float)P;
  }
  __syncthreads();
  if (t == 0 && aux) {
    double acc = 0.0;
    for (int i = 0; i < E; ++i) acc += fP[i];
    *aux = (float)((double)E * acc);
  }
  if (t == 128 && rounds_zero) *rounds_zero = 0;
  if (t == 64 && z_loss) {
    double zt = 0.0;
    for (int w = 0; w < kAuxThreads / 64; ++w) zt += wz[w];
    *z_loss = (float)(zt / (double)T_);
  }
  // Small layers: the dispatch layout too, saving the permute's own launch.
  if (perm) perm_small_layout(topk_idx, T_, k, E, capacity, true, counts, offsets, dest, src, psm);
}

bool router_can_permute(int assignments) { return assignments <= kPermChunk; }

template <typename T>
static hipError_t launch_router_t(const RouterArgs& a, hipStream_t s) {
  const int nblk = (a.T + kRouterTokens - 1) / kRouterTokens;
  const int nt = (a.E + 15) / 16;
  const T* x = static_cast<const T*>(a.x);
  const T* wr = static_cast<const T*>(a.w_router);
#define MOE_ROUTER_CASE(NT)                                                                   \
  case NT:                                                                                  \
    router_kernel<T, NT><<<nblk, kRouterWaves * 64, 0, s>>>(                                  \
        x, wr, a.b_router, a.b_select, a.T, a.d, a.E, a.k, a.renorm, a.topk_idx, a.topk_w,   \
        a.part_psum, a.part_top1, a.part_z, a.rr_score, a.rr_wt);                             \
    break;
  switch (nt) {
    MOE_ROUTER_CASE(1)
    MOE_ROUTER_CASE(2)
    MOE_ROUTER_CASE(3)
    MOE_ROUTER_CASE(4)
    default: return hipErrorInvalidValue;
  }
#undef MOE_ROUTER_CASE
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (a.perm && !router_can_permute(a.T * a.k)) return hipErrorInvalidValue;
  aux_finalize_kernel<<<1, kAuxThreads, 0, s>>>(a.part_psum, a.part_top1, a.part_z, nblk, a.T, a.E,
                                                a.top1_count, a.prob_mean, a.aux, a.z_loss,
                                                a.rounds_zero, a.topk_idx, a.k, a.perm, a.capacity,
                                                a.counts, a.offsets, a.dest, a.src);
  return hipGetLastError();
}

int router_blocks(int T) { return (T + kRouterTokens - 1) / kRouterTokens; }

hipError_t launch_router(const RouterArgs& a, hipStream_t s) {
  return a.bf16 ? launch_router_t<uint16_t>(a, s) : launch_router_t<float>(a, s);
}

}  // namespace moe
