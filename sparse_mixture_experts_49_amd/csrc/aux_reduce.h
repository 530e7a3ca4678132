// Fixed-order reduction of the router's per-block partials: f, P and the
// auxiliary loss, and the router z-loss (web page "Mixture of Experts: Scaling
// Parameters Without Scaling Compute", section "The central problem: load
// balancing": aux = E * sum_i f_i P_i, f_i the fraction of tokens whose first
// choice is i, P_i the mean router probability; z-loss = mean squared
// log-sum-exp of the logits).  One block of THREADS threads runs it.
#pragma once

#include "device_common.h"

namespace moe {

template <int THREADS>
struct AuxLds {
  double ps[THREADS / 64][64];   // per wave: expert e's sum over the wave's lanes of e
  int pc[THREADS / 64][64];
  double wz[THREADS / 64];
};

// The partials are [nblk][E] laid out flat.  With Ep the smallest power of two
// >= E, lane l of the block takes expert l % Ep and group g = thread / Ep of the
// THREADS / Ep groups; it sums rows g, g + groups, ... of its expert (adjacent
// lanes read adjacent experts of a row).  A fixed xor tree then adds the lanes
// of one expert inside each wave, and lane e of wave 0 adds the waves in order.
// The grouping depends only on (nblk, E, THREADS), so the result is
// deterministic, and no step is a long serial chain.  Every output may be null.
// Ends without a barrier.
template <int THREADS>
__device__ __forceinline__ void aux_reduce(const double* __restrict__ part_psum,
                                           const int32_t* __restrict__ part_top1,
                                           const double* __restrict__ part_z, int nblk, int T_,
                                           int E, int32_t* __restrict__ top1_count,
                                           float* __restrict__ prob_mean, float* __restrict__ aux,
                                           float* __restrict__ z_loss, AuxLds<THREADS>& sm) {
  constexpr int kWaves = THREADS / 64;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int lg = 0;
  while ((1 << lg) < E) ++lg;                        // Ep = 1 << lg <= 64
  const int e = lane & ((1 << lg) - 1);
  const int groups = THREADS >> lg;
  double sum = 0.0;
  int cnt = 0;
  if (e < E) {
    // Unrolled so that several loads are in flight; the sum still runs in row order.
#pragma unroll 8
    for (int b = t >> lg; b < nblk; b += groups) {
      sum += part_psum[(size_t)b * E + e];
      cnt += part_top1[(size_t)b * E + e];
    }
  }
  double zs = 0.0;                                   // z-loss: block partials t, t + threads, ...
#pragma unroll 4
  for (int b = t; b < nblk; b += THREADS) zs += part_z[b];
  for (int off = 32; off >= (1 << lg); off >>= 1) {
    sum += __shfl_xor(sum, off);
    cnt += __shfl_xor(cnt, off);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) zs += __shfl_xor(zs, off);
  if (lane < E && lane == e) {
    sm.ps[wave][lane] = sum;
    sm.pc[wave][lane] = cnt;
  }
  if (lane == 0) sm.wz[wave] = zs;
  __syncthreads();
  if (t < 64) {
    double S = 0.0, zt = 0.0;
    int C = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (t < E) {
        S += sm.ps[w][t];
        C += sm.pc[w][t];
      }
      zt += sm.wz[w];
    }
    const double P = S / (double)T_, f = (double)C / (double)T_;
    double fP = t < E ? f * P : 0.0;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) fP += __shfl_xor(fP, off);
    if (t < E) {
      if (top1_count) top1_count[t] = C;
      if (prob_mean) prob_mean[t] = (float)P;
    }
    if (t == 0 && aux) *aux = (float)((double)E * fP);
    if (t == 1 && z_loss) *z_loss = (float)(zt / (double)T_);
  }
}

}  // namespace moe
