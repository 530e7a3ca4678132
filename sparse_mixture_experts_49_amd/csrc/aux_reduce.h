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
  double ps[THREADS];
  long long pc[THREADS];
  double fP[64];
  double wz[THREADS / 64];
};

// The partials are [nblk][E] laid out flat.  Thread t < stride (a multiple of
// E) sums entries t, t + stride, ... (all of expert t % E, coalesced across
// the block); expert e's per-thread sums are then added in thread order.  The
// grouping depends only on (nblk, E, THREADS), so the result is deterministic.
// Every output may be null.  Ends without a barrier.
template <int THREADS>
__device__ __forceinline__ void aux_reduce(const double* __restrict__ part_psum,
                                           const int32_t* __restrict__ part_top1,
                                           const double* __restrict__ part_z, int nblk, int T_,
                                           int E, int32_t* __restrict__ top1_count,
                                           float* __restrict__ prob_mean, float* __restrict__ aux,
                                           float* __restrict__ z_loss, AuxLds<THREADS>& sm) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int stride = (THREADS / E) * E;
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
  sm.ps[t] = sum;
  sm.pc[t] = cnt;
  double zs = 0.0;                                   // z-loss: block partials t, t + threads, ...
#pragma unroll 4
  for (int b = t; b < nblk; b += THREADS) zs += part_z[b];
  // Fixed shuffle tree per wave, then the waves in order.
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) zs += __shfl_down(zs, off);
  if (lane == 0) sm.wz[wave] = zs;
  __syncthreads();
  if (t < E) {
    double S = 0.0;
    long long C = 0;
    for (int u = t; u < stride; u += E) {
      S += sm.ps[u];
      C += sm.pc[u];
    }
    const double P = S / (double)T_, f = (double)C / (double)T_;
    sm.fP[t] = f * P;
    if (top1_count) top1_count[t] = (int32_t)C;
    if (prob_mean) prob_mean[t] = (float)P;
  }
  __syncthreads();
  if (t == 0 && aux) {
    double acc = 0.0;
    for (int i = 0; i < E; ++i) acc += sm.fP[i];
    *aux = (float)((double)E * acc);
  }
  if (t == 64 && z_loss) {
    double zt = 0.0;
    for (int w = 0; w < THREADS / 64; ++w) zt += sm.wz[w];
    *z_loss = (float)(zt / (double)T_);
  }
}

}  // namespace moe
