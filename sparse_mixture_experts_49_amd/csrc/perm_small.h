// The dispatch layout of at most kPermChunk assignments, computed by one
// block (web page "Mixture of Experts: Scaling Parameters Without Scaling
// Compute", section "The MoE layer": rows grouped by expert, in token order;
// section "The central problem: load balancing": expert capacity).  Shared by
// the single-launch permute and by the aux-loss reduction, which runs it for
// the whole layer when the layer is small.
#pragma once

#include "device_common.h"

namespace moe {

constexpr int kPermChunk = 1024;   // assignments per block (4 waves x 4 batches x 64)

struct PermSmallLds {
  int wcount[4][64];
  int s_off[65];
  int s_dest[kPermChunk];
};

// Called by every thread of the block (it holds barriers); threads 0..255 do
// the work.  Wave w ranks assignments w*256 .. +255 in four batches of 64
// (lane e of the wave keeps its running count of expert e); the per-wave
// counts give each expert's total, the capacity clamp (capacity > 0) and the
// offsets; then every assignment gets its row (-1 if dropped or if its expert
// is outside [0, E)), kept in sm.s_dest.  With `write`, counts, offsets, dest
// and src are written to global memory too.
__device__ __forceinline__ void perm_small_layout(const int32_t* __restrict__ topk_idx, int T,
                                                  int k, int E, int capacity, bool write,
                                                  int32_t* __restrict__ counts,
                                                  int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ dest,
                                                  int32_t* __restrict__ src, PermSmallLds& sm) {
  const bool worker = threadIdx.x < 256;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int A = T * k;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int ex[4], rk[4], run = 0;
  if (worker) {
#pragma unroll
    for (int bt = 0; bt < 4; ++bt) {
      const int a = wave * 256 + bt * 64 + lane;
      int e = (a < A) ? topk_idx[a] : -1;
      if (e < 0 || e >= E) e = -1;
      int cnt;
      const int r = wave_rank(e, lt_mask, cnt);
      ex[bt] = e;
      rk[bt] = __shfl(run, e >= 0 ? e : 0) + r;   // this wave's earlier batches + rank in this one
      run += wave_count_of_lane(e, lane);         // lane x: requests for expert x in this batch
    }
    sm.wcount[wave][lane] = run;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int e = 0; e < E; ++e) {
      const int tot = sm.wcount[0][e] + sm.wcount[1][e] + sm.wcount[2][e] + sm.wcount[3][e];
      const int kept = capacity > 0 ? min(tot, capacity) : tot;
      sm.s_off[e] = acc;
      if (write) {
        offsets[e] = acc;
        counts[e] = kept;
      }
      acc += kept;
    }
    sm.s_off[E] = acc;
    if (write) offsets[E] = acc;
  }
  __syncthreads();
  if (worker) {
#pragma unroll
    for (int bt = 0; bt < 4; ++bt) {
      const int a = wave * 256 + bt * 64 + lane;
      if (a >= A) continue;
      const int e = ex[bt];
      int row = -1;
      if (e >= 0) {
        int r = rk[bt];
        for (int w = 0; w < wave; ++w) r += sm.wcount[w][e];
        if (capacity <= 0 || r < capacity) row = sm.s_off[e] + r;
      }
      sm.s_dest[a] = row;
      if (write) {
        dest[a] = row;
        if (row >= 0) src[row] = a;
      }
    }
  }
  __syncthreads();
}

}  // namespace moe
