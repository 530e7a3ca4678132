// The dispatch layout of a layer small enough for one block (web page
// "Mixture of Experts: Scaling Parameters Without Scaling Compute", section
// "The MoE layer": rows grouped by expert, in token order; section "The central
// problem: load balancing": expert capacity).  Used by the single-launch
// permute (up to kPermChunk assignments) and by the aux-loss reduction block,
// which runs it for the whole layer (up to kPermWide assignments) so that
// moe_forward needs no permute launch.
#pragma once

#include "device_common.h"

namespace moe {

constexpr int kPermChunk = 1024;   // assignments per block of the multi-block permute
constexpr int kPermWide = 8192;    // assignments the aux block lays out (16 waves x 8 batches x 64)

template <int WAVES, int BATCHES, bool KEEP>
struct PermLayoutLds {
  int pre[WAVES][64];     // wave w's count of expert e, then the count in waves before w
  int s_off[65];
  int s_dest[KEEP ? WAVES * BATCHES * 64 : 1];
};

// The expert of each assignment the thread lays out (-1 past the end), loaded
// before any is used; a caller may issue these loads early, ahead of other work,
// and pass them to perm_layout.
template <int WAVES, int BATCHES>
__device__ __forceinline__ void perm_load(const int32_t* __restrict__ topk_idx, int A,
                                          int (&ex)[BATCHES]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int bt = 0; bt < BATCHES; ++bt) {
    const int a = (wave * BATCHES + bt) * 64 + lane;
    ex[bt] = (threadIdx.x < WAVES * 64 && a < A) ? topk_idx[a] : -1;
  }
}

// Called by every thread of the block (it holds barriers), with ex from
// perm_load; the first WAVES waves do the work.  Wave w ranks assignments
// w*BATCHES*64 .. in BATCHES batches of 64 (lane e of the wave keeps its running
// count of expert e).
// Wave 0 then takes one expert per lane: the waves' counts give the number of
// each expert's requests in the waves before each wave, its total, the
// capacity clamp (capacity > 0) and, by a wave-wide scan, the offsets.  Every
// assignment then gets its row (-1 if dropped or if its expert is outside
// [0, E)), kept in sm.s_dest with KEEP.  With `write`, counts, offsets, dest and
// src are written to global memory too.
template <int WAVES, int BATCHES, bool KEEP>
__device__ __forceinline__ void perm_layout(int (&ex)[BATCHES], int T, int k,
                                            int E, int capacity, bool write,
                                            int32_t* __restrict__ counts,
                                            int32_t* __restrict__ offsets,
                                            int32_t* __restrict__ dest, int32_t* __restrict__ src,
                                            PermLayoutLds<WAVES, BATCHES, KEEP>& sm) {
  const bool worker = threadIdx.x < WAVES * 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int A = T * k;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int rk[BATCHES], run = 0;
  if (worker) {
#pragma unroll
    for (int bt = 0; bt < BATCHES; ++bt) {
      int e = ex[bt];
      if (e < 0 || e >= E) e = -1;
      ex[bt] = e;
      rk[bt] = 0;
      if (__ballot(e >= 0) == 0) continue;       // a batch with nothing to lay out (wave-uniform)
      int cnt;
      const int r = wave_rank(e, lt_mask, cnt);
      rk[bt] = __shfl(run, e >= 0 ? e : 0) + r;   // this wave's earlier batches + rank in this one
      run += wave_count_of_lane(e, lane);         // lane x: requests for expert x in this batch
    }
    sm.pre[wave][lane] = run;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int e = threadIdx.x;
    int tot = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const int c = sm.pre[w][e];
      sm.pre[w][e] = tot;
      tot += c;
    }
    const int kept = e < E ? (capacity > 0 ? min(tot, capacity) : tot) : 0;
    int incl = kept;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (e < E) {
      sm.s_off[e] = incl - kept;
      if (write) {
        offsets[e] = incl - kept;
        counts[e] = kept;
      }
    }
    if (e == E - 1) {
      sm.s_off[E] = incl;
      if (write) offsets[E] = incl;
    }
  }
  __syncthreads();
  if (worker) {
#pragma unroll
    for (int bt = 0; bt < BATCHES; ++bt) {
      const int a = (wave * BATCHES + bt) * 64 + lane;
      if (a >= A) continue;
      const int e = ex[bt];
      int row = -1;
      if (e >= 0) {
        const int r = rk[bt] + sm.pre[wave][e];
        if (capacity <= 0 || r < capacity) row = sm.s_off[e] + r;
      }
      if constexpr (KEEP) sm.s_dest[a] = row;
      if (write) {
        dest[a] = row;
        if (row >= 0) src[row] = a;
      }
    }
  }
  __syncthreads();
}

}  // namespace moe
