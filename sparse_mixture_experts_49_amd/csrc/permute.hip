// Dispatch of the MoE layer on gfx950: per-expert histogram, prefix scan,
// capacity, stable ranks in token order and the row scatter into
// expert-contiguous buffers.
//
// The lecture-hall page's listing ("Mixture of Experts: Scaling Parameters
// Without Scaling Compute", section "The MoE layer") collects the rows routed
// to each expert with a mask per expert.  Here the same grouping is a stable
// counting sort of the assignment ids a = t*k + s by expert, done without
// host synchronisation and without data-dependent atomics on global memory:
//   1. hist:    each block counts the experts of its chunk of assignments;
//   2. scan:    one block turns the block counts into per-(block, expert)
//               bases, applies the capacity (top-1 only: keep the first C
//               assignments of each expert in token order -- section "The
//               central problem: load balancing", expert capacity) and writes
//               counts and offsets;
//   3. rank:    each block ranks its chunk's assignments in order with wave
//               ballots, and writes dest[a] (or -1) and src[row] = a;
//   4. scatter: one wave per token reads x[t] once and writes it to every
//               kept destination row.
// With at most 1024 assignments (decode) one kernel does all four steps:
// every block builds the whole layout in LDS (it is small), block 0 writes
// it out, and each block scatters its own tokens' rows.
// Expert ids outside [0, E) are treated as dropped assignments.
#include "device_common.h"
#include "kernels.h"
#include "perm_small.h"

namespace moe {

int permute_blocks(int assignments) { return (assignments + kPermChunk - 1) / kPermChunk; }

__global__ __launch_bounds__(256) void perm_hist_kernel(const int32_t* __restrict__ topk_idx,
                                                        int A, int E,
                                                        int32_t* __restrict__ blk_hist) {
  __shared__ int h[64];
  if (threadIdx.x < 64) h[threadIdx.x] = 0;
  __syncthreads();
  const int base = blockIdx.x * kPermChunk;
  for (int i = threadIdx.x; i < kPermChunk; i += 256) {
    const int a = base + i;
    if (a < A) {
      const int e = topk_idx[a];
      if (e >= 0 && e < E) atomicAdd(&h[e], 1);   // integer counts: order-independent
    }
  }
  __syncthreads();
  if (threadIdx.x < E) blk_hist[(size_t)blockIdx.x * E + threadIdx.x] = h[threadIdx.x];
}

// The block counts are first copied to LDS by all threads (coalesced, loads in
// flight together) when they fit; expert e's thread then walks its column in
// block order.
constexpr int kScanThreads = 1024;
constexpr int kScanLds = 16384;     // block-count entries staged in LDS (64 KiB)

__global__ __launch_bounds__(kScanThreads) void perm_scan_kernel(const int32_t* __restrict__ blk_hist,
                                                                 int nblk, int E, int capacity,
                                                                 int32_t* __restrict__ blk_base,
                                                                 int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ offsets) {
  __shared__ int hs[kScanLds];
  __shared__ int kept[64];
  const int tid = threadIdx.x;
  const int n = nblk * E;
  const bool staged = n <= kScanLds;
  if (staged)
    for (int i = tid; i < n; i += kScanThreads) hs[i] = blk_hist[i];
  __syncthreads();
  if (tid < 64) {
    const int e = tid;
    int run = 0;
    if (e < E) {
      for (int b = 0; b < nblk; ++b) {
        blk_base[(size_t)b * E + e] = run;
        run += staged ? hs[b * E + e] : blk_hist[(size_t)b * E + e];
      }
    }
    kept[e] = (e < E) ? ((capacity > 0) ? min(run, capacity) : run) : 0;
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int i = 0; i < E; ++i) {
      offsets[i] = acc;
      counts[i] = kept[i];
      acc += kept[i];
    }
    offsets[E] = acc;
  }
}

// Wave w of block b ranks assignments [b*1024 + w*256, +256) in four batches
// of 64 lanes.  In a batch, the lanes that share an expert are matched with one
// ballot per bit of the expert id (wave_rank); a lane's rank is the number of
// earlier lanes of its group plus the wave's running count for that expert,
// which the group's first lane then advances (LDS, this wave's row only, so the
// wave's own program order keeps reads and updates in sequence).
__global__ __launch_bounds__(256) void perm_rank_kernel(const int32_t* __restrict__ topk_idx,
                                                        int A, int E, int capacity,
                                                        const int32_t* __restrict__ blk_base,
                                                        const int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ dest,
                                                        int32_t* __restrict__ src) {
  __shared__ int wcount[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int base = blockIdx.x * kPermChunk + wave * 256;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  wcount[wave][lane] = 0;
  int ex[4], rk[4];
#pragma unroll
  for (int bt = 0; bt < 4; ++bt) {
    const int a = base + bt * 64 + lane;
    int e = (a < A) ? topk_idx[a] : -1;
    if (e < 0 || e >= E) e = -1;
    int grp;
    const int within = wave_rank(e, lt_mask, grp);
    const int before = e >= 0 ? wcount[wave][e] : 0;
    ex[bt] = e;
    rk[bt] = before + within;
    if (e >= 0 && within == 0) wcount[wave][e] = before + grp;
  }
  __syncthreads();
#pragma unroll
  for (int bt = 0; bt < 4; ++bt) {
    const int a = base + bt * 64 + lane;
    if (a >= A) continue;
    const int e = ex[bt];
    if (e < 0) {
      dest[a] = -1;
      continue;
    }
    int r = blk_base[(size_t)blockIdx.x * E + e] + rk[bt];
    for (int w = 0; w < wave; ++w) r += wcount[w][e];
    if (capacity > 0 && r >= capacity) {
      dest[a] = -1;
    } else {
      const int row = offsets[e] + r;
      dest[a] = row;
      src[row] = a;
    }
  }
}

// One wave per token: load the row once (16 B per lane per step) and store it
// to each kept destination.
__global__ __launch_bounds__(256) void perm_scatter_kernel(const uint8_t* __restrict__ x,
                                                           const int32_t* __restrict__ dest,
                                                           int T, int k, int row_bytes,
                                                           uint8_t* __restrict__ x_perm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  int dst[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) dst[s] = (s < k) ? dest[(size_t)t * k + s] : -1;
  const uint8_t* xr = x + (size_t)t * row_bytes;
  const int nvec = row_bytes >> 4;
#pragma unroll 4
  for (int v = lane; v < nvec; v += 64) {
    const u32x4 val = ld16(xr + (size_t)v * 16);
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (dst[s] >= 0) st16(x_perm + (size_t)dst[s] * row_bytes + (size_t)v * 16, val);
  }
}

// All four steps for A <= kPermChunk assignments: every block builds the
// layout in LDS (perm_layout), block 0 writes it out, and block b scatters
// tokens 4b .. 4b+3, one wave each.
__global__ __launch_bounds__(256) void perm_small_kernel(
    const int32_t* __restrict__ topk_idx, int T, int k, int E, int capacity,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ dest,
    int32_t* __restrict__ src, const uint8_t* __restrict__ x, int row_bytes,
    uint8_t* __restrict__ x_perm) {
  __shared__ PermLayoutLds<4, kPermChunk / 256, true> sm;
  int ex[kPermChunk / 256];
  perm_load<4, kPermChunk / 256>(topk_idx, T * k, ex);
  perm_layout<4, kPermChunk / 256, true>(ex, T, k, E, capacity, blockIdx.x == 0, counts, offsets,
                                         dest, src, sm);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T || !x_perm) return;
  int dst[8];
#pragma unroll
  for (int sl = 0; sl < 8; ++sl) dst[sl] = (sl < k) ? sm.s_dest[t * k + sl] : -1;
  const uint8_t* xr = x + (size_t)t * row_bytes;
  const int nvec = row_bytes >> 4;
#pragma unroll 4
  for (int v = lane; v < nvec; v += 64) {
    const u32x4 val = ld16(xr + (size_t)v * 16);
#pragma unroll
    for (int sl = 0; sl < 8; ++sl)
      if (dst[sl] >= 0) st16(x_perm + (size_t)dst[sl] * row_bytes + (size_t)v * 16, val);
  }
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  const int A = a.T * a.k;
  const int row_bytes = a.d * (a.bf16 ? 2 : 4);
  if (A <= kPermChunk) {
    // Without x_perm only block 0's layout is needed.
    perm_small_kernel<<<a.x_perm ? (a.T + 3) / 4 : 1, 256, 0, s>>>(
        a.topk_idx, a.T, a.k, a.E, a.capacity, a.counts, a.offsets, a.dest, a.src,
        static_cast<const uint8_t*>(a.x), row_bytes, static_cast<uint8_t*>(a.x_perm));
    return hipGetLastError();
  }
  const int nblk = permute_blocks(A);
  perm_hist_kernel<<<nblk, 256, 0, s>>>(a.topk_idx, A, a.E, a.blk_hist);
  perm_scan_kernel<<<1, kScanThreads, 0, s>>>(a.blk_hist, nblk, a.E, a.capacity, a.blk_base, a.counts,
                                    a.offsets);
  perm_rank_kernel<<<nblk, 256, 0, s>>>(a.topk_idx, A, a.E, a.capacity, a.blk_base, a.offsets,
                                        a.dest, a.src);
  if (a.x_perm) {
    perm_scatter_kernel<<<(a.T + 3) / 4, 256, 0, s>>>(static_cast<const uint8_t*>(a.x), a.dest,
                                                      a.T, a.k, row_bytes,
                                                      static_cast<uint8_t*>(a.x_perm));
  }
  return hipGetLastError();
}

}  // namespace moe
