// Combine of the MoE layer on gfx950.
//
// Web page "Mixture of Experts: Scaling Parameters Without Scaling Compute",
// section "The MoE layer", step 3: the layer output is the weighted sum of the
// chosen experts' outputs.  Each token gathers its k expert-output rows and
// sums them in slot order (fp32 fma), so no two threads ever write the same
// output and no atomics are needed; the result is bitwise repeatable.  A token
// whose every slot was dropped by the capacity limit gets 0 (the residual
// connection outside the layer carries x).  A shared expert's output, when
// given, is added after the slot sum (same page, section "Design variations":
// shared experts are always active), also for tokens whose slots were dropped.
// When the second expert product left its k-split partial sums unreduced, each
// slot's row is summed here from them, in part order, exactly as the product's
// own reduction would have stored it.
#include "device_common.h"
#include "kernels.h"

namespace moe {

// Thread (blockIdx.y * 256 + threadIdx.x) of block row t sums four adjacent
// columns of token t: its k expert-output loads are independent, so they are
// all in flight at once, and a few tokens (decode) still spread over many waves.
template <bool PARTIAL>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o,
                                                      const int32_t* __restrict__ dest,
                                                      const float* __restrict__ topk_w,
                                                      const float* __restrict__ shared, int T,
                                                      int d, int k, float* __restrict__ y,
                                                      const float* __restrict__ partial, int splits,
                                                      int rows_cap) {
  const int t = blockIdx.x;
  const int v = blockIdx.y * 256 + threadIdx.x;   // float4 column group
  if (v >= (d >> 2)) return;
  int dst[8];
  float w[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    dst[s] = (s < k) ? dest[(size_t)t * k + s] : -1;
    w[s] = (s < k) ? topk_w[(size_t)t * k + s] : 0.f;
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (PARTIAL) {
    // Deferred split-k sums (few tokens): two slots at a time, the parts of both
    // (up to kMaxParts each) loaded before any is added, so they are in flight
    // together; each slot's sum runs in part order, then the slots are weighted
    // in slot order.
    constexpr int kMaxParts = 8;
#pragma unroll
    for (int s0 = 0; s0 < 8; s0 += 2) {
      if (s0 >= k) break;
      f32x4 part[2][kMaxParts];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int s = s0 + u;
        if (dst[s] >= 0) {
          const float* p = partial + (size_t)dst[s] * d + (size_t)v * 4;
#pragma unroll
          for (int sp = 0; sp < kMaxParts; ++sp)
            if (sp < splits)
              part[u][sp] = *reinterpret_cast<const f32x4*>(p + (size_t)sp * rows_cap * d);
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int s = s0 + u;
        if (dst[s] >= 0) {
          f32x4 ov = part[u][0];
#pragma unroll
          for (int sp = 1; sp < kMaxParts; ++sp)
            if (sp < splits) ov += part[u][sp];
          const float* p = partial + (size_t)dst[s] * d + (size_t)v * 4;
          for (int sp = kMaxParts; sp < splits; ++sp)
            ov += *reinterpret_cast<const f32x4*>(p + (size_t)sp * rows_cap * d);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = fmaf(w[s], ov[i], acc[i]);
        }
      }
    }
  } else {
    f32x4 ov[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (dst[s] >= 0) ov[s] = *reinterpret_cast<const f32x4*>(o + (size_t)dst[s] * d + (size_t)v * 4);
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (dst[s] >= 0)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(w[s], ov[s][i], acc[i]);
  }
  if (shared) acc += *reinterpret_cast<const f32x4*>(shared + (size_t)t * d + (size_t)v * 4);
  *reinterpret_cast<f32x4*>(y + (size_t)t * d + (size_t)v * 4) = acc;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  const dim3 grid(a.T, (a.d / 4 + 255) / 256);
  // Two instances: with deferred split-k parts (the loads of every part of two
  // slots in flight at once; few tokens) and without (few registers, many waves).
  if (a.partial)
    combine_kernel<true><<<grid, 256, 0, s>>>(a.o, a.dest, a.topk_w, a.shared, a.T, a.d, a.k, a.y,
                                              a.partial, a.splits, a.rows_cap);
  else
    combine_kernel<false><<<grid, 256, 0, s>>>(a.o, a.dest, a.topk_w, a.shared, a.T, a.d, a.k, a.y,
                                               a.partial, a.splits, a.rows_cap);
  return hipGetLastError();
}

}  // namespace moe
