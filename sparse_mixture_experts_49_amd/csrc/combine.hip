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
#include "device_common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o,
                                                      const int32_t* __restrict__ dest,
                                                      const float* __restrict__ topk_w,
                                                      const float* __restrict__ shared, int T,
                                                      int d, int k, float* __restrict__ y) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  int dst[8];
  float w[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    dst[s] = (s < k) ? dest[(size_t)t * k + s] : -1;
    w[s] = (s < k) ? topk_w[(size_t)t * k + s] : 0.f;
  }
  const int nvec = d >> 2;
  float* yr = y + (size_t)t * d;
#pragma unroll 2
  for (int v = lane; v < nvec; v += 64) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (dst[s] >= 0) {
        const f32x4 ov = *reinterpret_cast<const f32x4*>(o + (size_t)dst[s] * d + (size_t)v * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(w[s], ov[i], acc[i]);
      }
    }
    if (shared) acc += *reinterpret_cast<const f32x4*>(shared + (size_t)t * d + (size_t)v * 4);
    *reinterpret_cast<f32x4*>(yr + (size_t)v * 4) = acc;
  }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  combine_kernel<<<(a.T + 3) / 4, 256, 0, s>>>(a.o, a.dest, a.topk_w, a.shared, a.T, a.d, a.k, a.y);
  return hipGetLastError();
}

}  // namespace moe
