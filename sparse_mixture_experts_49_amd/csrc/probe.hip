// A plain streaming read of device memory: the practical HBM read ceiling that
// the layer's weight-bound kernels are compared with (the bench reports it beside
// the 8 TB/s grade).  Not part of the layer.
//
// Each wave reads its own contiguous 16 KiB, 1 KiB per load instruction with four
// loads in flight; the XOR of everything read is compared with a constant so that
// the loads cannot be removed.
#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kProbeWaveBytes = 16384;

__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ p,
                                                         uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const size_t base = ((size_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (kProbeWaveBytes / 16);
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < kProbeWaveBytes / 16; i += 256) {
    const u32x4 v0 = p[base + i + lane], v1 = p[base + i + 64 + lane];
    const u32x4 v2 = p[base + i + 128 + lane], v3 = p[base + i + 192 + lane];
    acc ^= v0 ^ v1 ^ v2 ^ v3;
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) sink[0] = acc.x;
}

size_t read_probe_granule() { return 4 * (size_t)kProbeWaveBytes; }

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s) {
  const size_t blocks = bytes / read_probe_granule();
  read_probe_kernel<<<(unsigned)blocks, 256, 0, s>>>(static_cast<const u32x4*>(buf), sink);
  return hipGetLastError();
}

}  // namespace moe
