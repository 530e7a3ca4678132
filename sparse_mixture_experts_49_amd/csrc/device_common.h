// Device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// 16-byte global / LDS vector accesses.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// bf16 <-> fp32.  Widening is exact; narrowing rounds to nearest, ties to even
// (inputs here are finite).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float to_f32(float v) { return v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }
};

// One 16x16 output tile, K = 32 (bf16) per instruction.  Operand lane layout:
// lane l holds row/column (l % 16) and the 8 consecutive k-slots 8*(l/16)..+7.
// Since the product sums over k, the kernels may map k-slots to any k as long
// as A and B use the same map.
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// fp32 variant, K = 4 per instruction: lane l holds row/column (l % 16), k-slot l/16.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// Output layout of both: lane l holds column (l % 16), rows 4*(l/16) + i, i = 0..3.

typedef float f32x16 __attribute__((ext_vector_type(16)));
// One 32x32 output tile, K = 16 (bf16) per instruction.  Operand lane layout:
// lane l holds row/column (l % 32) and k-slots 8*(l/32)..+7.  Output: lane l,
// register i holds row 8*(i/4) + 4*(l/32) + (i%4), column l % 32.  From a
// single wave per SIMD this shape keeps the matrix pipe ~85% busy, the
// 16x16x32 shape only ~53% (measured on MI355X), so the MFMA-bound kernel uses it.
__device__ __forceinline__ f32x16 mfma32_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// GELU(z) = z * Phi(z) = (z / 2) * (1 + erf(z / sqrt 2)), with erf from
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26
// (after Hastings): for a >= 0, erfc(a) ~= P(t) exp(-a^2) with t = 1/(1 + p a)
// and P a fifth-degree polynomial without constant term; |error| <= 1.5e-7.
// Using erfc directly for z < 0 (1 + erf(-a) = erfc(a)) avoids cancellation,
// so GELU's absolute error stays below ~1e-7 |z|.
__device__ __forceinline__ float gelu_erf(float z) {
  const float a = fabsf(z) * 0.70710678118654752440f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, a, 1.0f));
  float poly = fmaf(1.061405429f, t, -1.453152027f);
  poly = fmaf(poly, t, 1.421413741f);
  poly = fmaf(poly, t, -0.284496736f);
  poly = fmaf(poly, t, 0.254829592f);
  poly *= t;
  const float erfc_a = poly * __builtin_amdgcn_exp2f(-a * a * 1.44269504088896340736f);
  const float one_plus_erf = z < 0.f ? erfc_a : 2.0f - erfc_a;
  return 0.5f * z * one_plus_erf;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

}  // namespace moe
