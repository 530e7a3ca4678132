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

// Lanes e >= 0 (an expert id < 64; -1 = none) of a wave: the rank of this
// lane among the lanes with the same id (lower lanes first), and in `cnt` the
// size of that group.  The lanes whose id equals this lane's are the AND over
// the six bits of the id of the bit's ballot, complemented where this lane's
// bit is 0.  lt_mask = the lanes below this one.
__device__ __forceinline__ int wave_rank(int e, uint64_t lt_mask, int& cnt) {
  const uint64_t valid = __ballot(e >= 0);
  uint32_t lo = (uint32_t)valid, hi = (uint32_t)(valid >> 32);
#pragma unroll
  for (int b = 0; b < 6; ++b) {
    const uint64_t bb = __ballot((e >> b) & 1);
    const uint32_t flip = ((uint32_t)(e >> b) & 1u) - 1u;   // 0 where the bit is set, else ~0
    lo &= (uint32_t)bb ^ flip;
    hi &= (uint32_t)(bb >> 32) ^ flip;
  }
  const uint64_t same = ((uint64_t)hi << 32) | lo;
  cnt = __popcll(same);
  return __popcll(same & lt_mask);
}

// Lanes e >= 0 (an expert id < 64; -1 = none) of a wave: how many lanes hold
// id x, returned in lane x (the same bit-ballot match, against x's bits).
__device__ __forceinline__ int wave_count_of_lane(int e, int lane) {
  const uint64_t valid = __ballot(e >= 0);
  uint32_t lo = (uint32_t)valid, hi = (uint32_t)(valid >> 32);
#pragma unroll
  for (int b = 0; b < 6; ++b) {
    const uint64_t bb = __ballot((e >> b) & 1);
    const uint32_t flip = ((uint32_t)(lane >> b) & 1u) - 1u;
    lo &= (uint32_t)bb ^ flip;
    hi &= (uint32_t)(bb >> 32) ^ flip;
  }
  return __popcll(((uint64_t)hi << 32) | lo);
}

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
// (after Hastings): for a >= 0, erfc(a) ~= t P(t) exp(-a^2) with t = 1/(1 + p a)
// and P a fourth-degree polynomial; |error| <= 1.5e-7.  With a = |z| / sqrt 2
// and r = erfc(a) / 2:  GELU(z) = z - z r for z >= 0 and z r for z < 0
// (1 + erf(-a) = erfc(a)), i.e. max(z, 0) - |z| r in both cases (one fused
// multiply-add, no select), so there is no cancellation and GELU's absolute
// error stays below ~1e-7 |z|.  The 1/sqrt 2 is folded into p, the 1/2 into
// P's coefficients, and exp(-a^2) = exp2(-z^2 log2(e) / 2).
__device__ __forceinline__ float gelu_erf(float z) {
  constexpr float kP = 0.3275911f * 0.70710678118654752440f;
  constexpr float c1 = 0.5f * 0.254829592f, c2 = 0.5f * -0.284496736f, c3 = 0.5f * 1.421413741f,
                  c4 = 0.5f * -1.453152027f, c5 = 0.5f * 1.061405429f;
  const float t = __builtin_amdgcn_rcpf(fmaf(kP, fabsf(z), 1.0f));
  float q = fmaf(c5, t, c4);
  q = fmaf(q, t, c3);
  q = fmaf(q, t, c2);
  q = fmaf(q, t, c1);
  q *= t;
  const float e = __builtin_amdgcn_exp2f(z * z * -0.72134752044448170368f);
  return fmaf(-fabsf(z), q * e, fmaxf(z, 0.f));
}

// Two fp32 values rounded to bf16 (nearest, ties to even) and packed, lo in
// bits 0..15: one v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

}  // namespace moe
