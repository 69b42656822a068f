// Device helpers shared by the gfx950 kernels of the NVFP4 W4A4 expert path.
//
// Formats (OCP MX v1.0 FP4 E2M1; OCP OFP8 E4M3 with maximum 448): NVFP4 keeps
// 16-element blocks of E2M1 codes, an E4M3 scale per block and an FP32 scale
// per tensor ("The 4-bitter Lesson", section "Baseline: A starting recipe with
// stable training dynamics").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nv4 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// dev_status bits (mirror include/nv4moe.h)
constexpr int kDsNonFinite = 1;
constexpr int kDsBadExpert = 2;
constexpr int kDsNanLogit = 4;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// FP32 -> BF16 bits, round to nearest even (finite inputs; NaN is kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// E4M3 (OCP, max 448) from a non-negative FP32: saturate at 448, otherwise round
// to nearest with ties to the even code.  Below 2^-6 the grid is uniform with
// step 2^-9 (subnormals), so scaling by 2^9 and rounding to an integer is exact
// RNE; above it the FP32 mantissa is rounded to 3 bits.  NaN saturates as well.
__device__ __forceinline__ uint32_t e4m3_from_f32(float t) {
  if (!(t < 448.0f)) return 0x7Eu;
  if (t < 0.015625f) return (uint32_t)__builtin_rintf(t * 512.0f);
  uint32_t b = __float_as_uint(t);
  b += 0x7FFFFu + ((b >> 20) & 1u);
  return (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
}

// Value of a non-negative finite E4M3 code (exact in FP32).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t e = c >> 3, m = c & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// Tensor encode scale S from the group amax A: S = fp32(2688 / A), 1 when A == 0
// or the quotient is not finite (2688 = largest E2M1 magnitude 6 x largest E4M3 448).
__device__ __forceinline__ float tensor_encode_scale(float A) {
  if (!(A > 0.0f)) return 1.0f;
  float s = __fdiv_rn(2688.0f, A);
  return (s <= 3.402823466e38f) ? s : 1.0f;
}

// Two FP32 values -> two E2M1 codes (round to nearest even, saturating at 6, sign
// kept) written into byte `SEL` of `old`.  gfx950's converter does exactly this
// when its scale is 1.0 (its scale operand only contributes its exponent).
template <int SEL>
__device__ __forceinline__ uint32_t pack_e2m1_pair(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// Exact decode of 8 E2M1 codes (one dword, element 2i in the low nibble of byte
// i) times one block scale `s2` (the E4M3 value in both FP16 halves) to FP16.
// e2m1 * e4m3 has at most 6 significant bits and lies in [2^-10, 2688], so every
// product is exact in FP16; the packed multiply therefore never rounds.
__device__ __forceinline__ f16x8 decode8_f16(uint32_t w, f16x2 s2) {
  f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Two E4M3 scale bytes (the low 16 bits of `w`, or the high 16 bits with HI) -> two
// FP16 values (exact).
template <bool HI = false>
__device__ __forceinline__ f16x2 e4m3x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

// ---------------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// atomic max of a non-negative float through its bit pattern (order independent)
__device__ __forceinline__ void atomic_max_nonneg(float *p, float v) {
  atomicMax(reinterpret_cast<unsigned int *>(p), __float_as_uint(v));
}

}  // namespace nv4
