// Device-side building blocks shared by the gfx950 kernels: bf16 packing,
// the 16x16x32 bf16 matrix-core step, wavefront reductions and fast exp2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kascade {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16;

constexpr int kWave = 64;

// Finite stand-in for -infinity in running maxima: exp2(x - kNegBig) stays
// well defined when every key seen so far is masked.
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ float bf16_bits_to_float(u16 b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ u16 float_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(u16, h);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// One v_mfma_f32_16x16x32_bf16: C[16x16] += A[16x32] * B[32x16].
// Lane l supplies row (l % 16) of A and column (l % 16) of B, each as 8
// contraction elements of lane group l / 16; the same (group, slot) pairs
// index the contraction in A and in B. Lane l receives C rows
// 4*(l/16) .. 4*(l/16)+3 of column l % 16.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One v_mfma_f32_32x32x16_bf16: C[32x32] += A[32x16] * B[16x32].
// Lane l supplies row (l % 32) of A and column (l % 32) of B, each as the 8
// contraction elements 8*(l/32) .. 8*(l/32)+7. Lane l receives column l % 32,
// element i holding row 8*(i/4) + 4*(l/32) + (i%4).
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero_f32x16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8 load_bf16x8(const u16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = static_cast<__bf16>(0.0f);
  return z;
}

__device__ __forceinline__ bf16x8 pack_bf16x8(f32x4 lo, f32x4 hi) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = static_cast<__bf16>(lo[i]);
    r[i + 4] = static_cast<__bf16>(hi[i]);
  }
  return r;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// The values of lanes l and l^16 (v_permlane16_swap) and of lanes l and l^32
// (v_permlane32_swap): register-to-register lane exchanges on gfx950.
__device__ __forceinline__ void pair16(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  a = __int_as_float(r[0]);
  b = __int_as_float(r[1]);
}

__device__ __forceinline__ void pair32(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  a = __int_as_float(r[0]);
  b = __int_as_float(r[1]);
}

// Reductions across the four lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float group4_max(float v) {
  float a, b;
  pair16(v, a, b);
  pair32(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float group4_sum(float v) {
  float a, b;
  pair16(v, a, b);
  pair32(a + b, a, b);
  return a + b;
}

// Wave index as a scalar, so that wave-level conditions become scalar branches.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

}  // namespace kascade
