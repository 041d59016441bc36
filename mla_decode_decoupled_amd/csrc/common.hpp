// Shared device helpers for the libmla kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

#define MLA_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

template <typename T> __device__ __forceinline__ T from_f64(double x);
template <> __device__ __forceinline__ float from_f64<float>(double x) { return (float)x; }
// double -> float -> bf16 could round twice; go through the float with the right sticky bit.
template <> __device__ __forceinline__ bf16 from_f64<bf16>(double x) {
  float f = (float)x;
  // If the float conversion was inexact and f sits exactly on a bf16 tie, nudge it toward x
  // so the second rounding sees the true side of the tie.
  uint32_t u = __float_as_uint(f);
  if ((u & 0xFFFFu) == 0x8000u && (double)f != x) {
    u += ((double)f < x) == (f > 0.0f) ? 1u : (uint32_t)-1;
    f = __uint_as_float(u);
  }
  return (bf16)f;
}

// theta_j = base^(-2j/d) and the rotation angle p * theta_j, both in float64 so that the
// angle keeps full precision at positions up to 2^31 (float32 would lose ~0.016 rad at 131072).
__device__ __forceinline__ void rope_sincos(double base, int j, int d_rope, int64_t pos, double* s, double* c) {
  const double theta = pow(base, -2.0 * (double)j / (double)d_rope);
  sincos((double)pos * theta, s, c);
}

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace mla
