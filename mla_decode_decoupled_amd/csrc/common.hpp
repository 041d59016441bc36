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

// RoPE frequency theta_j = base^(-2j/d), in float64.
__device__ __forceinline__ double rope_theta(double base, int j, int d_rope) {
  return pow(base, -2.0 * (double)j / (double)d_rope);
}

// sin and cos of pos * theta entirely in float64 (float32 storage, where the rotated values must
// come out correctly rounded).
__device__ __forceinline__ void rope_sincos_f64(double theta, int64_t pos, double* s, double* c) {
  sincos((double)pos * theta, s, c);
}

// sin and cos of the angle pos * theta. The angle is formed and reduced to [-pi, pi] in float64,
// so positions up to 2^31 keep full precision (a float32 angle would be off by up to 0.008 rad
// at position 131072); the reduced angle is then evaluated in float32, whose error (~1e-7) is far
// below the bf16 / fp32 rounding of the rotated values.
__device__ __forceinline__ void rope_sincos(double theta, int64_t pos, float* s, float* c) {
  constexpr double kTwoPiHi = 6.283185307179586;        // 2 pi rounded to float64
  constexpr double kTwoPiLo = 2.4492935982947064e-16;   // 2 pi - kTwoPiHi
  const double a = (double)pos * theta;
  const double k = rint(a * 0.15915494309189535);        // a / (2 pi)
  const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, a));
  sincosf((float)r, s, c);
}

// Cache row of one new token at position p ("Decoupled RoPE · MLA Part 2", §3.4 and §4.3): the
// latent copied, the position key rotated in float64 and rounded once, so a stored row is exactly
// the rounding of the true rotated value. Threads tid, tid + nthr, ... share the row; with vec
// (16-byte aligned rows whose latent part is whole 16-byte pieces) the latent moves 16 bytes per
// thread. Every kernel that appends goes through here, so they all store the same bits.
template <typename T>
__device__ __forceinline__ void append_token(const T* __restrict__ c_src, const T* __restrict__ k_src,
                                             T* __restrict__ dst, int64_t p, int d_latent, int d_rope, double base,
                                             bool vec, int tid, int nthr) {
  if (vec) {
    const int n16 = d_latent * (int)sizeof(T) / 16;
    for (int c = tid; c < n16; c += nthr) reinterpret_cast<i32x4*>(dst)[c] = reinterpret_cast<const i32x4*>(c_src)[c];
  } else {
    for (int c = tid; c < d_latent; c += nthr) dst[c] = c_src[c];
  }
  for (int j = tid; j < d_rope / 2; j += nthr) {
    double s, co;
    rope_sincos_f64(rope_theta(base, j, d_rope), p, &s, &co);
    const double x0 = to_f32(k_src[2 * j]), x1 = to_f32(k_src[2 * j + 1]);
    dst[d_latent + 2 * j] = from_f64<T>(x0 * co - x1 * s);
    dst[d_latent + 2 * j + 1] = from_f64<T>(x0 * s + x1 * co);
  }
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
