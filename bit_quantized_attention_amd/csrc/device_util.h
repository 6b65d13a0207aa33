// Device helpers: 16-bit element unpacking, exact INT8 code rounding,
// error-free fp64 summation, wave-wide reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qattn {

// ---- 16-bit element access -------------------------------------------------

// Widen the 16-bit element in the low (hi=false) or high half of a dword.
template <bool BF16>
__device__ __forceinline__ float half_word_to_f32(uint32_t w, bool hi) {
  if constexpr (BF16) {
    return __uint_as_float(hi ? (w & 0xffff0000u) : (w << 16));
  } else {
    const uint16_t h = hi ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffffu);
    return (float)__builtin_bit_cast(_Float16, h);
  }
}

// Load 8 consecutive 16-bit elements (16 bytes, 16-byte aligned) as floats.
template <bool BF16>
__device__ __forceinline__ void load8_f32(const void* p, float (&x)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  x[0] = half_word_to_f32<BF16>(u.x, false);
  x[1] = half_word_to_f32<BF16>(u.x, true);
  x[2] = half_word_to_f32<BF16>(u.y, false);
  x[3] = half_word_to_f32<BF16>(u.y, true);
  x[4] = half_word_to_f32<BF16>(u.z, false);
  x[5] = half_word_to_f32<BF16>(u.z, true);
  x[6] = half_word_to_f32<BF16>(u.w, false);
  x[7] = half_word_to_f32<BF16>(u.w, true);
}

// ---- exact INT8 quantization -------------------------------------------------

// Block scale: fl32(amax / 127) with IEEE division, 1.0 when that is zero.
__device__ __forceinline__ float quant_scale(float amax) {
  float s = amax / 127.0f;
  return s == 0.0f ? 1.0f : s;
}

// clamp(round-half-even(x / scale), -127, 127) of the exact real quotient,
// without branches. `inv` is any close approximation of 1/scale, so the true
// quotient lies within half a unit of t = x * inv and its rounding is
// floor(t) or floor(t) + 1. The half-integer h = floor(t) + 1/2 between the two
// is compared with the quotient through the sign of one fused multiply-add,
// x - h * scale (exact, because the product inside an fma is not rounded):
// positive picks h + 1/2, negative h - 1/2, zero is a tie and rounding h itself
// to even picks the even neighbour.
__device__ __forceinline__ int quant_code(float x, float scale, float inv) {
  const float h = __builtin_floorf(x * inv) + 0.5f;
  const float e = __builtin_fmaf(-h, scale, x);
  const float g = e == 0.0f ? 0.0f : __builtin_copysignf(0.5f, e);
  float v = __builtin_fminf(__builtin_fmaxf(h + g, -127.0f), 127.0f);
  return (int)__builtin_rintf(v);
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
         ((uint32_t)(d & 0xff) << 24);
}

// ---- error-free fp64 summation ------------------------------------------------

// s + e == a + b exactly, s = fl64(a + b) (Knuth's TwoSum).
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  const double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

// (hi, lo) += x, keeping hi + lo equal to the exact running sum as long as the
// low parts stay within 53 bits (see the header of qattn_smooth_quant).
__device__ __forceinline__ void dd_add(double& hi, double& lo, double x) {
  double s, e;
  two_sum(hi, x, s, e);
  hi = s;
  lo += e;
}

__device__ __forceinline__ void dd_merge(double& hi, double& lo, double h2, double l2) {
  double s, e;
  two_sum(hi, h2, s, e);
  hi = s;
  lo += l2 + e;
}

// ---- wave reductions (wave64) ---------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace qattn
