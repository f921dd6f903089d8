// MXFP4 (OCP microscaling) encoding of 32-element blocks, shared by the key
// quantizer and the FP4 indexer's query path.
//
// A block of 32 values x gets one power-of-two scale 2^e, stored as the
// E8M0 byte e + 127, with e = floor(log2(max |x|)) - 2 (so the block maximum
// lands in [4, 8), the top binade of E2M1) and e = -127 for an all-zero
// block.  Each x / 2^e is rounded to the nearest E2M1 magnitude
// {0, 0.5, 1, 1.5, 2, 3, 4, 6}, a tie going to the even code, and saturates
// at 6; bit 3 of the 4-bit code is the sign, and zero is always code 0.
// Element 2i sits in the low nibble of byte i.
#pragma once
#include "common.hpp"

namespace dlc {

// E2M1 code of y = x / 2^e (y exact): the thresholds are the midpoints of the
// grid, strict where the upper neighbour has the odd code, inclusive where it
// has the even one
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const float a = fabsf(y);
  const uint32_t c = uint32_t(a > 0.25f) + uint32_t(a >= 0.75f) + uint32_t(a > 1.25f) + uint32_t(a >= 1.75f) +
                     uint32_t(a > 2.5f) + uint32_t(a >= 3.5f) + uint32_t(a > 5.f);
  return (c != 0u && y < 0.f) ? (c | 8u) : c;
}

// shared exponent e of a block with maximum magnitude amax (finite)
__device__ __forceinline__ int mxfp4_shared_exp(float amax) {
  if (!(amax > 0.f)) return -127;
  int ex;
  (void)frexpf(amax, &ex);  // amax = f * 2^ex, 0.5 <= f < 1
  const int e = ex - 3;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// encode 32 values (v[0..31]) into 16 code bytes and the E8M0 scale byte
__device__ __forceinline__ uint4 mxfp4_encode32(const float (&v)[32], uint32_t& e8m0) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = mxfp4_shared_exp(amax);
  e8m0 = uint32_t(e + 127);
  const float inv = ldexpf(1.f, -e);  // exact power of two (e >= -127, so at most 2^127)
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc |= e2m1_code(v[8 * q + i] * inv) << (4 * i);
    w[q] = acc;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<bf16_raw>(bf16_raw x) { return __uint_as_float(uint32_t(x) << 16); }

// 32 consecutive elements at p (16-byte aligned) as floats
template <typename T>
__device__ __forceinline__ void load32(const T* p, float (&v)[32]) {
  constexpr int PER = 16 / sizeof(T);
#pragma unroll
  for (int c = 0; c < 32 / PER; ++c) {
    const uint4 u = *reinterpret_cast<const uint4*>(p + c * PER);
    const T* e = reinterpret_cast<const T*>(&u);
#pragma unroll
    for (int i = 0; i < PER; ++i) v[c * PER + i] = to_f32<T>(e[i]);
  }
}

}  // namespace dlc
