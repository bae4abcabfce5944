// Shared device helpers for the HSMLA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hsmla {

// bfloat16 storage type: the upper 16 bits of an IEEE float32.
struct bf16 {
  uint16_t u;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) {
  return __uint_as_float(static_cast<uint32_t>(x.u) << 16);
}

template <typename T>
__device__ __forceinline__ T from_f32(float x);

template <>
__device__ __forceinline__ float from_f32<float>(float x) {
  return x;
}

// Round float32 to bfloat16, nearest even.  Adding 0x7fff plus the lowest
// kept bit to the pattern carries into the kept bits exactly when the
// dropped half is above one half ulp, or equal to it with an odd kept part.
// NaN is kept quiet.
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return bf16{static_cast<uint16_t>((u >> 16) | 0x40u)};
  u += 0x7fffu + ((u >> 16) & 1u);
  return bf16{static_cast<uint16_t>(u >> 16)};
}

__device__ __forceinline__ float relu(float x) { return x > 0.f ? x : 0.f; }

// Sum over a 64-lane wavefront (result valid in every lane).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace hsmla
