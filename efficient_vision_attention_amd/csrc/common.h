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

typedef __bf16 hw_bf16x2 __attribute__((ext_vector_type(2)));
typedef float hw_f32x2 __attribute__((ext_vector_type(2)));

// Round float32 to bfloat16, nearest even, with gfx950's conversion
// instruction (v_cvt_pk_bf16_f32, default round mode; NaN stays NaN).
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) {
  return bf16{__builtin_bit_cast(uint16_t, static_cast<__bf16>(x))};
}

// Two floats -> two bfloat16 in one 32-bit word (a in the low half).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const hw_f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, hw_bf16x2));
}

__device__ __forceinline__ float relu(float x) { return x > 0.f ? x : 0.f; }

// Buffer-resource loads and stores (raw, stride 0): an offset past the
// resource's byte count reads zeros and drops stores in hardware, so edge
// lanes need no branch and every memory instruction is unconditional (the
// compiler's wait counts then stay exact).
constexpr int kOob = INT32_MIN;  // an offset no resource here reaches

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base,
                                                          int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           bytes, 0x00020000);
}

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// 16 bytes, streamed (non-temporal: the readers of whole staged rows use
// each byte once; measured faster for the K/V state and no slower for the
// readout and the FFN conv).
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  const i32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
  return uint4{(uint32_t)t.x, (uint32_t)t.y, (uint32_t)t.z, (uint32_t)t.w};
}

// GELU(x) = x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)) with erf from
// Abramowitz & Stegun 7.1.28:
//   erf(z) = 1 - (1 + a1 z + a2 z^2 + ... + a6 z^6)^-16,  z >= 0,
//   |error| <= 3e-7,
// extended to z < 0 by oddness.  Written as
//   GELU(x) = max(x, 0) - |x| erfc(|x| / sqrt 2) / 2
//           = max(x, 0) - |x| / P(|x|)^16,
// with P's coefficients c_i = a_i 2^(-i/2) 2^(1/16) (c_0 = 2^(1/16)), so
// that P(|x|)^16 = 2 (1 + a1 z + ... + a6 z^6)^16: six FMAs in |x|, four
// squarings, one reciprocal, a max and an FMA.  No cancellation for x < 0
// (the result is the small term itself); measured against float64 erf on
// [-8, 8]: absolute error <= 7e-7, far below the bfloat16 output
// precision.  (Infinite x gives NaN; the inputs are sums of finite
// products.)
__device__ __forceinline__ float gelu_erf(float x) {
  constexpr float c0 = 1.0442737824e+00f, c1 = 5.2075163037e-02f,
                  c2 = 2.2076998457e-02f, c3 = 3.4227392389e-03f,
                  c4 = 3.9686137011e-05f, c5 = 5.1055209009e-05f,
                  c6 = 5.6212996640e-06f;
  const float ax = fabsf(x);
  float p = fmaf(fmaf(fmaf(fmaf(fmaf(fmaf(c6, ax, c5), ax, c4), ax, c3), ax, c2), ax, c1),
                 ax, c0);
  p *= p;
  p *= p;
  p *= p;
  p *= p;
  // max(x, 0) on the bit pattern: a float with the sign bit set is a
  // negative int32, so one integer max (fmaxf would first quieten x with an
  // extra max)
  const float pos = __int_as_float(max(__float_as_int(x), 0));
  return fmaf(-ax, __builtin_amdgcn_rcpf(p), pos);
}

// Sum over a 64-lane wavefront (result valid in every lane).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace hsmla
