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

// Sum over a 64-lane wavefront (result valid in every lane).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace hsmla
