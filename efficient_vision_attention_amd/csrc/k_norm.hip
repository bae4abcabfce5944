// LayerNorm over channels for the block wrapper (FT 3.5 block equation).
// Biased variance, eps 1e-5 (the usual definition; the pages do not state
// it).  One wavefront per token row; two passes over registers (mean, then
// centred variance).
#include "common.h"
#include "kernels.h"

namespace hsmla {
namespace {

constexpr int kMaxPerLane = 32;  // channels <= 2048 = 64 lanes x 32

// 16-byte vectors: 8 bf16 or 4 float channels.
template <typename T>
struct Vec;
template <>
struct Vec<bf16> {
  static constexpr int N = 8;
  __device__ static void load(const bf16* p, float* v) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static void store(bf16* p, const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    *reinterpret_cast<uint4*>(p) = uint4{w[0], w[1], w[2], w[3]};
  }
};
template <>
struct Vec<float> {
  static constexpr int N = 4;
  __device__ static void load(const float* p, float* v) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
  }
  __device__ static void store(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// One wavefront per row; lane l handles 16-byte vectors l, l + 64, ...
template <typename T>
__global__ __launch_bounds__(256) void layernorm_kernel(
    const T* __restrict__ x, const float* __restrict__ g,
    const float* __restrict__ be, T* __restrict__ y, int rows, int ch) {
  constexpr int V = Vec<T>::N;
  constexpr int NI = kMaxPerLane / V;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int row = blockIdx.x * 4 + wave;
  if (row >= rows) return;
  const int nvec = ch / V;
  const T* xr = x + (size_t)row * ch;
  float v[NI][V];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int vi = lane + 64 * i;
    if (vi < nvec) {
      Vec<T>::load(xr + vi * V, v[i]);
    } else {
#pragma unroll
      for (int j = 0; j < V; ++j) v[i][j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < V; ++j) s += v[i][j];
  }
  const float mean = wave_sum(s) / (float)ch;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (lane + 64 * i < nvec) {
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const float dlt = v[i][j] - mean;
        q = fmaf(dlt, dlt, q);
      }
    }
  }
  const float rstd = rsqrtf(wave_sum(q) / (float)ch + 1e-5f);
  T* yr = y + (size_t)row * ch;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int vi = lane + 64 * i;
    if (vi >= nvec) continue;
    float o[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int c = vi * V + j;
      o[j] = (v[i][j] - mean) * rstd * g[c] + be[c];
    }
    Vec<T>::store(yr + vi * V, o);
  }
}

}  // namespace

hipError_t launch_layernorm(bool bf, const void* x, const float* gamma,
                            const float* beta, void* y, int rows, int ch,
                            hipStream_t s) {
  const unsigned blocks = (unsigned)((rows + 3) / 4);
  if (bf)
    layernorm_kernel<bf16><<<blocks, 256, 0, s>>>(static_cast<const bf16*>(x),
                                                  gamma, beta,
                                                  static_cast<bf16*>(y), rows, ch);
  else
    layernorm_kernel<float><<<blocks, 256, 0, s>>>(static_cast<const float*>(x),
                                                   gamma, beta,
                                                   static_cast<float*>(y), rows, ch);
  return hipGetLastError();
}

}  // namespace hsmla
