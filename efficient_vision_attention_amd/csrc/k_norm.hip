// LayerNorm over channels for the block wrapper (FT 3.5 block equation).
// Biased variance, eps 1e-5 (the usual definition; the pages do not state
// it).  One wavefront per token row; two passes over registers (mean, then
// centred variance).
#include "common.h"
#include "kernels.h"

namespace hsmla {
namespace {

constexpr int kMaxPerLane = 32;  // channels <= 2048

template <typename T>
__global__ __launch_bounds__(256) void layernorm_kernel(
    const T* __restrict__ x, const float* __restrict__ g,
    const float* __restrict__ be, T* __restrict__ y, int rows, int ch) {
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int row = blockIdx.x * 4 + wave;
  if (row >= rows) return;
  const T* xr = x + (size_t)row * ch;
  float v[kMaxPerLane];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int c = lane + 64 * i;
    v[i] = c < ch ? to_f32(xr[c]) : 0.f;
    s += v[i];
  }
  const float mean = wave_sum(s) / (float)ch;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int c = lane + 64 * i;
    const float dlt = c < ch ? v[i] - mean : 0.f;
    q = fmaf(dlt, dlt, q);
  }
  const float rstd = rsqrtf(wave_sum(q) / (float)ch + 1e-5f);
  T* yr = y + (size_t)row * ch;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int c = lane + 64 * i;
    if (c < ch) yr[c] = from_f32<T>((v[i] - mean) * rstd * g[c] + be[c]);
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
