// Global ReLU linear attention (FT 3.1 Z/D sums; FT 3.3 lin-local ratio with
// the neighbourhood taken as every token).
//
//   Z[b,h] = sum_n relu(K_hat[b,n,h,:])^T V_hat[b,n,h,:]      (d x d)
//   D[b,h] = sum_n relu(K_hat[b,n,h,:])                       (d)
//   O[b,n,h,:] = relu(Q_hat) Z / (relu(Q_hat) . D), 0 if the sum is 0
//
// The token reduction is split into a fixed number of chunks per (image,
// head); stage 2 adds the chunk partials in chunk order, so the result does
// not depend on scheduling (no float atomics).
#include "common.h"
#include "kernels.h"

namespace hsmla {
namespace {

constexpr int kD = 32;               // head_dim
constexpr int kPart = kD * kD + kD;  // floats per partial (Z then D)
constexpr int kTok = 64;             // tokens staged per LDS tile

// grid (chunks, heads, batch), 256 threads: thread owns Z[i][j0..j0+3],
// i = tid / 8, j0 = 4 * (tid % 8); threads with tid % 8 == 0 also own D[i].
template <typename T>
__global__ __launch_bounds__(256) void kv_partial_kernel(
    const T* __restrict__ qkvh, float* __restrict__ part, int tokens,
    int heads, int chunk_len) {
  __shared__ float fk[kTok][kD + 1];
  __shared__ float vv[kTok][kD + 1];
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int nchunks = gridDim.x;
  const int C = heads * kD;
  const int tid = threadIdx.x;
  const int i = tid / 8, j0 = (tid % 8) * 4;
  const int n_begin = chunk * chunk_len;
  const int n_end = min(tokens, n_begin + chunk_len);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float dacc = 0.f;
  const T* base = qkvh + (size_t)b * tokens * 3 * C;
  for (int n0 = n_begin; n0 < n_end; n0 += kTok) {
    const int cnt = min(kTok, n_end - n0);
    for (int e = tid; e < kTok * kD; e += 256) {
      const int r = e / kD, c = e % kD;
      float kv = 0.f, vvv = 0.f;
      if (r < cnt) {
        const T* row = base + (size_t)(n0 + r) * 3 * C;
        kv = relu(to_f32(row[C + h * kD + c]));
        vvv = to_f32(row[2 * C + h * kD + c]);
      }
      fk[r][c] = kv;
      vv[r][c] = vvv;
    }
    __syncthreads();
    for (int r = 0; r < cnt; ++r) {
      const float a = fk[r][i];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = fmaf(a, vv[r][j0 + j], acc[j]);
      dacc += a;
    }
    __syncthreads();
  }
  float* out = part + ((size_t)(b * heads + h) * nchunks + chunk) * kPart;
#pragma unroll
  for (int j = 0; j < 4; ++j) out[i * kD + j0 + j] = acc[j];
  if (tid % 8 == 0) out[kD * kD + i] = dacc;
}

// grid (batch * heads), 256 threads: fixed-order sum of the chunk partials.
__global__ __launch_bounds__(256) void kv_combine_kernel(
    const float* __restrict__ part, float* __restrict__ kv,
    float* __restrict__ ksum, int nchunks) {
  const int bh = blockIdx.x;
  const float* p = part + (size_t)bh * nchunks * kPart;
  for (int e = threadIdx.x; e < kPart; e += blockDim.x) {
    float s = 0.f;
    for (int c = 0; c < nchunks; ++c) s += p[(size_t)c * kPart + e];
    if (e < kD * kD)
      kv[(size_t)bh * kD * kD + e] = s;
    else
      ksum[(size_t)bh * kD + (e - kD * kD)] = s;
  }
}

// grid (ceil(tokens/64), heads, batch), 64 threads: one token per thread.
template <typename T>
__global__ __launch_bounds__(64) void lin_apply_kernel(
    const T* __restrict__ qkvh, const float* __restrict__ kv,
    const float* __restrict__ ksum, T* __restrict__ o, int tokens,
    int heads) {
  __shared__ float z[kD][kD];
  __shared__ float dd[kD];
  const int h = blockIdx.y, b = blockIdx.z;
  const int C = heads * kD;
  const size_t bh = (size_t)b * heads + h;
  for (int e = threadIdx.x; e < kD * kD; e += 64) z[e / kD][e % kD] = kv[bh * kD * kD + e];
  if (threadIdx.x < kD) dd[threadIdx.x] = ksum[bh * kD + threadIdx.x];
  __syncthreads();
  const int n = blockIdx.x * 64 + threadIdx.x;
  if (n >= tokens) return;
  const T* q = qkvh + ((size_t)b * tokens + n) * 3 * C + h * kD;
  float fq[kD];
#pragma unroll
  for (int i = 0; i < kD; ++i) fq[i] = relu(to_f32(q[i]));
  float den = 0.f;
#pragma unroll
  for (int i = 0; i < kD; ++i) den = fmaf(fq[i], dd[i], den);
  T* out = o + ((size_t)b * tokens + n) * C + h * kD;
  const float inv = den > 0.f ? 1.f / den : 0.f;
  for (int j = 0; j < kD; ++j) {
    float num = 0.f;
#pragma unroll
    for (int i = 0; i < kD; ++i) num = fmaf(fq[i], z[i][j], num);
    out[j] = from_f32<T>(den > 0.f ? num * inv : 0.f);
  }
}

}  // namespace

int kv_chunks(int batch, int heads, int tokens) {
  // Enough workgroups to cover the chip (256 CUs) several times over, but
  // never chunks shorter than one LDS tile.
  const int bh = batch * heads;
  int chunks = (2048 + bh - 1) / bh;
  const int max_chunks = (tokens + kTok - 1) / kTok;
  if (chunks > max_chunks) chunks = max_chunks;
  if (chunks < 1) chunks = 1;
  return chunks;
}

hipError_t launch_kv_state(bool bf, const void* qkv_hat, float* kv,
                           float* ksum, float* partials, int batch, int tokens,
                           int heads, hipStream_t s) {
  const int chunks = kv_chunks(batch, heads, tokens);
  const int chunk_len = (tokens + chunks - 1) / chunks;
  dim3 grid(chunks, heads, batch);
  if (bf)
    kv_partial_kernel<bf16><<<grid, 256, 0, s>>>(
        static_cast<const bf16*>(qkv_hat), partials, tokens, heads, chunk_len);
  else
    kv_partial_kernel<float><<<grid, 256, 0, s>>>(
        static_cast<const float*>(qkv_hat), partials, tokens, heads, chunk_len);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  kv_combine_kernel<<<batch * heads, 256, 0, s>>>(partials, kv, ksum, chunks);
  return hipGetLastError();
}

hipError_t launch_lin_apply(bool bf, const void* qkv_hat, const float* kv,
                            const float* ksum, void* o, int batch, int tokens,
                            int heads, hipStream_t s) {
  dim3 grid((tokens + 63) / 64, heads, batch);
  if (bf)
    lin_apply_kernel<bf16><<<grid, 64, 0, s>>>(static_cast<const bf16*>(qkv_hat),
                                               kv, ksum, static_cast<bf16*>(o),
                                               tokens, heads);
  else
    lin_apply_kernel<float><<<grid, 64, 0, s>>>(static_cast<const float*>(qkv_hat),
                                                kv, ksum, static_cast<float*>(o),
                                                tokens, heads);
  return hipGetLastError();
}

}  // namespace hsmla
