// Dense projections: C = A . B (+ R).  FT 3.1 (Q, K, V = LinearProjection(X))
// and the C x C output projection that returns the module to C channels
// (FT 3.5 block equation); the FFN projections of the block use the same
// kernel.
#include "common.h"
#include "kernels.h"

namespace hsmla {
namespace {

constexpr int kTM = 64, kTN = 64, kTK = 16;

// 64x64 output tile per 256-thread workgroup, each thread a 4x4 sub-tile,
// float32 accumulation, K staged through LDS in steps of 16.
template <typename T>
__global__ __launch_bounds__(256) void gemm_valu(const T* __restrict__ A,
                                                 const T* __restrict__ B,
                                                 const T* __restrict__ R,
                                                 T* __restrict__ C, int M,
                                                 int N, int K) {
  __shared__ float As[kTK][kTM + 4];
  __shared__ float Bs[kTK][kTN + 4];
  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  const int m0 = blockIdx.y * kTM, n0 = blockIdx.x * kTN;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += kTK) {
    for (int i = tid; i < kTM * kTK; i += 256) {
      const int mm = i / kTK, kk = i % kTK;
      const int gm = m0 + mm, gk = k0 + kk;
      As[kk][mm] = (gm < M && gk < K) ? to_f32(A[(size_t)gm * K + gk]) : 0.f;
    }
    for (int i = tid; i < kTK * kTN; i += 256) {
      const int kk = i / kTN, nn = i % kTN;
      const int gk = k0 + kk, gn = n0 + nn;
      Bs[kk][nn] = (gk < K && gn < N) ? to_f32(B[(size_t)gk * N + gn]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kTK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gm = m0 + ty * 4 + i;
    if (gm >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + tx * 4 + j;
      if (gn >= N) continue;
      float v = acc[i][j];
      if (R) v += to_f32(R[(size_t)gm * N + gn]);
      C[(size_t)gm * N + gn] = from_f32<T>(v);
    }
  }
}

template <typename T>
hipError_t run(const void* A, const void* B, const void* R, void* C, int M,
               int N, int K, hipStream_t s) {
  dim3 grid((N + kTN - 1) / kTN, (M + kTM - 1) / kTM);
  gemm_valu<T><<<grid, 256, 0, s>>>(static_cast<const T*>(A),
                                    static_cast<const T*>(B),
                                    static_cast<const T*>(R),
                                    static_cast<T*>(C), M, N, K);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(bool bf, const void* A, const void* B, const void* R,
                       void* C, int M, int N, int K, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  return bf ? run<bf16>(A, B, R, C, M, N, K, s)
            : run<float>(A, B, R, C, M, N, K, s);
}

}  // namespace hsmla
