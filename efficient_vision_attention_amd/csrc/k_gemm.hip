// Dense projections: C = A . W^T (+ R).  FT 3.1 (Q, K, V = LinearProjection(X))
// and the C x C output projection that returns the module to C channels
// (FT 3.5 block equation); the FFN projections of the block use the same
// kernels.
//
// A is [M][K] row-major (tokens x input channels), W is [N][K] row-major
// (output x input channels, the nn.Linear layout), so both MFMA operands read
// eight consecutive k values per lane straight from a row.
//
// bfloat16: 128x128 output tile per 256-thread workgroup (2x2 waves of 64x64,
// each a 2x2 grid of 32x32x16 MFMAs), K staged through double-buffered LDS in
// steps of 64, workgroups mapped so that each XCD walks whole row panels of A
// (its L2 then serves the A panel to every column tile).
// float32: a plain LDS-tiled FMA kernel (small shapes only).
#include "common.h"
#include "kernels.h"

namespace hsmla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// bfloat16 MFMA kernel
// ---------------------------------------------------------------------------

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // bf16 per LDS row (16-byte pad)
constexpr int kXcds = 8;

__device__ __forceinline__ uint4 ld16(const bf16* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// SITE only names the call site (one kernel symbol per projection, so
// profiles tell the four GEMMs apart); the code is the same.
template <int SITE>
__global__ __launch_bounds__(256, 2) void gemm_mfma_bf16(
    const bf16* __restrict__ A, const bf16* __restrict__ W,
    const bf16* __restrict__ R, bf16* __restrict__ C, int M, int N, int K,
    int tiles_n, int tiles_total, int per_xcd) {
  __shared__ __attribute__((aligned(16))) bf16 As[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) bf16 Ws[2][BN * LDS_STRIDE];

  // XCD-aware tile order: dispatch id b runs on XCD b % 8; give that XCD a
  // contiguous range of tiles, row panel by row panel.
  const int b = blockIdx.x;
  const int tile = (b % kXcds) * per_xcd + b / kXcds;
  if (tile >= tiles_total) return;
  const int m0 = (tile / tiles_n) * BM;
  const int n0 = (tile % tiles_n) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;

  // global -> register staging: 4 x 16 bytes of A and of W per thread
  uint4 ra[4], rw[4];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;         // 16-byte chunk id in the tile
      const int r = c >> 3, kc = (c & 7) * 8;
      const int gk = k0 + kc;
      const int gm = m0 + r, gn = n0 + r;
      ra[i] = (gm < M && gk < K) ? ld16(A + (size_t)gm * K + gk) : uint4{0, 0, 0, 0};
      rw[i] = (gn < N && gk < K) ? ld16(W + (size_t)gn * K + gk) : uint4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int r = c >> 3, kc = (c & 7) * 8;
      *reinterpret_cast<uint4*>(&As[buf][r * LDS_STRIDE + kc]) = ra[i];
      *reinterpret_cast<uint4*>(&Ws[buf][r * LDS_STRIDE + kc]) = rw[i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (K + BK - 1) / BK;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  const int frow = lane & 31;          // operand row within a 32-row fragment
  const int fk = (lane >> 5) * 8;      // operand k offset within a 16-k step
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tile((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK; ks += 16) {
      bf16x8 af[2], wf[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        af[t] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(
                        &As[cur][(wm + 32 * t + frow) * LDS_STRIDE + ks + fk]));
        wf[t] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(
                        &Ws[cur][(wn + 32 * t + frow) * LDS_STRIDE + ks + fk]));
      }
      // D^T tile: rows index output columns n, columns index rows m, so that
      // each lane ends up holding runs of 4 consecutive n of one row m.
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], af[i],
                                                              acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      store_tile(cur ^ 1);
      __syncthreads();
    }
  }

  // epilogue: lane holds C[m][n .. n+3] for 4 runs; add R, round, store 8 B
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int gm = m0 + wm + 32 * i + (lane & 31);
    if (gm >= M) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int gn = n0 + wn + 32 * j + 8 * g + 4 * (lane >> 5);
        if (gn >= N) continue;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * g + r];
        const size_t off = (size_t)gm * N + gn;
        if (R) {
          const uint2 rr = *reinterpret_cast<const uint2*>(R + off);
          v[0] += __uint_as_float(rr.x << 16);
          v[1] += __uint_as_float(rr.x & 0xffff0000u);
          v[2] += __uint_as_float(rr.y << 16);
          v[3] += __uint_as_float(rr.y & 0xffff0000u);
        }
        uint2 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(C + off) = o;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// float32 FMA kernel
// ---------------------------------------------------------------------------

constexpr int kTM = 64, kTN = 64, kTK = 16;

__global__ __launch_bounds__(256) void gemm_f32(const float* __restrict__ A,
                                                const float* __restrict__ W,
                                                const float* __restrict__ R,
                                                float* __restrict__ C, int M,
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
      As[kk][mm] = (gm < M && gk < K) ? A[(size_t)gm * K + gk] : 0.f;
    }
    for (int i = tid; i < kTN * kTK; i += 256) {
      const int nn = i / kTK, kk = i % kTK;
      const int gn = n0 + nn, gk = k0 + kk;
      Bs[kk][nn] = (gk < K && gn < N) ? W[(size_t)gn * K + gk] : 0.f;
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
      if (R) v += R[(size_t)gm * N + gn];
      C[(size_t)gm * N + gn] = v;
    }
  }
}


template <int SITE>
void run_mfma(const void* A, const void* W, const void* R, void* C, int M,
              int N, int K, hipStream_t s) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int total = tiles_m * tiles_n;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  gemm_mfma_bf16<SITE><<<per_xcd * kXcds, 256, 0, s>>>(
      static_cast<const bf16*>(A), static_cast<const bf16*>(W),
      static_cast<const bf16*>(R), static_cast<bf16*>(C), M, N, K, tiles_n,
      total, per_xcd);
}

}  // namespace

hipError_t launch_gemm(bool bf, const void* A, const void* W, const void* R,
                       void* C, int M, int N, int K, hipStream_t s,
                       GemmSite site) {
  if (M == 0 || N == 0) return hipSuccess;
  if (bf) {
    switch (site) {
      case GemmSite::kQkv: run_mfma<0>(A, W, R, C, M, N, K, s); break;
      case GemmSite::kOut: run_mfma<1>(A, W, R, C, M, N, K, s); break;
      case GemmSite::kFfn1: run_mfma<2>(A, W, R, C, M, N, K, s); break;
      default: run_mfma<3>(A, W, R, C, M, N, K, s); break;
    }
  } else {
    dim3 grid((N + kTN - 1) / kTN, (M + kTM - 1) / kTM);
    gemm_f32<<<grid, 256, 0, s>>>(static_cast<const float*>(A),
                                  static_cast<const float*>(W),
                                  static_cast<const float*>(R),
                                  static_cast<float*>(C), M, N, K);
  }
  return hipGetLastError();
}

}  // namespace hsmla
