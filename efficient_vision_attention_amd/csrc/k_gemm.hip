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
//
// Workgroup tile BM x BN, WGM x WGN waves each owning (BM/WGM) x (BN/WGN) =
// FM x FN fragments of 32 x 32 (v_mfma_f32_32x32x16_bf16).  A and W tiles of
// BK k go through double-buffered LDS (16-byte loads staged in registers one
// tile ahead, rows padded by 16 bytes).  The MFMA computes the transposed
// tile so each lane ends up with runs of 4 consecutive output columns; the
// finished tile is staged in LDS as float32 and written back row by row with
// 16-byte stores.  Tiles are remapped so each XCD walks whole row panels of A.
// ---------------------------------------------------------------------------

constexpr int kXcds = 8;

__device__ __forceinline__ uint4 ld16(const bf16* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// SITE only names the call site (one kernel symbol per projection, so
// profiles tell the four GEMMs apart); the code is the same.
template <int BM, int BN, int BK, int WGM, int WGN, int SITE>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_mfma_bf16(
    const bf16* __restrict__ A, const bf16* __restrict__ W,
    const bf16* __restrict__ R, bf16* __restrict__ C, int M, int N, int K,
    int tiles_n, int tiles_total, int per_xcd) {
  constexpr int NT = 64 * WGM * WGN;         // threads
  constexpr int STR = BK + 8;                // bf16 per LDS row
  constexpr int FM = BM / WGM / 32, FN = BN / WGN / 32;
  constexpr int CPR = BK / 8;                // 16-byte chunks per row
  constexpr int LA = BM * CPR / NT;          // A chunks per thread
  constexpr int LW = BN * CPR / NT;          // W chunks per thread
  static_assert(BM * CPR % NT == 0 && BN * CPR % NT == 0, "tile/threads");
  constexpr int TN = BN / WGN;                 // wave tile width
  constexpr int CSTR = TN + 4;                 // floats per staged row
  constexpr int kTileBytes = 2 * (BM + BN) * STR * 2;
  constexpr int kStageBytes = WGM * WGN * 32 * CSTR * 4;
  __shared__ __attribute__((aligned(16)))
      char smem[kTileBytes > kStageBytes ? kTileBytes : kStageBytes];
  bf16 (*As)[BM * STR] = reinterpret_cast<bf16 (*)[BM * STR]>(smem);
  bf16 (*Ws)[BN * STR] = reinterpret_cast<bf16 (*)[BN * STR]>(smem + 2 * BM * STR * 2);

  const int b = blockIdx.x;
  const int tile = (b % kXcds) * per_xcd + b / kXcds;
  if (tile >= tiles_total) return;
  const int m0 = (tile / tiles_n) * BM;
  const int n0 = (tile % tiles_n) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = (wave / WGN) * (BM / WGM), wn = (wave % WGN) * (BN / WGN);

  uint4 ra[LA], rw[LW];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int c = tid + NT * i;
      const int r = c / CPR, kc = (c % CPR) * 8;
      const int gm = m0 + r, gk = k0 + kc;
      ra[i] = (gm < M && gk < K) ? ld16(A + (size_t)gm * K + gk) : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < LW; ++i) {
      const int c = tid + NT * i;
      const int r = c / CPR, kc = (c % CPR) * 8;
      const int gn = n0 + r, gk = k0 + kc;
      rw[i] = (gn < N && gk < K) ? ld16(W + (size_t)gn * K + gk) : uint4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int c = tid + NT * i;
      *reinterpret_cast<uint4*>(&As[buf][(c / CPR) * STR + (c % CPR) * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < LW; ++i) {
      const int c = tid + NT * i;
      *reinterpret_cast<uint4*>(&Ws[buf][(c / CPR) * STR + (c % CPR) * 8]) = rw[i];
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
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
      bf16x8 af[FM], wf[FN];
#pragma unroll
      for (int t = 0; t < FM; ++t)
        af[t] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(
                        &As[cur][(wm + 32 * t + frow) * STR + ks + fk]));
#pragma unroll
      for (int t = 0; t < FN; ++t)
        wf[t] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(
                        &Ws[cur][(wn + 32 * t + frow) * STR + ks + fk]));
      // D^T tile: rows index output columns n, columns index rows m
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], af[i],
                                                              acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      store_tile(cur ^ 1);
      __syncthreads();
    }
  }

  // Epilogue through LDS: each wave stages one 32-row fragment row of its
  // tile at a time as float32 in its own slice of the (now idle) tile
  // buffers, then writes those rows back with 16-byte stores by consecutive
  // lanes (R added in float32, one rounding to bf16).
  float* Cs = reinterpret_cast<float*>(smem) + wave * 32 * CSTR;
  constexpr int CPRO = TN / 8;  // 16-byte output chunks per staged row
  __syncthreads();
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int cc = 32 * j + 8 * g + 4 * (lane >> 5);
        *reinterpret_cast<float4*>(&Cs[frow * CSTR + cc]) =
            make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                        acc[i][j][4 * g + 3]);
      }
    __syncthreads();
#pragma unroll
    for (int c = lane; c < 32 * CPRO; c += 64) {
      const int r = c / CPRO, cc = (c % CPRO) * 8;
      const int gm = m0 + wm + 32 * i + r, gn = n0 + wn + cc;
      if (gm >= M || gn >= N) continue;
      const float4 lo = *reinterpret_cast<const float4*>(&Cs[r * CSTR + cc]);
      const float4 hi = *reinterpret_cast<const float4*>(&Cs[r * CSTR + cc + 4]);
      float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      const size_t off = (size_t)gm * N + gn;
      if (R) {
        const uint4 rr = ld16(R + off);
        const uint32_t rw4[4] = {rr.x, rr.y, rr.z, rr.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[2 * q] += __uint_as_float(rw4[q] << 16);
          v[2 * q + 1] += __uint_as_float(rw4[q] & 0xffff0000u);
        }
      }
      *reinterpret_cast<uint4*>(C + off) =
          uint4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
    }
    __syncthreads();
  }
}

template <int BM, int BN, int BK, int WGM, int WGN, int SITE>
void run_tiles(const void* A, const void* W, const void* R, void* C, int M,
               int N, int K, hipStream_t s) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int total = tiles_m * tiles_n;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  gemm_mfma_bf16<BM, BN, BK, WGM, WGN, SITE><<<per_xcd * kXcds, 64 * WGM * WGN, 0, s>>>(
      static_cast<const bf16*>(A), static_cast<const bf16*>(W),
      static_cast<const bf16*>(R), static_cast<bf16*>(C), M, N, K, tiles_n,
      total, per_xcd);
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


// Tile shapes picked by measurement on MI355X for the projection shapes of
// the block (M = 65536): wide N with K = C favours 256x256 (8 waves) or
// 128x256 tiles, the C-wide outputs 128x128.
template <int SITE>
void run_mfma(const void* A, const void* W, const void* R, void* C, int M,
              int N, int K, hipStream_t s) {
  if (N >= 1024 && K <= 512 && M >= 8192) {
    if (N % 256 == 0)
      run_tiles<128, 256, 32, 2, 2, SITE>(A, W, R, C, M, N, K, s);
    else
      run_tiles<256, 256, 32, 4, 2, SITE>(A, W, R, C, M, N, K, s);
  } else if (K <= 512) {
    run_tiles<128, 128, 32, 2, 2, SITE>(A, W, R, C, M, N, K, s);
  } else {
    run_tiles<128, 128, 64, 2, 2, SITE>(A, W, R, C, M, N, K, s);
  }
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
