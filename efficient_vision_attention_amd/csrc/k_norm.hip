// LayerNorm over channels for the block wrapper (FT 3.5 block equation).
// Biased variance, eps 1e-5 (the usual definition; the pages do not state
// it).  Two passes over registers (mean, then centred variance).  Rows of
// 128, 256, 384 or 512 bf16 channels (or 64 .. 256 float32) take 16 lanes
// each; other widths one wavefront per row.
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
  __device__ static uint4 raw(const bf16* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ static void load(const bf16* p, float* v) { cvt(raw(p), v); }
  __device__ static void cvt(const uint4 u, float* v) {
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
  __device__ static uint4 raw(const float* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ static void load(const float* p, float* v) { cvt(raw(p), v); }
  __device__ static void cvt(const uint4 u, float* v) {
    v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
  }
  __device__ static void store(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// One wavefront per row, kRows rows per wave with all loads issued first;
// lane l handles the 16-byte vectors l, l + 64, ... of a row.
constexpr int kRows = 4;

// NI = 16-byte vectors per lane (ceil(ch / V / 64)).
template <typename T, int NI>
__global__ __launch_bounds__(256) void layernorm_kernel(
    const T* __restrict__ x, const float* __restrict__ g,
    const float* __restrict__ be, T* __restrict__ y, int rows, int ch) {
  constexpr int V = Vec<T>::N;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int row0 = (blockIdx.x * 4 + wave) * kRows;
  const int nvec = ch / V;
  float v[kRows][NI][V];
#pragma unroll
  for (int q = 0; q < kRows; ++q) {
    const int row = row0 + q;
    const T* xr = x + (size_t)(row < rows ? row : 0) * ch;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int vi = lane + 64 * i;
      if (vi < nvec && row < rows) {
        Vec<T>::load(xr + vi * V, v[q][i]);
      } else {
#pragma unroll
        for (int j = 0; j < V; ++j) v[q][i][j] = 0.f;
      }
    }
  }
#pragma unroll
  for (int q = 0; q < kRows; ++q) {
    const int row = row0 + q;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < V; ++j) s += v[q][i][j];
    const float mean = wave_sum(s) / (float)ch;
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (lane + 64 * i < nvec) {
#pragma unroll
        for (int j = 0; j < V; ++j) {
          const float dlt = v[q][i][j] - mean;
          sq = fmaf(dlt, dlt, sq);
        }
      }
    }
    const float rstd = rsqrtf(wave_sum(sq) / (float)ch + 1e-5f);
    if (row >= rows) continue;
    T* yr = y + (size_t)row * ch;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int vi = lane + 64 * i;
      if (vi >= nvec) continue;
      float o[V];
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int c = vi * V + j;
        o[j] = (v[q][i][j] - mean) * rstd * g[c] + be[c];
      }
      Vec<T>::store(yr + vi * V, o);
    }
  }
}

// Rows whose 16-byte vectors split evenly over 16 lanes (channels a multiple
// of 16 vectors, up to 128 per row): 16 lanes per row, so a wave holds 4
// rows at once with every lane busy, and kSteps of those 4-row groups have
// all their loads in flight before any reduction (kept as raw 16-byte
// vectors and converted at each use).  gamma and beta stay in registers
// across the rows of a wave.  Reductions use xor shuffles inside the 16-lane
// group, in a fixed order.  Two groups per wave (8 rows) measured faster
// than four or eight (C = 384: 22.0 -> 20.3 us and 20.6 -> 18.8 us for the
// block's two norms against four; one group no faster): more, shorter waves
// spread each CU's reads and writes over time instead of issuing them all
// at once.
constexpr int kSteps = 2;

// BLK: y is written tile-blocked for the GEMM (row r, channel k at
// ((r / 256) * (ch / 32) + k / 32) * 8192 + (r % 256) * 32 + k % 32).
template <typename T, int NV, bool BLK>
__global__ __launch_bounds__(256) void layernorm16_kernel(
    const T* __restrict__ x, const float* __restrict__ g,
    const float* __restrict__ be, T* __restrict__ y, int rows, int ch) {
  constexpr int V = Vec<T>::N;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int grp = lane / 16, gl = lane % 16;
  const int row_base = (blockIdx.x * 4 + wave) * 4 * kSteps;
  float gv[NV][V], bv[NV][V];
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int c = (gl + 16 * i) * V + j;
      gv[i][j] = g[c];
      bv[i][j] = be[c];
    }
  uint4 raw[kSteps][NV];
#pragma unroll
  for (int q = 0; q < kSteps; ++q) {
    const int row = min(row_base + 4 * q + grp, rows - 1);
    const T* xr = x + (size_t)row * ch;
#pragma unroll
    for (int i = 0; i < NV; ++i) raw[q][i] = Vec<T>::raw(xr + (gl + 16 * i) * V);
  }
  const float inv_ch = 1.f / (float)ch;
#pragma unroll
  for (int q = 0; q < kSteps; ++q) {
    const int row = row_base + 4 * q + grp;
    float v[NV][V];
#pragma unroll
    for (int i = 0; i < NV; ++i) Vec<T>::cvt(raw[q][i], v[i]);
    float sm = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int j = 0; j < V; ++j) sm += v[i][j];
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) sm += __shfl_xor(sm, off, 16);
    const float mean = sm * inv_ch;
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const float dlt = v[i][j] - mean;
        sq = fmaf(dlt, dlt, sq);
      }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) sq += __shfl_xor(sq, off, 16);
    const float rstd = rsqrtf(sq * inv_ch + 1e-5f);
    if (row >= rows) continue;
    T* yr = y + (size_t)row * ch;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float o[V];
#pragma unroll
      for (int j = 0; j < V; ++j) o[j] = (v[i][j] - mean) * rstd * gv[i][j] + bv[i][j];
      const int k = (gl + 16 * i) * V;
      if constexpr (BLK)
        Vec<T>::store(y + ((size_t)(row / kGemmTileM) * (ch / kGemmTileK) + k / kGemmTileK) *
                              (kGemmTileM * kGemmTileK) +
                          (row % kGemmTileM) * kGemmTileK + k % kGemmTileK,
                      o);
      else
        Vec<T>::store(yr + k, o);
    }
  }
}

template <typename T, int NV>
hipError_t run_ln16(const T* x, const float* gamma, const float* beta, T* y,
                    int rows, int ch, bool blocked, hipStream_t s) {
  const unsigned blocks = (unsigned)((rows + 16 * kSteps - 1) / (16 * kSteps));
  if (blocked)
    layernorm16_kernel<T, NV, true><<<blocks, 256, 0, s>>>(x, gamma, beta, y, rows, ch);
  else
    layernorm16_kernel<T, NV, false><<<blocks, 256, 0, s>>>(x, gamma, beta, y, rows, ch);
  return hipGetLastError();
}

template <typename T>
hipError_t run_ln(const void* x, const float* gamma, const float* beta, void* y,
                  int rows, int ch, bool blocked, hipStream_t s) {
  const unsigned blocks = (unsigned)((rows + 4 * kRows - 1) / (4 * kRows));
  const int ni = (ch / Vec<T>::N + 63) / 64;
  const T* xi = static_cast<const T*>(x);
  T* yo = static_cast<T*>(y);
  const int nvec = ch / Vec<T>::N;
  if (nvec % 16 == 0) {
    switch (nvec / 16) {
      case 1: return run_ln16<T, 1>(xi, gamma, beta, yo, rows, ch, blocked, s);
      case 2: return run_ln16<T, 2>(xi, gamma, beta, yo, rows, ch, blocked, s);
      case 3: return run_ln16<T, 3>(xi, gamma, beta, yo, rows, ch, blocked, s);
      case 4: return run_ln16<T, 4>(xi, gamma, beta, yo, rows, ch, blocked, s);
      default: break;
    }
  }
  if (blocked) return hipErrorInvalidValue;
  if (ni <= 1)
    layernorm_kernel<T, 1><<<blocks, 256, 0, s>>>(xi, gamma, beta, yo, rows, ch);
  else if (ni <= 2)
    layernorm_kernel<T, 2><<<blocks, 256, 0, s>>>(xi, gamma, beta, yo, rows, ch);
  else if (ni <= 4)
    layernorm_kernel<T, 4><<<blocks, 256, 0, s>>>(xi, gamma, beta, yo, rows, ch);
  else
    layernorm_kernel<T, kMaxPerLane / Vec<T>::N><<<blocks, 256, 0, s>>>(
        xi, gamma, beta, yo, rows, ch);
  return hipGetLastError();
}

}  // namespace

bool layernorm_can_block(bool bf, int rows, int ch) {
  const int nvec = ch / 8;
  return bf && ch % 8 == 0 && nvec % 16 == 0 && nvec / 16 <= 4 &&
         rows % kGemmTileM == 0 && ch % kGemmTileK == 0;
}

hipError_t launch_layernorm(bool bf, const void* x, const float* gamma,
                            const float* beta, void* y, int rows, int ch,
                            hipStream_t s, bool blocked) {
  if (blocked && !layernorm_can_block(bf, rows, ch)) return hipErrorInvalidValue;
  return bf ? run_ln<bf16>(x, gamma, beta, y, rows, ch, blocked, s)
            : run_ln<float>(x, gamma, beta, y, rows, ch, blocked, s);
}

}  // namespace hsmla
