// Depthwise convolutions on the NHWC token grid.
//
// Multi-scale branches: T_hat = T + sum_s DWConv_{k_s}(T) for every channel
// of Q, K and V (abstract and EX section 2: depthwise kernels of several
// sizes enrich the tokens).  Because every branch is linear in T, the
// identity and all branches are folded into one kmax x kmax tap set per
// channel before the convolution runs.  The FFN's 3x3 depthwise conv (FT 3.5
// block equation) uses the same kernel with a GELU epilogue.
//
// Kernel shape: a workgroup owns 16 columns x 64 channels of a strip of 32
// output rows.  It streams the input rows of the strip (plus the vertical
// halo) through a double-buffered LDS row that carries the horizontal halo;
// each thread keeps the kmax partial output rows that the current input row
// feeds in registers, so every input element is read from HBM once and from
// LDS kmax times.  Each thread handles 4 consecutive channels (8-byte bf16
// accesses, 128 contiguous bytes per 16 lanes).
#include "common.h"
#include "kernels.h"

namespace hsmla {
namespace {

struct KernelSet {
  const void* p[3];
  int k[3];
};

// grid covers kmax*kmax taps x ch channels, one (tap, channel) per thread.
template <typename T>
__global__ void dw_taps_kernel(KernelSet ks, int nk, int kmax, int ch,
                               int identity, float* __restrict__ weff) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= kmax * kmax * ch) return;
  const int c = idx % ch, tap = idx / ch;
  const int dy = tap / kmax, dx = tap % kmax;
  const int rmax = (kmax - 1) / 2;
  float v = (identity && dy == rmax && dx == rmax) ? 1.f : 0.f;
  for (int i = 0; i < nk; ++i) {
    const int k = ks.k[i], r = (k - 1) / 2;
    const int ky = dy - rmax + r, kx = dx - rmax + r;
    if (ky >= 0 && ky < k && kx >= 0 && kx < k)
      v += to_f32(static_cast<const T*>(ks.p[i])[((size_t)c * k + ky) * k + kx]);
  }
  weff[idx] = v;
}

__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.f + erff(x * 0.70710678118654752f));
}

constexpr int TW = 16;   // output columns per workgroup
constexpr int CG = 16;   // 4-channel groups per workgroup (64 channels)
constexpr int TH = 32;   // output rows per workgroup strip

struct f4 {
  float v[4];
};

template <typename T>
__device__ __forceinline__ f4 load4(const T* p);
template <>
__device__ __forceinline__ f4 load4<bf16>(const bf16* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  f4 r;
  r.v[0] = __uint_as_float(u.x << 16);
  r.v[1] = __uint_as_float(u.x & 0xffff0000u);
  r.v[2] = __uint_as_float(u.y << 16);
  r.v[3] = __uint_as_float(u.y & 0xffff0000u);
  return r;
}
template <>
__device__ __forceinline__ f4 load4<float>(const float* p) {
  const float4 u = *reinterpret_cast<const float4*>(p);
  return f4{{u.x, u.y, u.z, u.w}};
}

template <typename T>
__device__ __forceinline__ void store4(T* p, const float* v);
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, const float* v) {
  uint2 o;
  o.x = (uint32_t)from_f32<bf16>(v[0]).u | ((uint32_t)from_f32<bf16>(v[1]).u << 16);
  o.y = (uint32_t)from_f32<bf16>(v[2]).u | ((uint32_t)from_f32<bf16>(v[3]).u << 16);
  *reinterpret_cast<uint2*>(p) = o;
}
template <>
__device__ __forceinline__ void store4<float>(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

// grid: (column tiles * channel tiles, row strips, batch); 256 threads.
template <typename T, int K, bool GELU>
__global__ __launch_bounds__(256) void dwconv_rows(
    const T* __restrict__ in, T* __restrict__ out,
    const float* __restrict__ weff, int gh, int gw, int ch, int col_tiles) {
  constexpr int R = (K - 1) / 2;
  constexpr int SEG = TW + 2 * R;  // columns held per LDS row
  __shared__ float4 row[2][SEG * CG];

  const int tc = threadIdx.x % CG;   // channel group within the tile
  const int tx = threadIdx.x / CG;   // output column within the tile
  const int x0 = (blockIdx.x % col_tiles) * TW;
  const int c0 = (blockIdx.x / col_tiles) * (CG * 4);
  const int y0 = blockIdx.y * TH;
  const int b = blockIdx.z;
  const int c = c0 + tc * 4;
  const bool c_ok = c < ch;
  const int x = x0 + tx;
  const size_t img = (size_t)b * gh * gw;

  // this thread's taps, K x K x 4 channels
  float w[K][K][4];
#pragma unroll
  for (int ky = 0; ky < K; ++ky)
#pragma unroll
    for (int kx = 0; kx < K; ++kx)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[ky][kx][j] = c_ok ? weff[(size_t)(ky * K + kx) * ch + c + j] : 0.f;

  float acc[K][4];
#pragma unroll
  for (int i = 0; i < K; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  const int y_end = min(gh, y0 + TH);
  const int r_begin = y0 - R, r_end = y_end + R;

  // Each thread stages up to two 4-channel vectors of an input row segment.
  // Loads for row r+1 are issued one iteration ahead and written to LDS
  // after the compute of row r, so their latency overlaps that compute.
  constexpr int kFill = (SEG * CG + 255) / 256;
  auto issue = [&](f4 (&st)[kFill], int r) {
#pragma unroll
    for (int i = 0; i < kFill; ++i) {
      const int e = threadIdx.x + 256 * i;
      const int sx = e / CG, sc = e % CG;
      const int gx = x0 - R + sx, gc = c0 + sc * 4;
      if (e < SEG * CG && r >= 0 && r < gh && gx >= 0 && gx < gw && gc < ch)
        st[i] = load4<T>(in + (img + (size_t)r * gw + gx) * ch + gc);
      else
        st[i] = f4{{0.f, 0.f, 0.f, 0.f}};
    }
  };
  auto commit = [&](const f4 (&st)[kFill], int buf) {
#pragma unroll
    for (int i = 0; i < kFill; ++i) {
      const int e = threadIdx.x + 256 * i;
      if (e < SEG * CG)
        row[buf][e] = make_float4(st[i].v[0], st[i].v[1], st[i].v[2], st[i].v[3]);
    }
  };

  f4 stage[kFill];
  issue(stage, r_begin);
  commit(stage, 0);
  if (r_begin + 1 < r_end) issue(stage, r_begin + 1);
  __syncthreads();
  for (int r = r_begin; r < r_end; ++r) {
    const int buf = (r - r_begin) & 1;
    float xin[K][4];
#pragma unroll
    for (int kx = 0; kx < K; ++kx) {
      const float4 v = row[buf][(tx + kx) * CG + tc];
      xin[kx][0] = v.x;
      xin[kx][1] = v.y;
      xin[kx][2] = v.z;
      xin[kx][3] = v.w;
    }
    // row r+1 (already in flight) goes to the other buffer; row r+2 is issued
    if (r + 1 < r_end) {
      commit(stage, buf ^ 1);
      if (r + 2 < r_end) issue(stage, r + 2);
    }
    // input row r feeds output row r - R + i with vertical tap K - 1 - i
#pragma unroll
    for (int i = 0; i < K; ++i)
#pragma unroll
      for (int kx = 0; kx < K; ++kx)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = fmaf(w[K - 1 - i][kx][j], xin[kx][j], acc[i][j]);
    const int yo = r - R;  // completed output row
    if (yo >= y0 && yo < y_end && x < gw && c_ok) {
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = GELU ? gelu_erf(acc[0][j]) : acc[0][j];
      store4<T>(out + (img + (size_t)yo * gw + x) * ch + c, v);
    }
#pragma unroll
    for (int i = 0; i + 1 < K; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = acc[i + 1][j];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[K - 1][j] = 0.f;
    __syncthreads();
  }
}

template <typename T, int K, bool GELU>
hipError_t run_dw(const void* in, void* out, const float* weff, int batch,
                  int gh, int gw, int ch, hipStream_t s) {
  const int col_tiles = (gw + TW - 1) / TW;
  const int ch_tiles = (ch + CG * 4 - 1) / (CG * 4);
  dim3 grid(col_tiles * ch_tiles, (gh + TH - 1) / TH, batch);
  dwconv_rows<T, K, GELU><<<grid, 256, 0, s>>>(
      static_cast<const T*>(in), static_cast<T*>(out), weff, gh, gw, ch,
      col_tiles);
  return hipGetLastError();
}

template <typename T, bool GELU>
hipError_t dispatch_k(int kmax, const void* in, void* out, const float* weff,
                      int batch, int gh, int gw, int ch, hipStream_t s) {
  switch (kmax) {
    case 1: return run_dw<T, 1, GELU>(in, out, weff, batch, gh, gw, ch, s);
    case 3: return run_dw<T, 3, GELU>(in, out, weff, batch, gh, gw, ch, s);
    case 5: return run_dw<T, 5, GELU>(in, out, weff, batch, gh, gw, ch, s);
    case 7: return run_dw<T, 7, GELU>(in, out, weff, batch, gh, gw, ch, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_dw_taps(bool bf, const void* const* kernels, const int* ks,
                          int nk, int kmax, int ch, int identity, float* weff,
                          hipStream_t s) {
  KernelSet set{};
  for (int i = 0; i < nk; ++i) {
    set.p[i] = kernels[i];
    set.k[i] = ks[i];
  }
  const unsigned blocks = (unsigned)((kmax * kmax * ch + 255) / 256);
  if (bf)
    dw_taps_kernel<bf16><<<blocks, 256, 0, s>>>(set, nk, kmax, ch, identity, weff);
  else
    dw_taps_kernel<float><<<blocks, 256, 0, s>>>(set, nk, kmax, ch, identity, weff);
  return hipGetLastError();
}

hipError_t launch_dwconv(bool bf, const void* in, void* out, const float* weff,
                         int kmax, int batch, int gh, int gw, int ch,
                         bool gelu, hipStream_t s) {
  if (bf)
    return gelu ? dispatch_k<bf16, true>(kmax, in, out, weff, batch, gh, gw, ch, s)
                : dispatch_k<bf16, false>(kmax, in, out, weff, batch, gh, gw, ch, s);
  return gelu ? dispatch_k<float, true>(kmax, in, out, weff, batch, gh, gw, ch, s)
              : dispatch_k<float, false>(kmax, in, out, weff, batch, gh, gw, ch, s);
}

}  // namespace hsmla
