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
// output rows; each thread handles 4 consecutive channels of one column
// (8-byte bf16 accesses, 128 contiguous bytes per 16 lanes) and keeps the
// kmax partial output rows that the current input row feeds in registers.
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

// GELU(x) = x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)) with erf from
// Abramowitz & Stegun 7.1.26 (Hastings' rational approximation):
//   erf(z) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2),
//   t = 1 / (1 + p z),  z >= 0,  |error| <= 1.5e-7,
// extended to z < 0 by oddness.  Far below the bfloat16 output precision.
__device__ __forceinline__ float gelu_erf(float x) {
  constexpr float p = 0.3275911f, a1 = 0.254829592f, a2 = -0.284496736f,
                  a3 = 1.421413741f, a4 = -1.453152027f, a5 = 1.061405429f;
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(p, z, 1.f));
  const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, a5, a4), a3), a2), a1);
  const float e = __builtin_amdgcn_exp2f(-z * z * 1.4426950408889634f);
  const float erf_abs = fmaf(-poly, e, 1.f);
  const float erf_v = copysignf(erf_abs, x);
  return 0.5f * x * (1.f + erf_v);
}

constexpr int TH = 32;   // output rows per workgroup strip
constexpr int kPoolMinBlock = 4;
constexpr int kXcds = 8;
constexpr int kWgChannels = 64;  // channels per workgroup

// V consecutive channels as loaded from memory (V = 2 or 4), converted to
// float at use.
template <typename T, int V>
struct Raw;
template <>
struct Raw<bf16, 4> {
  uint2 u;
  __device__ __forceinline__ void load(const bf16* p) { u = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void cvt(float* f) const {
    f[0] = __uint_as_float(u.x << 16);
    f[1] = __uint_as_float(u.x & 0xffff0000u);
    f[2] = __uint_as_float(u.y << 16);
    f[3] = __uint_as_float(u.y & 0xffff0000u);
  }
};
template <>
struct Raw<bf16, 2> {
  uint32_t u;
  __device__ __forceinline__ void load(const bf16* p) { u = *reinterpret_cast<const uint32_t*>(p); }
  __device__ __forceinline__ void cvt(float* f) const {
    f[0] = __uint_as_float(u << 16);
    f[1] = __uint_as_float(u & 0xffff0000u);
  }
};
template <>
struct Raw<float, 4> {
  float4 u;
  __device__ __forceinline__ void load(const float* p) { u = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ void cvt(float* f) const {
    f[0] = u.x; f[1] = u.y; f[2] = u.z; f[3] = u.w;
  }
};
template <>
struct Raw<float, 2> {
  float2 u;
  __device__ __forceinline__ void load(const float* p) { u = *reinterpret_cast<const float2*>(p); }
  __device__ __forceinline__ void cvt(float* f) const { f[0] = u.x; f[1] = u.y; }
};

template <typename T, int V>
__device__ __forceinline__ void storev(T* p, const float* v);
template <>
__device__ __forceinline__ void storev<bf16, 4>(bf16* p, const float* v) {
  *reinterpret_cast<uint2*>(p) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
template <>
__device__ __forceinline__ void storev<bf16, 2>(bf16* p, const float* v) {
  *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(v[0], v[1]);
}
template <>
__device__ __forceinline__ void storev<float, 4>(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
template <>
__device__ __forceinline__ void storev<float, 2>(float* p, const float* v) {
  *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
}

// Store, and leave in v the values as stored (rounded to T).
template <typename T, int V>
__device__ __forceinline__ void storev_round(T* p, float* v) {
  if constexpr (sizeof(T) == 4) {
    storev<T, V>(p, v);
  } else {
    uint32_t w[V / 2];
#pragma unroll
    for (int i = 0; i < V / 2; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    if constexpr (V == 4)
      *reinterpret_cast<uint2*>(p) = uint2{w[0], w[1]};
    else
      *reinterpret_cast<uint32_t*>(p) = w[0];
#pragma unroll
    for (int i = 0; i < V / 2; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}

// A thread owns one output column x and V consecutive channels of a 32-row
// strip and walks down the input rows of the strip.  For each input row it
// loads the K horizontal neighbours it needs (the K-fold reuse across
// neighbouring threads is served by the L1), and the row feeds the K partial
// output rows it belongs to, kept in registers.  NB rows of loads are in
// flight at any time; there is no LDS and no barrier, so every wave streams
// independently.  A workgroup covers 64 channels x (256 V / 64) columns.
// Grid: 1-D over (batch, strip, channel tile, column tile) with the column
// tile fastest, remapped so each XCD walks a contiguous run of neighbouring
// tiles (their halo columns then hit in that XCD's L2).
// With POOL the kernel also writes, for the gate, the sum over every
// block x block block of the values it stores (as stored, i.e. after
// rounding to T): bsum[b][t][c].  Each thread adds its column's rows and
// parks the sum of each finished block row in LDS (its own slot, no
// barrier); after the strip one barrier, then the block's columns are
// added in order.  block must divide the workgroup width and the strip
// height, and be at least kPoolMinBlock (LDS room).
template <typename T, int K, bool GELU, int V, int NB, bool POOL>
__global__ __launch_bounds__(256) void dwconv_stream(
    const T* __restrict__ in, T* __restrict__ out,
    const float* __restrict__ weff, float* __restrict__ bsum, int block,
    int gh, int gw, int ch, int col_tiles, int ch_tiles, int strips,
    int total, int per_xcd) {
  constexpr int R = (K - 1) / 2;
  constexpr int CG = kWgChannels / V;  // channel groups per workgroup
  constexpr int TW = 256 / CG;         // columns per workgroup
  __shared__ float red[POOL ? TH / kPoolMinBlock : 1][POOL ? TW : 1][POOL ? kWgChannels : 1];
  const int bid = blockIdx.x;
  const int tile = (bid % kXcds) * per_xcd + bid / kXcds;
  if (tile >= total) return;
  int rest = tile;
  const int col_t = rest % col_tiles;
  rest /= col_tiles;
  const int ch_t = rest % ch_tiles;
  rest /= ch_tiles;
  const int strip = rest % strips;
  const int b = rest / strips;

  const int tc = threadIdx.x % CG;
  const int tx = threadIdx.x / CG;
  const int x = col_t * TW + tx;
  const int c = ch_t * kWgChannels + tc * V;
  const bool c_ok = c < ch;
  const int y0 = strip * TH;
  const size_t img = (size_t)b * gh * gw;

  float w[K][K][V];
#pragma unroll
  for (int ky = 0; ky < K; ++ky)
#pragma unroll
    for (int kx = 0; kx < K; ++kx)
#pragma unroll
      for (int j = 0; j < V; ++j)
        w[ky][kx][j] = c_ok ? weff[(size_t)(ky * K + kx) * ch + c + j] : 0.f;

  float acc[K][V];
#pragma unroll
  for (int i = 0; i < K; ++i)
#pragma unroll
    for (int j = 0; j < V; ++j) acc[i][j] = 0.f;
  float psum[V];
#pragma unroll
  for (int j = 0; j < V; ++j) psum[j] = 0.f;

  const int y_end = min(gh, y0 + TH);
  const int r_begin = y0 - R, r_end = y_end + R;

  // Branch-free row loads: addresses are clamped into the tensor and the
  // values of out-of-grid taps are zeroed afterwards.
  const int cc = c_ok ? c : ch - V;
  bool col_ok[K];
  int col_off[K];
#pragma unroll
  for (int kx = 0; kx < K; ++kx) {
    const int xx = x + kx - R;
    col_ok[kx] = xx >= 0 && xx < gw;
    col_off[kx] = min(max(xx, 0), gw - 1) * ch + cc;
  }
  auto load_row = [&](Raw<T, V> (&rr)[K], int r) {
    const T* base = in + (img + (size_t)min(max(r, 0), gh - 1) * gw) * ch;
#pragma unroll
    for (int kx = 0; kx < K; ++kx) rr[kx].load(base + col_off[kx]);
  };
  // only tiles touching the left/right border have lanes with invalid taps
  const bool edge_tile = col_t * TW - R < 0 || col_t * TW + TW + R > gw;

  Raw<T, V> rbuf[NB][K];
#pragma unroll
  for (int q = 0; q < NB; ++q) load_row(rbuf[q], r_begin + q);
  // Rows are processed in groups of NB*K so that both the accumulator ring
  // slot ((row - r_begin) mod K) and the staging buffer ((row - r_begin) mod
  // NB) are compile-time constants of the unrolled body.
  for (int r0 = r_begin; r0 < r_end; r0 += NB * K) {
#pragma unroll
    for (int u = 0; u < NB * K; ++u) {
      const int r = r0 + u;
      if (r >= r_end) break;
      Raw<T, V>(&cur)[K] = rbuf[u % NB];
      // A halo row outside the grid contributes nothing: skip it (uniform).
      if (r >= 0 && r < gh) {
        float xin[K][V];
#pragma unroll
        for (int kx = 0; kx < K; ++kx) cur[kx].cvt(xin[kx]);
        if (edge_tile) {
#pragma unroll
          for (int kx = 0; kx < K; ++kx)
#pragma unroll
            for (int j = 0; j < V; ++j) xin[kx][j] = col_ok[kx] ? xin[kx][j] : 0.f;
        }
        // input row r feeds output row r - R + i with vertical tap K - 1 - i
#pragma unroll
        for (int i = 0; i < K; ++i) {
          const int slot = (u - R + i + NB * K) % K;
#pragma unroll
          for (int kx = 0; kx < K; ++kx)
#pragma unroll
            for (int j = 0; j < V; ++j)
              acc[slot][j] = fmaf(w[K - 1 - i][kx][j], xin[kx][j], acc[slot][j]);
        }
      }
      // unconditional (clamped) prefetch keeps the load/wait pattern regular
      load_row(cur, r + NB);
      const int done = (u - R + NB * K) % K;  // slot of output row r - R
      const int yo = r - R;
      if (yo >= y0 && yo < y_end && x < gw && c_ok) {
        float v[V];
#pragma unroll
        for (int j = 0; j < V; ++j) v[j] = GELU ? gelu_erf(acc[done][j]) : acc[done][j];
        if constexpr (POOL) {
          storev_round<T, V>(out + (img + (size_t)yo * gw + x) * ch + c, v);
#pragma unroll
          for (int j = 0; j < V; ++j) psum[j] += v[j];
        } else {
          storev<T, V>(out + (img + (size_t)yo * gw + x) * ch + c, v);
        }
      }
      if constexpr (POOL) {
        // end of a block row: park this thread's column sums
        if (yo >= y0 && yo < y_end && (yo + 1) % block == 0) {
          const int br = (yo - y0) / block;
#pragma unroll
          for (int j = 0; j < V; ++j) {
            red[br][tx][tc * V + j] = psum[j];
            psum[j] = 0.f;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < V; ++j) acc[done][j] = 0.f;
    }
  }
  if constexpr (POOL) {
    __syncthreads();
    if (tx % block == 0 && x < gw && c_ok) {
      const int nbc = gw / block;
      for (int br = 0; br < (y_end - y0) / block; ++br) {
        const size_t t = (size_t)(y0 / block + br) * nbc + x / block;
        float* dst = bsum + ((size_t)b * (gh / block) * nbc + t) * ch + c;
#pragma unroll
        for (int j = 0; j < V; ++j) {
          float sm = 0.f;
          for (int q = 0; q < block; ++q) sm += red[br][tx + q][tc * V + j];
          dst[j] = sm;
        }
      }
    }
  }
}

template <typename T, int K, bool GELU, int V, int NB = 3>
hipError_t run_dw(const void* in, void* out, const float* weff, float* bsum,
                  int block, int batch, int gh, int gw, int ch, hipStream_t s) {
  constexpr int TW = 256 / (kWgChannels / V);
  const int col_tiles = (gw + TW - 1) / TW;
  const int ch_tiles = (ch + kWgChannels - 1) / kWgChannels;
  const int strips = (gh + TH - 1) / TH;
  const int total = col_tiles * ch_tiles * strips * batch;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  if constexpr (!GELU) {
    if (bsum) {
      dwconv_stream<T, K, false, V, NB, true><<<per_xcd * kXcds, 256, 0, s>>>(
          static_cast<const T*>(in), static_cast<T*>(out), weff, bsum, block, gh,
          gw, ch, col_tiles, ch_tiles, strips, total, per_xcd);
      return hipGetLastError();
    }
  }
    dwconv_stream<T, K, GELU, V, NB, false><<<per_xcd * kXcds, 256, 0, s>>>(
        static_cast<const T*>(in), static_cast<T*>(out), weff, nullptr, 1, gh,
        gw, ch, col_tiles, ch_tiles, strips, total, per_xcd);
  return hipGetLastError();
}

// Wider kernels keep fewer channels per thread so their taps fit in
// registers at useful occupancy; rows in flight (NB) measured per size.
// channels per thread for each kernel size (also fixes the workgroup width)
constexpr int vec_for(int kmax) { return kmax <= 3 ? 4 : 2; }

template <typename T, bool GELU>
hipError_t dispatch_k(int kmax, const void* in, void* out, const float* weff,
                      float* bsum, int block, int batch, int gh, int gw, int ch,
                      hipStream_t s) {
  switch (kmax) {
    case 1: return run_dw<T, 1, GELU, vec_for(1)>(in, out, weff, bsum, block, batch, gh, gw, ch, s);
    case 3: return run_dw<T, 3, GELU, vec_for(3), GELU ? 2 : 3>(in, out, weff, bsum, block, batch, gh, gw, ch, s);
    case 5: return run_dw<T, 5, GELU, vec_for(5), 4>(in, out, weff, bsum, block, batch, gh, gw, ch, s);
    case 7: return run_dw<T, 7, GELU, vec_for(7), 3>(in, out, weff, bsum, block, batch, gh, gw, ch, s);
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

bool dwconv_can_pool(int kmax, int block) {
  const int tw = 256 / (kWgChannels / vec_for(kmax));
  return block >= kPoolMinBlock && tw % block == 0 && TH % block == 0;
}

hipError_t launch_dwconv(bool bf, const void* in, void* out, const float* weff,
                         int kmax, int batch, int gh, int gw, int ch,
                         bool gelu, float* bsum, int block, hipStream_t s) {
  if (bsum && (gelu || !dwconv_can_pool(kmax, block))) return hipErrorInvalidValue;
  if (bf)
    return gelu ? dispatch_k<bf16, true>(kmax, in, out, weff, nullptr, 1, batch, gh, gw, ch, s)
                : dispatch_k<bf16, false>(kmax, in, out, weff, bsum, block, batch, gh, gw, ch, s);
  return gelu ? dispatch_k<float, true>(kmax, in, out, weff, nullptr, 1, batch, gh, gw, ch, s)
              : dispatch_k<float, false>(kmax, in, out, weff, bsum, block, batch, gh, gw, ch, s);
}

}  // namespace hsmla
