// Depthwise convolutions on the NHWC token grid.
//
// Multi-scale branches: T_hat = T + sum_s DWConv_{k_s}(T) for every channel
// of Q, K and V (abstract and EX section 2: depthwise kernels of several
// sizes enrich the tokens).  Because every branch is linear in T, the
// identity and all branches are folded into one kmax x kmax tap set per
// channel before the convolution runs.  The FFN's 3x3 depthwise conv (FT 3.5
// block equation) uses the same kernel with a GELU epilogue.
//
// Two kernel shapes, both walking down a strip of 32 output rows with the
// kmax partial output rows that the current input row feeds kept in
// registers: up to 3x3 the workgroup stages each input row in LDS and every
// thread reads its horizontal neighbours there (dwconv_lds); the 5x5 and 7x7
// tap sets take so many registers that a register-only kernel, each thread
// loading its neighbours through L1, keeps more loads in flight
// (dwconv_stream).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace hsmla {
namespace {

constexpr int TH = 32;   // output rows per workgroup strip
constexpr int kPoolMinBlock = 4;
constexpr int kXcds = 8;

// V consecutive channels as loaded (V = 2, 4 or 8), converted to float at
// use.
template <typename T, int V>
struct Raw;
template <>
struct Raw<bf16, 8> {
  uint4 u;
  __device__ __forceinline__ void load(const bf16* p) { u = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, int off) {
    const i32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    u = uint4{(uint32_t)t.x, (uint32_t)t.y, (uint32_t)t.z, (uint32_t)t.w};
  }
  __device__ __forceinline__ void cvt(float* f) const {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <>
struct Raw<float, 8> {
  float4 u, v;
  __device__ __forceinline__ void load(const float* p) {
    u = *reinterpret_cast<const float4*>(p);
    v = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, int off) {
    const i32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    const i32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, off == kOob ? off : off + 16, 0, 0);
    u = make_float4(__int_as_float(a.x), __int_as_float(a.y), __int_as_float(a.z), __int_as_float(a.w));
    v = make_float4(__int_as_float(b.x), __int_as_float(b.y), __int_as_float(b.z), __int_as_float(b.w));
  }
  __device__ __forceinline__ void cvt(float* f) const {
    f[0] = u.x; f[1] = u.y; f[2] = u.z; f[3] = u.w;
    f[4] = v.x; f[5] = v.y; f[6] = v.z; f[7] = v.w;
  }
};
template <>
struct Raw<bf16, 4> {
  uint2 u;
  __device__ __forceinline__ void load(const bf16* p) { u = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, int off) {
    const i32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    u = uint2{(uint32_t)t.x, (uint32_t)t.y};
  }
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
  __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, int off) {
    u = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
  __device__ __forceinline__ void cvt(float* f) const {
    f[0] = __uint_as_float(u << 16);
    f[1] = __uint_as_float(u & 0xffff0000u);
  }
};
template <>
struct Raw<float, 4> {
  float4 u;
  __device__ __forceinline__ void load(const float* p) { u = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, int off) {
    const i32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    u = make_float4(__int_as_float(t.x), __int_as_float(t.y), __int_as_float(t.z), __int_as_float(t.w));
  }
  __device__ __forceinline__ void cvt(float* f) const {
    f[0] = u.x; f[1] = u.y; f[2] = u.z; f[3] = u.w;
  }
};
template <>
struct Raw<float, 2> {
  float2 u;
  __device__ __forceinline__ void load(const float* p) { u = *reinterpret_cast<const float2*>(p); }
  __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, int off) {
    const i32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    u = make_float2(__int_as_float(t.x), __int_as_float(t.y));
  }
  __device__ __forceinline__ void cvt(float* f) const { f[0] = u.x; f[1] = u.y; }
};

// Cache policy of the buffer stores: 0, or kStoreStream (non-temporal:
// the line is not kept for reuse).
constexpr int kStoreStream = 2;

template <typename T, int V, int CP = 0>
__device__ __forceinline__ void store_buf(__amdgpu_buffer_rsrc_t r, int off,
                                          const float* v) {
  if constexpr (sizeof(T) == 2 && V == 8) {
    const i32x4 d = {(int)pack_bf16x2(v[0], v[1]), (int)pack_bf16x2(v[2], v[3]),
                     (int)pack_bf16x2(v[4], v[5]), (int)pack_bf16x2(v[6], v[7])};
    __builtin_amdgcn_raw_buffer_store_b128(d, r, off, 0, CP);
  } else if constexpr (sizeof(T) == 4 && V == 8) {
    const i32x4 d0 = {__float_as_int(v[0]), __float_as_int(v[1]),
                      __float_as_int(v[2]), __float_as_int(v[3])};
    const i32x4 d1 = {__float_as_int(v[4]), __float_as_int(v[5]),
                      __float_as_int(v[6]), __float_as_int(v[7])};
    __builtin_amdgcn_raw_buffer_store_b128(d0, r, off, 0, CP);
    __builtin_amdgcn_raw_buffer_store_b128(d1, r, off + (off == kOob ? 0 : 16), 0, CP);
  } else if constexpr (sizeof(T) == 2 && V == 4) {
    const i32x2 d = {(int)pack_bf16x2(v[0], v[1]), (int)pack_bf16x2(v[2], v[3])};
    __builtin_amdgcn_raw_buffer_store_b64(d, r, off, 0, CP);
  } else if constexpr (sizeof(T) == 2 && V == 2) {
    __builtin_amdgcn_raw_buffer_store_b32((int)pack_bf16x2(v[0], v[1]), r, off, 0, CP);
  } else if constexpr (V == 4) {
    const i32x4 d = {__float_as_int(v[0]), __float_as_int(v[1]),
                     __float_as_int(v[2]), __float_as_int(v[3])};
    __builtin_amdgcn_raw_buffer_store_b128(d, r, off, 0, CP);
  } else {
    const i32x2 d = {__float_as_int(v[0]), __float_as_int(v[1])};
    __builtin_amdgcn_raw_buffer_store_b64(d, r, off, 0, CP);
  }
}

// Round v to T in place (the values as stored).
template <typename T, int V>
__device__ __forceinline__ void round_to(float* v) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < V / 2; ++i) {
      const uint32_t w = pack_bf16x2(v[2 * i], v[2 * i + 1]);
      v[2 * i] = __uint_as_float(w << 16);
      v[2 * i + 1] = __uint_as_float(w & 0xffff0000u);
    }
  }
}

// Sum over aligned groups of N (8 or 16) lanes by DPP moves (neighbour
// swap, pair swap, mirror in 8, mirror in 16); every lane of a group ends
// with the same value.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
template <int N>
__device__ __forceinline__ float sum_lanes(float v) {
  static_assert(N == 8 || N == 16, "8 or 16 lanes");
  v += dpp_mov<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  if constexpr (N == 16) v += dpp_mov<0x140>(v);  // row_mirror
  return v;
}

// End of a strip with POOL (after the barrier): the block sums parked in
// red[block row][column group][channel] leave the workgroup either whole,
// bsum[b][t][c] (gate_w == nullptr), or already reduced into the gate's
// partial logits of each 32-channel head slice (channel c = s C + 32 h + j,
// C = 32 heads):
//   plog[b][t][s][h] = sum_j gate_w[h][32 s + j] * blocksum(s C + 32 h + j),
// summed over the 32 / V lanes that hold the slice (one aligned DPP group,
// fixed order), written to bsum's memory.  A thread's CX columns lie in one
// block (block is a multiple of CX).
template <int V, int CX, int TT, int WC, int RB>
__device__ __forceinline__ void pool_store(const float (&red)[RB][TT][WC],
                                           float* bsum, const float* gate_w, int heads,
                                           int block, int b, int gh, int gw, int ch, int x,
                                           int tx, int tc, int c, bool c_ok, int y0,
                                           int y_end) {
  const int nbc = gw / block, T = (gh / block) * nbc;
  if (x % block != 0 || x >= gw) return;  // uniform over each lane group
  if (!gate_w) {
    if (!c_ok) return;
    for (int br = 0; br < (y_end - y0) / block; ++br) {
      const size_t t = (size_t)(y0 / block + br) * nbc + x / block;
      float* dst = bsum + ((size_t)b * T + t) * ch + c;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        float sm = 0.f;
        for (int q = 0; q < block / CX; ++q) sm += red[br][tx + q][tc * V + j];
        dst[j] = sm;
      }
    }
    return;
  }
  static_assert(32 % V == 0 && WC % 32 == 0, "head slices of 32 channels");
  constexpr int L = 32 / V;  // lanes per head slice
  const int C = 32 * heads;
  const int sc = c / C, h = (c % C) / 32;
  float gwt[V];
#pragma unroll
  for (int j = 0; j < V; ++j) gwt[j] = c_ok ? gate_w[h * 96 + sc * 32 + (c % 32) + j] : 0.f;
  for (int br = 0; br < (y_end - y0) / block; ++br) {
    float p = 0.f;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      float sm = 0.f;
      for (int q = 0; q < block / CX; ++q) sm += red[br][tx + q][tc * V + j];
      p = fmaf(gwt[j], sm, p);
    }
    p = sum_lanes<L>(p);
    if (tc % L == 0 && c_ok) {
      const size_t t = (size_t)(y0 / block + br) * nbc + x / block;
      bsum[(((size_t)b * T + t) * 3 + sc) * heads + h] = p;
    }
  }
}

constexpr int kStreamChannels = 64;  // channels per workgroup
// Streaming kernel (5x5, 7x7): channels and output columns per thread, rows
// of loads in flight.  Measured on the folded 5x5 (7x7) with gate sums:
// 1 column of 4 channels 116 (196) us, 2 columns 100, 4 columns of 4
// channels 97, 4 columns of 2 channels 93 (139), 8 columns about the same
// as 4 but no longer dividing 4 x 4 gate blocks; then one row of loads in
// flight instead of two 85 us (fewer registers: 5 waves per SIMD, not 4;
// three or four rows slower).
constexpr int kStreamV = 2, kStreamCols = 4, kStreamRows = 1;
// Strip heights TH, TH / 2 or TH / 4 (kMinStrip): the tallest that still
// gives kStreamMinWgs workgroups (two per CU).  Shorter strips re-read more
// halo rows and load the taps more often, so they only pay where CUs would
// idle (measured on the folded 5x5 with gate sums: 4 x 64x128 tokens at
// C = 256, 384 workgroups, 51.8 -> 45.8 us with strips of 8 rows; 8 x
// 128x128 at C = 128, 768 workgroups, 59.9 -> 70.8 us with 16 rows).
constexpr int kMinStrip = TH / 4, kStreamMinWgs = 512;
constexpr int kCus = 256;  // compute units of an MI355X
// LDS-staged kernel (up to 3x3): output columns per thread.
constexpr int kLdsCols = 2;

// Register-streaming variant (the wider kernels, whose taps take most of the
// registers).  A thread owns CX adjacent output columns x .. x + CX - 1 and
// V consecutive channels of a 32-row strip and walks down the input rows of
// the strip.  For each input row it loads the K + CX - 1 horizontal
// neighbours it needs (the reuse across neighbouring threads is served by
// the L1) and converts each once; every tap read serves the CX columns, and
// the row feeds the K partial output rows it belongs to, kept in
// registers.  NB rows of loads are in flight at any time; there is no
// barrier in the row loop, so every wave streams independently.  A
// workgroup covers 64 channels x (256 V CX / 64) columns.
// Grid: 1-D over (batch, strip, channel tile, column tile) with the column
// tile fastest, remapped so each XCD walks a contiguous run of neighbouring
// tiles (their halo columns then hit in that XCD's L2).
// With POOL the kernel also writes, for the gate, the sum over every
// block x block block of the values it stores (as stored, i.e. after
// rounding to T): bsum[b][t][c], or those sums already reduced into the
// gate's partial logits (pool_store).  Each thread adds its column's rows and
// parks the sum of each finished block row in LDS (its own slot, no
// barrier); after the strip one barrier, then the block's columns are
// added in order.  block must divide the workgroup width and the strip
// height, be a multiple of CX, and be at least kPoolMinBlock (LDS room).
template <typename T, int K, bool GELU, int V, int NB, bool POOL, bool TL, int CX = 1,
          int SH = TH>
__global__ __launch_bounds__(256) void dwconv_stream(
    const T* __restrict__ in, T* __restrict__ out,
    const float* __restrict__ weff, float* __restrict__ bsum, int block,
    int gh, int gw, int ch, int col_tiles, int ch_tiles, int strips,
    int total, int per_xcd, const float* __restrict__ gate_w, int heads, int nwhole) {
  constexpr int R = (K - 1) / 2;
  constexpr int CG = kStreamChannels / V;  // channel groups per workgroup
  constexpr int TT = 256 / CG;             // column groups per workgroup
  constexpr int TW = TT * CX;              // columns per workgroup
  constexpr int KL = K + CX - 1;           // input columns per thread
  __shared__ float red[POOL ? SH / kPoolMinBlock : 1][POOL ? TT : 1][POOL ? kStreamChannels : 1];
  // Tiles [0, nwhole) run whole, on the first per_xcd * 8 workgroups
  // (XCD-remapped); each later tile runs as two half-height strips, on one
  // workgroup each, after them (see run_dw).
  const int bid = blockIdx.x;
  int tile, y_off = 0, y_len = SH;
  if (bid < per_xcd * kXcds) {
    tile = (bid % kXcds) * per_xcd + bid / kXcds;
    if (tile >= nwhole) return;
  } else {
    const int j = bid - per_xcd * kXcds;
    tile = nwhole + j / 2;
    if (tile >= total) return;
    y_off = (j % 2) * (SH / 2);
    y_len = SH / 2;
  }
  int rest = tile;
  const int col_t = rest % col_tiles;
  rest /= col_tiles;
  const int ch_t = rest % ch_tiles;
  rest /= ch_tiles;
  const int strip = rest % strips;
  const int b = rest / strips;

  const int tc = threadIdx.x % CG;
  const int tx = threadIdx.x / CG;  // column group
  const int x = col_t * TW + tx * CX;
  const int c = ch_t * kStreamChannels + tc * V;
  const bool c_ok = c < ch;
  const int y0 = strip * SH + y_off;
  const size_t img = (size_t)b * gh * gw;

  // Taps: in registers, or (TL) in LDS, read at every use -- the lanes of
  // one channel group read the same 16 bytes (a broadcast), which frees
  // the K*K*V tap registers for more channels per thread.
  float w[TL ? 1 : K][TL ? 1 : K][V];
  __shared__ __attribute__((aligned(16))) float wl[TL ? K * K : 1][TL ? kStreamChannels : 1];
  if constexpr (TL) {
    for (int idx = threadIdx.x; idx < K * K * kStreamChannels; idx += 256) {
      const int tap = idx / kStreamChannels, cc = idx % kStreamChannels;
      const int cg = ch_t * kStreamChannels + cc;
      wl[tap][cc] = cg < ch ? weff[(size_t)tap * ch + cg] : 0.f;
    }
    __syncthreads();
  } else {
#pragma unroll
    for (int ky = 0; ky < K; ++ky)
#pragma unroll
      for (int kx = 0; kx < K; ++kx)
#pragma unroll
        for (int j = 0; j < V; ++j)
          w[ky][kx][j] = c_ok ? weff[(size_t)(ky * K + kx) * ch + c + j] : 0.f;
  }
  auto tap = [&](int ky, int kx, float (&t)[V]) {
    if constexpr (TL) {
      const float* p = &wl[ky * K + kx][tc * V];
      if constexpr (V == 4) {
        const float4 q = *reinterpret_cast<const float4*>(p);
        t[0] = q.x; t[1] = q.y; t[2] = q.z; t[3] = q.w;
      } else {
#pragma unroll
        for (int j = 0; j < V; ++j) t[j] = p[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < V; ++j) t[j] = w[ky][kx][j];
    }
  };

  float acc[K][CX][V];
#pragma unroll
  for (int i = 0; i < K; ++i)
#pragma unroll
    for (int cx = 0; cx < CX; ++cx)
#pragma unroll
      for (int j = 0; j < V; ++j) acc[i][cx][j] = 0.f;
  float psum[V];
#pragma unroll
  for (int j = 0; j < V; ++j) psum[j] = 0.f;

  const int y_end = min(gh, y0 + y_len);
  const int r_begin = y0 - R, r_end = y_end + R;

  // Row loads through a buffer resource over the workgroup's in-grid
  // columns of the row: taps outside the grid (and rows outside it) read
  // zeros, with no branch and no select.
  const int x0 = col_t * TW;
  const int lx0 = max(x0 - R, 0);
  const int row_bytes = (min(gw, x0 + TW + R) - lx0) * ch * (int)sizeof(T);
  int col_off[KL];
#pragma unroll
  for (int kx = 0; kx < KL; ++kx) {
    const int xx = x + kx - R;
    col_off[kx] = (xx >= 0 && xx < gw && c_ok) ? ((xx - lx0) * ch + c) * (int)sizeof(T)
                                               : kOob;
  }
  auto load_row = [&](Raw<T, V> (&rr)[KL], int r) {
    const bool in_grid = r >= 0 && r < gh;
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(
        in + (img + (size_t)min(max(r, 0), gh - 1) * gw + lx0) * ch,
        in_grid ? row_bytes : 0);
#pragma unroll
    for (int kx = 0; kx < KL; ++kx) rr[kx].load_buf(rs, col_off[kx]);
  };
  const int out_bytes = (min(gw, x0 + TW) - x0) * ch * (int)sizeof(T);
  int st_off[CX];
#pragma unroll
  for (int cx = 0; cx < CX; ++cx)
    st_off[cx] = (x + cx < gw && c_ok) ? ((tx * CX + cx) * ch + c) * (int)sizeof(T) : kOob;

  Raw<T, V> rbuf[NB][KL];
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
      Raw<T, V>(&cur)[KL] = rbuf[u % NB];
      // A halo row outside the grid contributes nothing: skip it (uniform),
      // but start the output row it would have started.
      if (r >= 0 && r < gh) {
        float xin[KL][V];
#pragma unroll
        for (int kx = 0; kx < KL; ++kx) cur[kx].cvt(xin[kx]);
        // input row r feeds output row r - R + i with vertical tap K - 1 - i;
        // for i = K - 1 it is that output row's first input row, whose first
        // product starts the slot (freed by the row stored just before)
#pragma unroll
        for (int i = 0; i < K; ++i) {
          const int slot = (u - R + i + NB * K) % K;
#pragma unroll
          for (int kx = 0; kx < K; ++kx) {
            float t[V];
            tap(K - 1 - i, kx, t);
#pragma unroll
            for (int cx = 0; cx < CX; ++cx)
#pragma unroll
              for (int j = 0; j < V; ++j)
                acc[slot][cx][j] = (i == K - 1 && kx == 0)
                                       ? t[j] * xin[cx + kx][j]
                                       : fmaf(t[j], xin[cx + kx][j], acc[slot][cx][j]);
          }
        }
      } else {
        const int slot = (u - R + K - 1 + NB * K) % K;
#pragma unroll
        for (int cx = 0; cx < CX; ++cx)
#pragma unroll
          for (int j = 0; j < V; ++j) acc[slot][cx][j] = 0.f;
      }
      // unconditional (clamped) prefetch keeps the load/wait pattern regular
      load_row(cur, r + NB);
      const int done = (u - R + NB * K) % K;  // slot of output row r - R
      const int yo = r - R;
      const bool row_out = yo >= y0 && yo < y_end;  // uniform
      {
        const __amdgpu_buffer_rsrc_t rs = buf_rsrc(
            out + (img + (size_t)min(max(yo, 0), gh - 1) * gw + x0) * ch,
            row_out ? out_bytes : 0);
#pragma unroll
        for (int cx = 0; cx < CX; ++cx) {
          float v[V];
#pragma unroll
          for (int j = 0; j < V; ++j)
            v[j] = GELU ? gelu_erf(acc[done][cx][j]) : acc[done][cx][j];
          // streamed past the caches (measured: 124 -> 114 us on the folded
          // 5x5, its readers no slower)
          store_buf<T, V, kStoreStream>(rs, st_off[cx], v);
          // lanes outside the grid add values that the block reduction never
          // reads (it reads in-grid blocks only); rows outside the strip
          // are skipped (uniform)
          if (POOL && row_out) {
            round_to<T, V>(v);
#pragma unroll
            for (int j = 0; j < V; ++j) psum[j] += v[j];
          }
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
    }
  }
  if constexpr (POOL) {
    __syncthreads();
    pool_store<V, CX, TT, kStreamChannels>(red, bsum, gate_w, heads, block, b, gh, gw, ch, x,
                                           tx, tc, c, c_ok, y0, y_end);
  }
}

// LDS-staged variant.  The workgroup (TW columns x 64 channels of a TH-row
// strip, as above) loads each input row once, TW + 2R columns wide, with
// 16-byte loads spread over all 256 threads (at most a few chunks each), and
// keeps P rows of those loads in flight in registers.  Rows pass through
// two LDS slots; one barrier per row orders "row r written" before "row r
// read" and "row r - 1 read" before "slot reused".  Each thread then reads
// the K + CX - 1 horizontal neighbours of its CX columns from LDS instead
// of from L1, and accumulates as above (K partial output rows in
// registers).  Compared with the
// register-only kernel the bytes in flight per workgroup no longer scale
// with the per-thread tap registers.
// BO > 0: out is written tile-blocked for the GEMM (token m of the launch,
// channel k at ((m / 256) * (ch / 32) + k / 32) * 8192 + (m % 256) * 32 +
// k % 32); out_bytes_all is then the whole output's size in bytes.  BO = 2
// when gw is a multiple of 256: grid row yo is then whole tiles, one
// contiguous gw * ch run, so the offset within the row is fixed per thread
// and the row is a scalar base.
// PIN: in is channel-planar (64-channel planes, element (m, c) of the
// launch's tokens at (c / 64) * tokens * 64 + m * 64 + c % 64; WC = 64):
// a staged row is then one contiguous run of the workgroup's plane.
template <typename T, int K, bool GELU, int V, int P, bool POOL, int WC, int BO,
          int CX = 1, bool PIN = false>
__global__ __launch_bounds__(256) void dwconv_lds(
    const T* __restrict__ in, T* __restrict__ out,
    const float* __restrict__ weff, float* __restrict__ bsum, int block,
    int gh, int gw, int ch, int col_tiles, int ch_tiles, int strips,
    int total, int per_xcd, int out_bytes_all, const float* __restrict__ gate_w,
    int heads) {
  constexpr int R = (K - 1) / 2;
  constexpr int CG = WC / V;  // channel groups per workgroup
  constexpr int TT = 256 / CG;         // column groups per workgroup
  constexpr int TW = TT * CX;          // columns per workgroup
  constexpr int KL = K + CX - 1;       // input columns per thread
  constexpr int LC = TW + 2 * R;       // columns per staged row
  constexpr int EPC = 16 / (int)sizeof(T);       // elements per 16-byte chunk
  constexpr int CPC = WC / EPC;         // chunks per column
  constexpr int CHUNKS = LC * CPC;               // chunks per row
  constexpr int LPT = (CHUNKS + 255) / 256;      // chunks per thread
  constexpr int SLOT = LPT * 256 * 16;           // bytes per LDS row slot
  constexpr int CB = WC * (int)sizeof(T);  // bytes per staged column
  // group of rows after which every register index repeats
  constexpr int G = (K % P == 0) ? K : (P % K == 0 ? P : K * P);
  __shared__ __attribute__((aligned(16))) char ring[2 * SLOT];
  __shared__ float red[POOL ? TH / kPoolMinBlock : 1][POOL ? TT : 1][POOL ? WC : 1];
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

  const int tid = threadIdx.x;
  const int tc = tid % CG;
  const int tx = tid / CG;
  const int x0 = col_t * TW;
  const int x = x0 + tx * CX;
  const int c0 = ch_t * WC;
  const int c = c0 + tc * V;
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

  // This thread's chunks of a staged row: byte offset from the row's first
  // in-grid staged column, or kOob for chunks outside the grid (read as 0).
  const int lx0 = max(x0 - R, 0);
  const int lx1 = min(gw, x0 + TW + R);
  // column stride of the input (elements), its channel base
  static_assert(!PIN || WC == 64, "64-channel planes");
  const int cs = PIN ? WC : ch;
  const int cb = PIN ? c0 : 0;
  const T* inb = in;
  if constexpr (PIN) {
    const int batch = total / (col_tiles * ch_tiles * strips);
    inb = in + (size_t)ch_t * ((size_t)batch * gh * gw * WC);
  }
  const int row_bytes = (lx1 - lx0) * cs * (int)sizeof(T);
  int ld_off[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int q = tid + 256 * i;
    const int col = q / CPC, part = q % CPC;
    const int xg = x0 - R + col;
    const int cg = c0 + part * EPC;
    const bool ok = q < CHUNKS && xg >= 0 && xg < gw && cg < ch;
    ld_off[i] = ok ? ((xg - lx0) * cs + cg - cb) * (int)sizeof(T) : kOob;
  }
  auto load_row = [&](uint4 (&d)[LPT], int r) {
    const bool in_grid = r >= 0 && r < gh;
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(
        inb + (img + (size_t)min(max(r, 0), gh - 1) * gw + lx0) * cs,
        in_grid ? row_bytes : 0);
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const i32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rs, ld_off[i], 0, 0);
      d[i] = uint4{(uint32_t)t.x, (uint32_t)t.y, (uint32_t)t.z, (uint32_t)t.w};
    }
  };
  // every thread writes (chunks past the row land in the slot's spare room)
  auto store_row = [&](const uint4 (&d)[LPT], int slot) {
#pragma unroll
    for (int i = 0; i < LPT; ++i)
      *reinterpret_cast<uint4*>(ring + slot * SLOT + (tid + 256 * i) * 16) = d[i];
  };
  // output: this thread's byte offset within its output row segment
  const int ox1 = min(gw, x0 + TW);
  const int out_bytes = (ox1 - x0) * ch * (int)sizeof(T);
  int st_off[CX];
#pragma unroll
  for (int cx = 0; cx < CX; ++cx) {
    const int xc = x + cx;
    const bool ok = xc < gw && c_ok;
    if (BO == 2)
      st_off[cx] = ok
                       ? (((xc / kGemmTileM) * (ch / kGemmTileK) + c / kGemmTileK) *
                              (kGemmTileM * kGemmTileK) +
                          (xc % kGemmTileM) * kGemmTileK + c % kGemmTileK) *
                             (int)sizeof(T)
                       : kOob;
    else
      st_off[cx] = ok ? ((tx * CX + cx) * ch + c) * (int)sizeof(T) : kOob;
  }

  float acc[K][CX][V];
#pragma unroll
  for (int i = 0; i < K; ++i)
#pragma unroll
    for (int cx = 0; cx < CX; ++cx)
#pragma unroll
      for (int j = 0; j < V; ++j) acc[i][cx][j] = 0.f;
  float psum[V];
#pragma unroll
  for (int j = 0; j < V; ++j) psum[j] = 0.f;

  const int y_end = min(gh, y0 + TH);
  const int r_begin = y0 - R;
  const int nrows = y_end + R - r_begin;

  uint4 pre[P][LPT];
#pragma unroll
  for (int q = 0; q < P; ++q) load_row(pre[q], r_begin + q);
  store_row(pre[0], 0);
  load_row(pre[0], r_begin + P);
  const char* my = ring + tx * CX * CB + tc * V * (int)sizeof(T);
  for (int u0 = 0; u0 < nrows; u0 += G) {
#pragma unroll
    for (int v = 0; v < G; ++v) {
      const int u = u0 + v;
      if (u >= nrows) break;
      const int r = r_begin + u;
      __syncthreads();
      {
        // rows outside the grid were staged as zeros (empty resource)
        float xin[KL][V];
#pragma unroll
        for (int kx = 0; kx < KL; ++kx) {
          Raw<T, V> rr;
          rr.load(reinterpret_cast<const T*>(my + (u & 1) * SLOT + kx * CB));
          rr.cvt(xin[kx]);
        }
        // input row r feeds output row r - R + i with vertical tap K - 1 - i;
        // for i = K - 1 it is that output row's first input row, whose first
        // product starts the slot (freed by the row stored just before)
#pragma unroll
        for (int i = 0; i < K; ++i) {
          const int slot = (v - R + i + G) % K;
#pragma unroll
          for (int kx = 0; kx < K; ++kx)
#pragma unroll
            for (int cx = 0; cx < CX; ++cx)
#pragma unroll
              for (int j = 0; j < V; ++j)
                acc[slot][cx][j] = (i == K - 1 && kx == 0)
                                       ? w[K - 1 - i][kx][j] * xin[cx + kx][j]
                                       : fmaf(w[K - 1 - i][kx][j], xin[cx + kx][j],
                                              acc[slot][cx][j]);
        }
      }
      // stage row r + 1 (its loads were issued P - 1 rows ago) and issue
      // the loads of row r + 1 + P
      store_row(pre[(v + 1) % P], (u + 1) & 1);
      load_row(pre[(v + 1) % P], r + 1 + P);
      const int done = (v - R + G) % K;  // slot of output row r - R
      const int yo = r - R;
      const bool row_out = yo >= y0 && yo < y_end;  // uniform
#pragma unroll
      for (int cx = 0; cx < CX; ++cx) {
        float o[V];
#pragma unroll
        for (int j = 0; j < V; ++j)
          o[j] = GELU ? gelu_erf(acc[done][cx][j]) : acc[done][cx][j];
        if constexpr (BO == 2) {
          const __amdgpu_buffer_rsrc_t rs = buf_rsrc(
              out + (img + (size_t)min(max(yo, 0), gh - 1) * gw) * ch,
              row_out ? gw * ch * (int)sizeof(T) : 0);
          store_buf<T, V>(rs, st_off[cx], o);
        } else if constexpr (BO == 1) {
          const int m = (b * gh + yo) * gw + x + cx;
          const int off =
              (row_out && x + cx < gw && c_ok)
                  ? (((m / kGemmTileM) * (ch / kGemmTileK) + c / kGemmTileK) *
                         (kGemmTileM * kGemmTileK) +
                     (m % kGemmTileM) * kGemmTileK + c % kGemmTileK) *
                        (int)sizeof(T)
                  : kOob;
          store_buf<T, V>(buf_rsrc(out, out_bytes_all), off, o);
        } else {
          const __amdgpu_buffer_rsrc_t rs = buf_rsrc(
              out + (img + (size_t)min(max(yo, 0), gh - 1) * gw + x0) * ch,
              row_out ? out_bytes : 0);
          store_buf<T, V>(rs, st_off[cx], o);
        }
        // lanes outside the grid add values that the block reduction never
        // reads; rows outside the strip are skipped (uniform)
        if (POOL && row_out) {
          round_to<T, V>(o);
#pragma unroll
          for (int j = 0; j < V; ++j) psum[j] += o[j];
        }
      }
      if constexpr (POOL) {
        if (yo >= y0 && yo < y_end && (yo + 1) % block == 0) {
          const int br = (yo - y0) / block;
#pragma unroll
          for (int j = 0; j < V; ++j) {
            red[br][tx][tc * V + j] = psum[j];
            psum[j] = 0.f;
          }
        }
      }
    }
  }
  if constexpr (POOL) {
    __syncthreads();
    pool_store<V, CX, TT, WC>(red, bsum, gate_w, heads, block, b, gh, gw, ch, x, tx, tc, c,
                              c_ok, y0, y_end);
  }
}

// Per kernel size: channels per thread V, rows of loads in flight P,
// channels per workgroup WC and output columns per thread CX (the
// workgroup is 256 CX / (WC / V) columns wide).  Sizes up to 3 take the
// LDS-staged kernel, 5 and 7 the streaming one with the taps in LDS (the
// LDS-staged kernel measured 130-170 us on the folded 5x5 in every shape
// tried, against the figures given with kStreamV).
struct DwCfg {
  int v, p, wc;
  bool tl;  // streaming kernel: taps in LDS
  int cx;   // streaming kernel: output columns per thread
};
constexpr DwCfg dw_cfg(int k, bool gelu) {
  return k <= 3 ? DwCfg{4, 3, 64, false, kLdsCols}
                : DwCfg{kStreamV, kStreamRows, kStreamChannels, true, kStreamCols};
  (void)gelu;
}
constexpr int dw_width(int k, bool gelu) {
  return 256 / (dw_cfg(k, gelu).wc / dw_cfg(k, gelu).v) * dw_cfg(k, gelu).cx;
}

template <typename T, int K, bool GELU>
hipError_t run_dw_lds(const void* in, void* out, const float* weff, float* bsum,
                      int block, int batch, int gh, int gw, int ch, bool out_blocked,
                      hipStream_t s, const float* gate_w, int heads, int col_tiles,
                      int ch_tiles, int strips, int total, int per_xcd);

template <typename T, int K, bool GELU>
hipError_t run_dw(const void* in, void* out, const float* weff, float* bsum,
                  int block, int batch, int gh, int gw, int ch, bool out_blocked,
                  hipStream_t s, const float* gate_w, int heads) {
  constexpr DwCfg cf = dw_cfg(K, GELU);
  constexpr int TW = dw_width(K, GELU);
  const int col_tiles = (gw + TW - 1) / TW;
  const int ch_tiles = (ch + cf.wc - 1) / cf.wc;
  const int strips = (gh + TH - 1) / TH;
  const int total = col_tiles * ch_tiles * strips * batch;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  if constexpr (K >= 5) {
    // Shorter strips where TH-row strips give too few workgroups to fill
    // the chip (each output is summed in the same order whatever the
    // strip, and pooled block rows stay inside one strip).
    int sh = TH;
    while (sh > kMinStrip && (sh / 2) % (bsum ? block : 1) == 0 &&
           col_tiles * ch_tiles * ((gh + sh - 1) / sh) * batch < kStreamMinWgs)
      sh /= 2;
    auto go = [&](auto sh_c) {
      constexpr int SH = decltype(sh_c)::value;
      const int st = (gh + SH - 1) / SH;
      const int tot = col_tiles * ch_tiles * st * batch;
      // The conv is bound by VALU issue and every workgroup of a launch is
      // resident at once (five per CU), so a CU's time is its workgroups'
      // total work.  Where the tiles are a whole number of workgroups per
      // CU plus at most half a round (the block's 1152 on 256 CUs: half
      // the CUs would run five, half four), the remainder tiles run as two
      // half-height strips each, one more per CU: every CU then runs four
      // whole tiles and one half.  Outputs are summed in the same order
      // whatever the strip, and pooled block rows stay inside a half strip.
      const int rem = tot % kCus;
      const bool halves = rem > 0 && 2 * rem <= kCus && (SH / 2) % (bsum ? block : 1) == 0 &&
                          SH / 2 >= kMinStrip;
      const int nwhole = halves ? tot - rem : tot;
      const int px = (nwhole + kXcds - 1) / kXcds;
      const int grid = px * kXcds + 2 * (tot - nwhole);
      if (bsum && !GELU)
        dwconv_stream<T, K, false, cf.v, cf.p, true, cf.tl, cf.cx, SH><<<grid, 256, 0, s>>>(
            static_cast<const T*>(in), static_cast<T*>(out), weff, bsum, block, gh,
            gw, ch, col_tiles, ch_tiles, st, tot, px, gate_w, heads, nwhole);
      else
        dwconv_stream<T, K, GELU, cf.v, cf.p, false, cf.tl, cf.cx, SH><<<grid, 256, 0, s>>>(
            static_cast<const T*>(in), static_cast<T*>(out), weff, nullptr, 1, gh,
            gw, ch, col_tiles, ch_tiles, st, tot, px, nullptr, 0, nwhole);
    };
    if (sh == TH)
      go(std::integral_constant<int, TH>{});
    else if (sh == TH / 2)
      go(std::integral_constant<int, TH / 2>{});
    else
      go(std::integral_constant<int, TH / 4>{});
    return hipGetLastError();
  } else {
    return run_dw_lds<T, K, GELU>(in, out, weff, bsum, block, batch, gh, gw, ch, out_blocked,
                                  s, gate_w, heads, col_tiles, ch_tiles, strips, total, per_xcd);
  }
}

template <typename T, int K, bool GELU>
hipError_t run_dw_lds(const void* in, void* out, const float* weff, float* bsum,
                      int block, int batch, int gh, int gw, int ch, bool out_blocked,
                      hipStream_t s, const float* gate_w, int heads, int col_tiles,
                      int ch_tiles, int strips, int total, int per_xcd) {
  constexpr DwCfg cf = dw_cfg(K, GELU);
  if constexpr (!GELU) {
    if (bsum) {
      dwconv_lds<T, K, false, cf.v, cf.p, true, cf.wc, 0, cf.cx><<<per_xcd * kXcds, 256, 0, s>>>(
          static_cast<const T*>(in), static_cast<T*>(out), weff, bsum, block, gh,
          gw, ch, col_tiles, ch_tiles, strips, total, per_xcd, 0, gate_w, heads);
      return hipGetLastError();
    }
  }
  if (out_blocked && gw % kGemmTileM == 0)
    dwconv_lds<T, K, GELU, cf.v, cf.p, false, cf.wc, 2, cf.cx><<<per_xcd * kXcds, 256, 0, s>>>(
        static_cast<const T*>(in), static_cast<T*>(out), weff, nullptr, 1, gh,
        gw, ch, col_tiles, ch_tiles, strips, total, per_xcd,
        (int)((size_t)batch * gh * gw * ch * sizeof(T)), nullptr, 0);
  else if (out_blocked)
    dwconv_lds<T, K, GELU, cf.v, cf.p, false, cf.wc, 1, cf.cx><<<per_xcd * kXcds, 256, 0, s>>>(
        static_cast<const T*>(in), static_cast<T*>(out), weff, nullptr, 1, gh,
        gw, ch, col_tiles, ch_tiles, strips, total, per_xcd,
        (int)((size_t)batch * gh * gw * ch * sizeof(T)), nullptr, 0);
  else
    dwconv_lds<T, K, GELU, cf.v, cf.p, false, cf.wc, 0, cf.cx><<<per_xcd * kXcds, 256, 0, s>>>(
        static_cast<const T*>(in), static_cast<T*>(out), weff, nullptr, 1, gh,
        gw, ch, col_tiles, ch_tiles, strips, total, per_xcd, 0, nullptr, 0);
  return hipGetLastError();
}

template <typename T, bool GELU>
hipError_t dispatch_k(int kmax, const void* in, void* out, const float* weff,
                      float* bsum, int block, int batch, int gh, int gw, int ch,
                      bool out_blocked, hipStream_t s, const float* gate_w, int heads) {
  switch (kmax) {
    case 1: return run_dw<T, 1, GELU>(in, out, weff, bsum, block, batch, gh, gw, ch, out_blocked, s, gate_w, heads);
    case 3: return run_dw<T, 3, GELU>(in, out, weff, bsum, block, batch, gh, gw, ch, out_blocked, s, gate_w, heads);
    case 5: return run_dw<T, 5, GELU>(in, out, weff, bsum, block, batch, gh, gw, ch, out_blocked, s, gate_w, heads);
    case 7: return run_dw<T, 7, GELU>(in, out, weff, bsum, block, batch, gh, gw, ch, out_blocked, s, gate_w, heads);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool dwconv_planar_ok(bool bf, int batch, int gh, int gw, int ch) {
  return dwconv_can_block_out(bf, 3, true, batch, gh, gw, ch) && gw % kGemmTileM == 0 &&
         ch % 64 == 0 && dw_cfg(3, true).wc == 64;
}

hipError_t launch_dwconv_gelu_planar(const void* in, void* out, const float* weff, int batch,
                                     int gh, int gw, int ch, hipStream_t s) {
  if (!dwconv_planar_ok(true, batch, gh, gw, ch)) return hipErrorInvalidValue;
  constexpr DwCfg cf = dw_cfg(3, true);
  // each staged row is one contiguous run here: two rows of loads in
  // flight measured 1.5-2 us faster than three (which the row-major input
  // needs).  Four output columns per thread (64-column tiles): each staged
  // row serves twice the outputs per LDS read and the horizontal halo is
  // half as wide (measured on the block's hidden tensor, 2 x 128x256 tokens
  // x 1536 channels: 91.7 -> 87.0 us; 64-row strips 91.9 with two columns
  // and 108 with four, where 384 workgroups leave CUs idle).
  constexpr int kPlanarRows = 2, kPlanarCols = 4;
  constexpr int TW = 256 / (cf.wc / cf.v) * kPlanarCols;
  const int col_tiles = (gw + TW - 1) / TW;
  const int ch_tiles = ch / cf.wc;
  const int strips = (gh + TH - 1) / TH;
  const int total = col_tiles * ch_tiles * strips * batch;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  dwconv_lds<bf16, 3, true, cf.v, kPlanarRows, false, cf.wc, 2, kPlanarCols, true>
      <<<per_xcd * kXcds, 256, 0, s>>>(
          static_cast<const bf16*>(in), static_cast<bf16*>(out), weff, nullptr, 1, gh, gw, ch,
          col_tiles, ch_tiles, strips, total, per_xcd,
          (int)((size_t)batch * gh * gw * ch * sizeof(bf16)), nullptr, 0);
  return hipGetLastError();
}

bool dwconv_can_pool(int kmax, int block) {
  const int tw = dw_width(kmax, false);
  return block >= kPoolMinBlock && tw % block == 0 && TH % block == 0 &&
         block % dw_cfg(kmax, false).cx == 0;
}

bool dwconv_can_block_out(bool bf, int kmax, bool gelu, int batch, int gh, int gw,
                          int ch) {
  const size_t tokens = (size_t)batch * gh * gw;
  return bf && gelu && kmax <= 3 && tokens % kGemmTileM == 0 && ch % kGemmTileK == 0 &&
         tokens * ch * 2 < ((size_t)1 << 31);
}

hipError_t launch_dwconv(bool bf, const void* in, void* out, const float* weff,
                         int kmax, int batch, int gh, int gw, int ch,
                         bool gelu, float* bsum, int block, hipStream_t s,
                         bool out_blocked, const float* gate_w, int heads) {
  if (bsum && (gelu || !dwconv_can_pool(kmax, block))) return hipErrorInvalidValue;
  if (gate_w && (!bsum || heads <= 0 || ch != 3 * 32 * heads)) return hipErrorInvalidValue;
  if (out_blocked && !dwconv_can_block_out(bf, kmax, gelu, batch, gh, gw, ch))
    return hipErrorInvalidValue;
  if (bf)
    return gelu ? dispatch_k<bf16, true>(kmax, in, out, weff, nullptr, 1, batch, gh, gw, ch,
                                         out_blocked, s, nullptr, 0)
                : dispatch_k<bf16, false>(kmax, in, out, weff, bsum, block, batch, gh, gw,
                                          ch, false, s, gate_w, heads);
  return gelu ? dispatch_k<float, true>(kmax, in, out, weff, nullptr, 1, batch, gh, gw, ch,
                                        false, s, nullptr, 0)
              : dispatch_k<float, false>(kmax, in, out, weff, bsum, block, batch, gh, gw, ch,
                                         false, s, gate_w, heads);
}

}  // namespace hsmla
