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

// grid (batch * heads, ceil(kPart / 64)), 64 threads: one entry per thread,
// chunk partials added in chunk order.
__global__ __launch_bounds__(64) void kv_combine_kernel(
    const float* __restrict__ part, float* __restrict__ kv,
    float* __restrict__ ksum, int nchunks) {
  const int bh = blockIdx.x;
  const float* p = part + (size_t)bh * nchunks * kPart;
  const int e = blockIdx.y * 64 + threadIdx.x;
  if (e < kPart) {
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

// ---------------------------------------------------------------------------
// bfloat16 MFMA kernels.  A workgroup covers a group of 4 heads (one wave per
// head), so every token contributes 256 contiguous bytes per tensor.
// ---------------------------------------------------------------------------

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kHG = 4;          // heads per workgroup
constexpr int kTT = 32;         // tokens per LDS tile
constexpr int kTS = kTT + 8;    // bf16 stride of channel-major rows
constexpr int kChunkTok = 512;  // tokens per partial (bf16 path)

__device__ __forceinline__ uint16_t relu_bits(uint16_t u) {
  return (u & 0x8000u) ? 0 : u;
}

// Z^T tile per head: lane holds Z[i][c] for column c = lane % 32 and rows
// i = 8(r/4) + 4g + r%4; the token contraction runs through LDS copies of
// relu(K^) and V^ stored [channel][token].
// grid (chunks, ceil(heads/4), batch), 256 threads.
__global__ __launch_bounds__(256) void kv_partial_mfma(
    const bf16* __restrict__ qkvh, float* __restrict__ part, int tokens,
    int heads, int nchunks) {
  __shared__ __attribute__((aligned(16))) bf16 kt[kHG * kD * kTS];
  __shared__ __attribute__((aligned(16))) bf16 vt[kHG * kD * kTS];
  __shared__ float dsum[kHG][kD];
  __shared__ float dpart[256][8];
  const int chunk = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
  const int C = heads * kD, C3 = 3 * C;
  const int h0 = hg * kHG;
  const int nh = min(kHG, heads - h0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5;
  const int n_begin = chunk * kChunkTok;
  const int n_end = min(tokens, n_begin + kChunkTok);
  const bf16* base = qkvh + (size_t)b * tokens * C3;

  // loader: 32 tokens x 4 heads x 4 chunks of 8 channels x 2 tensors
  // = 1024 chunks; thread -> 4 of them.  chunk id: tensor | token | head | cg
  uint4 stg[4];
  float dacc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) dacc[j] = 0.f;
  auto issue = [&](int n0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cidx = tid + 256 * i;
      const int tensor = cidx >> 9, tok = (cidx >> 4) & 31;
      const int hh = (cidx >> 2) & 3, cg = cidx & 3;
      const int n = n0 + tok;
      uint4 u = {0, 0, 0, 0};
      if (n < n_end && hh < nh)
        u = *reinterpret_cast<const uint4*>(base + (size_t)n * C3 + (1 + tensor) * C +
                                            (h0 + hh) * kD + 8 * cg);
      stg[i] = u;
    }
  };
  auto commit = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cidx = tid + 256 * i;
      const int tensor = cidx >> 9, tok = (cidx >> 4) & 31;
      const int hh = (cidx >> 2) & 3, cg = cidx & 3;
      uint16_t* hv = reinterpret_cast<uint16_t*>(&stg[i]);
      bf16* dst = tensor == 0 ? kt : vt;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint16_t v = hv[j];
        if (tensor == 0) {
          v = relu_bits(v);
          dacc[j] += __uint_as_float((uint32_t)v << 16);
        }
        dst[((hh * kD) + 8 * cg + j) * kTS + tok].u = v;
      }
    }
  };

  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const bf16* ka = kt + wave * kD * kTS;
  const bf16* va = vt + wave * kD * kTS;
  if (n_begin < n_end) issue(n_begin);
  for (int n0 = n_begin; n0 < n_end; n0 += kTT) {
    commit();
    __syncthreads();
    if (n0 + kTT < n_end) issue(n0 + kTT);
#pragma unroll
    for (int ks = 0; ks < kTT / 16; ++ks) {
      const bf16x8 a = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(&ka[(lane & 31) * kTS + 16 * ks + 8 * g]));
      const bf16x8 v = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(&va[(lane & 31) * kTS + 16 * ks + 8 * g]));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, v, acc, 0, 0, 0);
    }
    __syncthreads();
  }
  // D: thread t summed channels 8cg..8cg+7 of head hh for its tokens, where
  // (hh, cg) = ((t >> 2) & 3, t & 3); the 16 threads sharing t & 15 are
  // added in thread order.
#pragma unroll
  for (int j = 0; j < 8; ++j) dpart[tid][j] = dacc[j];
  __syncthreads();
  if (tid < kHG * kD) {
    const int hh = tid / kD, ch = tid % kD, cg = ch / 8, j = ch % 8;
    float sum = 0.f;
    for (int t2 = hh * 4 + cg; t2 < 256; t2 += 16) sum += dpart[t2][j];
    dsum[hh][ch] = sum;
  }
  __syncthreads();
  if (wave < nh) {
    float* out = part + ((size_t)(b * heads + h0 + wave) * nchunks + chunk) * kPart;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 8 * (r >> 2) + 4 * g + (r & 3);
      out[i * kD + (lane & 31)] = acc[r];
    }
    if (lane < kD) out[kD * kD + lane] = dsum[wave][lane];
  }
}

// O^T = Z^T relu(Q^)^T with Z split into bf16 hi + lo parts, normalised by
// relu(q^) . D.  grid (ceil(tokens/64), ceil(heads/4), batch), 256 threads;
// wave = head, two 32-token tiles per wave.
__global__ __launch_bounds__(256) void lin_apply_mfma(
    const bf16* __restrict__ qkvh, const float* __restrict__ kv,
    const float* __restrict__ ksum, bf16* __restrict__ o, int tokens,
    int heads) {
  const int hg = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = hg * kHG + wave;
  if (h >= heads) return;
  const int C = heads * kD, C3 = 3 * C;
  const int g = lane >> 5, col = lane & 31;
  const size_t bh = (size_t)b * heads + h;
  const float* Z = kv + bh * kD * kD;
  const float* Dv = ksum + bh * kD;

  // A operand (Z^T): row c = col, k = i = 16 ks + 8 g + e
  bf16x8 zhi[2], zlo[2];
  float dreg[2][8];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int i0 = 16 * ks + 8 * g + e;
      const float z0 = Z[i0 * kD + col], z1 = Z[(i0 + 1) * kD + col];
      const bf16 h0 = from_f32<bf16>(z0), h1 = from_f32<bf16>(z1);
      const bf16 l0 = from_f32<bf16>(z0 - to_f32(h0));
      const bf16 l1 = from_f32<bf16>(z1 - to_f32(h1));
      hw[e / 2] = (uint32_t)h0.u | ((uint32_t)h1.u << 16);
      lw[e / 2] = (uint32_t)l0.u | ((uint32_t)l1.u << 16);
      dreg[ks][e] = Dv[i0];
      dreg[ks][e + 1] = Dv[i0 + 1];
    }
    zhi[ks] = __builtin_bit_cast(bf16x8, uint4{hw[0], hw[1], hw[2], hw[3]});
    zlo[ks] = __builtin_bit_cast(bf16x8, uint4{lw[0], lw[1], lw[2], lw[3]});
  }

  for (int tt = 0; tt < 2; ++tt) {
    const int n = blockIdx.x * 64 + tt * 32 + col;
    const bool ok = n < tokens;
    const bf16* qrow = qkvh + ((size_t)b * tokens + (ok ? n : 0)) * C3 + h * kD;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    float den = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 u = ok ? *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * g)
                   : uint4{0, 0, 0, 0};
      uint16_t* hv = reinterpret_cast<uint16_t*>(&u);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hv[e] = relu_bits(hv[e]);
        den = fmaf(__uint_as_float((uint32_t)hv[e] << 16), dreg[ks][e], den);
      }
      const bf16x8 qb = __builtin_bit_cast(bf16x8, u);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(zhi[ks], qb, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(zlo[ks], qb, acc, 0, 0, 0);
    }
    den += __shfl_xor(den, 32, 64);
    if (!ok) continue;
    const float inv = den > 0.f ? 1.f / den : 0.f;
    bf16* orow = o + ((size_t)b * tokens + n) * C + h * kD;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 8 * j + 4 * g;
      uint2 w;
      w.x = pack_bf16x2(acc[4 * j + 0] * inv, acc[4 * j + 1] * inv);
      w.y = pack_bf16x2(acc[4 * j + 2] * inv, acc[4 * j + 3] * inv);
      *reinterpret_cast<uint2*>(orow + c) = w;
    }
  }
}

}  // namespace

int kv_chunks(bool bf, int batch, int heads, int tokens) {
  if (bf) return (tokens + kChunkTok - 1) / kChunkTok;
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
  const int chunks = kv_chunks(bf, batch, heads, tokens);
  if (bf) {
    dim3 grid(chunks, (heads + kHG - 1) / kHG, batch);
    kv_partial_mfma<<<grid, 256, 0, s>>>(static_cast<const bf16*>(qkv_hat),
                                         partials, tokens, heads, chunks);
  } else {
    const int chunk_len = (tokens + chunks - 1) / chunks;
    dim3 grid(chunks, heads, batch);
    kv_partial_kernel<float><<<grid, 256, 0, s>>>(
        static_cast<const float*>(qkv_hat), partials, tokens, heads, chunk_len);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 cgrid(batch * heads, (kPart + 63) / 64);
  kv_combine_kernel<<<cgrid, 64, 0, s>>>(partials, kv, ksum, chunks);
  return hipGetLastError();
}

hipError_t launch_lin_apply(bool bf, const void* qkv_hat, const float* kv,
                            const float* ksum, void* o, int batch, int tokens,
                            int heads, hipStream_t s) {
  if (bf) {
    dim3 grid((tokens + 63) / 64, (heads + kHG - 1) / kHG, batch);
    lin_apply_mfma<<<grid, 256, 0, s>>>(static_cast<const bf16*>(qkv_hat), kv,
                                        ksum, static_cast<bf16*>(o), tokens, heads);
    return hipGetLastError();
  }
  dim3 grid((tokens + 63) / 64, heads, batch);
    lin_apply_kernel<float><<<grid, 64, 0, s>>>(static_cast<const float*>(qkv_hat),
                                                kv, ksum, static_cast<float*>(o),
                                                tokens, heads);
  return hipGetLastError();
}

}  // namespace hsmla
