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
    // loads issued 32 at a time, added strictly in chunk order
    float s = 0.f;
    int c = 0;
    for (; c + 32 <= nchunks; c += 32) {
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = p[(size_t)(c + i) * kPart + e];
#pragma unroll
      for (int i = 0; i < 32; ++i) s += v[i];
    }
    for (; c < nchunks; ++c) s += p[(size_t)c * kPart + e];
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
constexpr int kTT = 32;         // tokens per tile
constexpr int kChunkTok = 512;  // tokens per partial (bf16 path)
constexpr int kApplyTok = 256;  // tokens per wave in the readout

__device__ __forceinline__ uint16_t relu_bits(uint16_t u) {
  return (u & 0x8000u) ? 0 : u;
}

// One wave per head of a 4-head group, tiles of 32 tokens.  Each tile's
// K^ and V^ rows (32 tokens x 4 heads x 64 bytes each) are loaded with
// 16-byte loads over whole 256-byte rows into one of two LDS buffers (one
// barrier per tile), then every wave reads its head in token-major form
// (lane = token, 8 consecutive features per 16 bytes), which is the MFMA
// A-operand layout; multiplying it by the 32x32 identity returns it in the
// accumulator layout, where a lane owns one feature and 16 tokens -- i.e.
// transposed, exactly (one nonzero product per output).  The transposed
// relu(K^) and V^ tiles then feed Z += relu(K^)^T V^ with the token order
// the accumulator already has.  Tokens past the chunk read zeros (which add
// nothing) through per-tile buffer resources.
// grid (chunks, ceil(heads/4), batch), 256 threads = 4 heads.
constexpr int kKvRowB = 2 * kHG * kD * 2 + 16;  // LDS bytes per token row: K^ | V^

__global__ __launch_bounds__(256) void kv_partial_mfma(
    const bf16* __restrict__ qkvh, float* __restrict__ part, int tokens,
    int heads, int nchunks) {
  __shared__ __attribute__((aligned(16))) char ts[2][kTT * kKvRowB];
  const int chunk = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = hg * kHG + wave;  // h >= heads: stages, computes nothing kept
  const int C = heads * kD, C3 = 3 * C;
  const int g = lane >> 5, col = lane & 31;
  const int n_begin = chunk * kChunkTok;
  const int n_end = min(tokens, n_begin + kChunkTok);
  const int gch = min(kHG * kD, C - hg * kHG * kD);  // channels of this group

  // identity as the B operand: column col, k = 16 ks + 8 g + e
  bf16x8 eye[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    uint16_t e16[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) e16[e] = (16 * ks + 8 * g + e == col) ? 0x3f80 : 0;
    eye[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(e16));
  }

  // thread's four 16-byte chunks of a tile: token tid / 16 (+ 16),
  // part tid % 16 of K^ and of V^
  const int prt = tid & 15, trow = tid >> 4;
  const bool part_ok = prt * 8 < gch;
  auto issue = [&](uint4 (&d)[4], int n0) {
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(
        qkvh + ((size_t)b * tokens + n0) * C3, max(0, min(kTT, n_end - n0)) * C3 * 2);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int tv = 0; tv < 2; ++tv) {
        const int off =
            part_ok ? ((trow + 16 * i) * C3 + (1 + tv) * C + hg * kHG * kD + prt * 8) * 2
                    : kOob;
        d[2 * i + tv] = buf_load16(rs, off);
      }
  };

  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  float dacc = 0.f;
  uint4 st[4];
  issue(st, n_begin);
  int buf = 0;
  for (int n0 = n_begin; n0 < n_end; n0 += kTT, buf ^= 1) {
    char* T = ts[buf];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int tv = 0; tv < 2; ++tv)
        *reinterpret_cast<uint4*>(T + (trow + 16 * i) * kKvRowB + tv * kHG * kD * 2 +
                                  prt * 16) = st[2 * i + tv];
    if (n0 + kTT < n_end) issue(st, n0 + kTT);
    __syncthreads();
    uint4 cur[4];  // [K^ ks0, K^ ks1, V^ ks0, V^ ks1]
#pragma unroll
    for (int tv = 0; tv < 2; ++tv)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        cur[2 * tv + ks] = *reinterpret_cast<const uint4*>(
            T + col * kKvRowB + tv * kHG * kD * 2 + wave * kD * 2 + (16 * ks + 8 * g) * 2);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {  // relu on K^ (bf16 sign bit)
      uint16_t* hv = reinterpret_cast<uint16_t*>(&cur[ks]);
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[e] = relu_bits(hv[e]);
    }
    f32x16 kt, vt;
#pragma unroll
    for (int r = 0; r < 16; ++r) kt[r] = vt[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      kt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cur[ks]),
                                                   eye[ks], kt, 0, 0, 0);
      vt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cur[2 + ks]),
                                                   eye[ks], vt, 0, 0, 0);
    }
    // kt[r], vt[r]: feature col of token 8(r/4) + 4g + r%4
#pragma unroll
    for (int r = 0; r < 16; ++r) dacc += kt[r];
#pragma unroll
    for (int slab = 0; slab < 2; ++slab) {
      uint4 ka, vb;
      ka.x = pack_bf16x2(kt[8 * slab + 0], kt[8 * slab + 1]);
      ka.y = pack_bf16x2(kt[8 * slab + 2], kt[8 * slab + 3]);
      ka.z = pack_bf16x2(kt[8 * slab + 4], kt[8 * slab + 5]);
      ka.w = pack_bf16x2(kt[8 * slab + 6], kt[8 * slab + 7]);
      vb.x = pack_bf16x2(vt[8 * slab + 0], vt[8 * slab + 1]);
      vb.y = pack_bf16x2(vt[8 * slab + 2], vt[8 * slab + 3]);
      vb.z = pack_bf16x2(vt[8 * slab + 4], vt[8 * slab + 5]);
      vb.w = pack_bf16x2(vt[8 * slab + 6], vt[8 * slab + 7]);
      z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka),
                                                  __builtin_bit_cast(bf16x8, vb), z,
                                                  0, 0, 0);
    }
  }
  if (h >= heads) return;
  dacc += __shfl_xor(dacc, 32, 64);
  // z[r] = Z[i][c] with c = col, i = 8(r/4) + 4g + r%4
  float* out = part + ((size_t)(b * heads + h) * nchunks + chunk) * kPart;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = 8 * (r >> 2) + 4 * g + (r & 3);
    out[i * kD + col] = z[r];
  }
  if (g == 0) out[kD * kD + col] = dacc;
}

// O^T = Z^T relu(Q^)^T with Z split into bf16 hi + lo parts, normalised by
// relu(q^) . D.  grid (ceil(tokens/256), ceil(heads/4), batch), 256
// threads; wave = head of a 4-head group, eight 32-token tiles per
// workgroup.  Each tile's Q^ rows (32 tokens x 4 heads x 64 bytes) are
// loaded with 16-byte loads over whole 256-byte rows into LDS, read back in
// the MFMA operand layout (lane = token), and the normalised output goes
// back through LDS to 256-byte row stores: per-lane token-major global
// accesses would touch 32-byte pieces of 32 rows per instruction.  The next
// tile's loads are in flight while a tile is computed.
constexpr int kRowB = kHG * kD * 2 + 16;  // LDS bytes per staged token row

__global__ __launch_bounds__(256) void lin_apply_mfma(
    const bf16* __restrict__ qkvh, const float* __restrict__ kv,
    const float* __restrict__ ksum, bf16* __restrict__ o, int tokens,
    int heads) {
  __shared__ __attribute__((aligned(16))) char qs[kTT * kRowB];
  __shared__ __attribute__((aligned(16))) char os[kTT * kRowB];
  const int hg = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = hg * kHG + wave;
  const bool h_ok = h < heads;  // every wave takes part in the staging
  const int C = heads * kD, C3 = 3 * C;
  const int g = lane >> 5, col = lane & 31;
  const size_t bh = (size_t)b * heads + (h_ok ? h : 0);
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

  // This group's channels of a token row: heads * 32 may end inside the
  // group, and tokens may end inside a tile; both read zeros / store
  // nothing through per-tile buffer resources (which also keep every
  // offset small).
  const int n_base = blockIdx.x * kApplyTok;
  const int gch = min(kHG * kD, C - hg * kHG * kD);  // channels of this group
  // thread's two 16-byte chunks of a tile: token tid / 16 (+ 16), part tid % 16
  const int part = tid & 15, trow = tid >> 4;
  const bool part_ok = part * 8 < gch;
  auto tile_rows = [&](int n0) { return max(0, min(kTT, tokens - n0)); };
  auto issue = [&](uint4 (&d)[2], int n0) {
    const __amdgpu_buffer_rsrc_t rs =
        buf_rsrc(qkvh + ((size_t)b * tokens + n0) * C3, tile_rows(n0) * C3 * 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int off = part_ok ? ((trow + 16 * i) * C3 + hg * kHG * kD + part * 8) * 2 : kOob;
      d[i] = buf_load16(rs, off);
    }
  };
  uint4 st[2][2];
  issue(st[0], n_base);
#pragma unroll
  for (int tt = 0; tt < kApplyTok / kTT; ++tt) {
    const int n0 = n_base + tt * kTT;
    if (tt + 1 < kApplyTok / kTT) issue(st[(tt + 1) & 1], n0 + kTT);
    // stage this tile's rows (the previous tile's readers have passed the
    // barrier that ended their iteration)
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<uint4*>(qs + (trow + 16 * i) * kRowB + part * 16) = st[tt & 1][i];
    __syncthreads();
    uint4 cur[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      cur[ks] = *reinterpret_cast<const uint4*>(qs + col * kRowB + wave * kD * 2 +
                                                (16 * ks + 8 * g) * 2);
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    float den = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint16_t* hv = reinterpret_cast<uint16_t*>(&cur[ks]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hv[e] = relu_bits(hv[e]);
        den = fmaf(__uint_as_float((uint32_t)hv[e] << 16), dreg[ks][e], den);
      }
      const bf16x8 qb = __builtin_bit_cast(bf16x8, cur[ks]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(zhi[ks], qb, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(zlo[ks], qb, acc, 0, 0, 0);
    }
    den += __shfl_xor(den, 32, 64);
    const float inv = den > 0.f ? 1.f / den : 0.f;
    // acc[4j + e]: feature 8j + 4g + e of token col
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint2 w;
      w.x = pack_bf16x2(acc[4 * j + 0] * inv, acc[4 * j + 1] * inv);
      w.y = pack_bf16x2(acc[4 * j + 2] * inv, acc[4 * j + 3] * inv);
      *reinterpret_cast<uint2*>(os + col * kRowB + wave * kD * 2 + (8 * j + 4 * g) * 2) = w;
    }
    __syncthreads();
    const __amdgpu_buffer_rsrc_t ors =
        buf_rsrc(o + ((size_t)b * tokens + n0) * C, tile_rows(n0) * C * 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 v = *reinterpret_cast<const uint4*>(os + (trow + 16 * i) * kRowB + part * 16);
      const int off = part_ok ? ((trow + 16 * i) * C + hg * kHG * kD + part * 8) * 2 : kOob;
      __builtin_amdgcn_raw_buffer_store_b128(
          i32x4{(int)v.x, (int)v.y, (int)v.z, (int)v.w}, ors, off, 0, 0);
    }
  }
  (void)h_ok;
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
    dim3 grid((tokens + kApplyTok - 1) / kApplyTok, (heads + kHG - 1) / kHG, batch);
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
