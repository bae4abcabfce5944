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
#include "gate_select.h"
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

// grid (batch * heads, ceil(kPart / 64)), 256 threads: entry e of the
// workgroup's 64 per group of 64 threads; group q adds chunks
// [q nc/4, (q+1) nc/4) in chunk order, then the four group sums are added in
// group order (a fixed association: bitwise reproducible).
__device__ void kv_combine_body(const float* __restrict__ part, float* __restrict__ kv,
                                float* __restrict__ ksum, int nchunks, int bh, int grp) {
  __shared__ float red[4][64];
  const float* p = part + (size_t)bh * nchunks * kPart;
  const int t = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int e = grp * 64 + t;
  const int c0 = (nchunks * q) / 4, c1 = (nchunks * (q + 1)) / 4;
  float s = 0.f;
  if (e < kPart) {
    // loads issued 16 (then 4) at a time, added strictly in chunk order
    int c = c0;
    for (; c + 16 <= c1; c += 16) {
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = p[(size_t)(c + i) * kPart + e];
#pragma unroll
      for (int i = 0; i < 16; ++i) s += v[i];
    }
    for (; c + 4 <= c1; c += 4) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = p[(size_t)(c + i) * kPart + e];
#pragma unroll
      for (int i = 0; i < 4; ++i) s += v[i];
    }
    for (; c < c1; ++c) s += p[(size_t)c * kPart + e];
  }
  red[q][t] = s;
  __syncthreads();
  if (q == 0 && e < kPart) {
    s = ((red[0][t] + red[1][t]) + red[2][t]) + red[3][t];
    if (e < kD * kD)
      kv[(size_t)bh * kD * kD + e] = s;
    else
      ksum[(size_t)bh * kD + (e - kD * kD)] = s;
  }
}

constexpr int kCombineGroups = (kPart + 63) / 64;  // entry groups per (image, head)

__global__ __launch_bounds__(256) void kv_combine_kernel(
    const float* __restrict__ part, float* __restrict__ kv,
    float* __restrict__ ksum, int nchunks) {
  kv_combine_body(part, kv, ksum, nchunks, blockIdx.x, blockIdx.y);
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
constexpr int kChunkTok = 512;  // tokens per partial (bf16 path), at most
constexpr int kMinChunkTok = 128;
// Partials are kept at kChunkTok tokens while the launch yields at least one
// workgroup per CU; smaller launches halve the chunk (down to kMinChunkTok).
// Smaller chunks cost partial traffic and a longer combine, so they only pay
// where CUs would idle (measured: 4 x 64x128 tokens, 8 heads 19.4 -> 14.7
// us; 8 x 128x128 at 4 heads 21.5 -> 24.9 us with four times the chunks).
// The decision takes the batch of the whole call, so a call split over
// image ranges sums the same chunks.
constexpr int kChunkMinWgs = 256;
constexpr int kApplyTok = 256;  // tokens per workgroup in the readout, at most
// A readout launch with fewer than this many workgroups takes 128 tokens per
// workgroup instead (the Z setup of a workgroup is then amortised over half
// the tokens, which only pays where CUs would otherwise idle).
constexpr int kApplyMinWgs = 512;

// Tokens of a 32-token tile that lie before `left` more tokens, 0..32.  The
// clamp is a vector instruction (there is no scalar med3); taken back into a
// scalar register, the buffer resources built from it stay scalar.  Left in a
// vector register, every buffer load over such a resource became a
// single-pass readfirstlane loop (readout 22.0 -> 21.5 us).
__device__ __forceinline__ int tile_tokens(int left) {
  return __builtin_amdgcn_readfirstlane(max(0, min(kTT, left)));
}

__device__ __forceinline__ uint16_t relu_bits(uint16_t u) {
  return (u & 0x8000u) ? 0 : u;
}

// One wave per head of a 4-head group, tiles of 32 tokens.  Each tile's
// K^ and V^ rows (32 tokens x 4 heads x 64 bytes each) are loaded with
// 16-byte loads over whole 256-byte rows into one of two LDS buffers (one
// barrier per tile), token-major as they lie in HBM.  Z += relu(K^)^T V^
// contracts over tokens, so both MFMA operands need eight consecutive tokens
// of one feature per lane: gfx950's transposing LDS read (ds_read_b64_tr_b16)
// supplies them.  Within each group of 16 lanes, lane j receives element
// j % 4 of the four 16-bit values that lane 4e + j / 4 addresses, e = 0..3;
// so when lane k of the group addresses features f0 + 4 (k % 4) .. + 3 of
// token t0 + k / 4, lane j gets feature f0 + j of tokens t0 .. t0 + 3.  Two
// such reads give a lane its eight tokens, the matrix cores do only the
// contraction, relu is a packed 16-bit integer max with 0 on the loaded
// K^ values (the bf16 sign bit is the int16 sign), and D sums them.  Tokens
// past the chunk read zeros (which add nothing) through per-tile buffer
// resources.
// grid (chunks, ceil(heads/4), batch), 256 threads = 4 heads.
constexpr int kKvRowB = 2 * kHG * kD * 2 + 32;  // LDS bytes per token row: K^ | V^

typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ uint32_t relu_bf16x2(uint32_t w) {
  const i16x2 v = __builtin_bit_cast(i16x2, w);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(v, (i16x2){0, 0}));
}

__device__ void kv_partial_body(const bf16* __restrict__ qkvh, float* __restrict__ part,
                                int tokens, int heads, int nchunks, int chunk_tok, int chunk,
                                int hg, int b) {
  __shared__ __attribute__((aligned(16))) char ts[2][kTT * kKvRowB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = hg * kHG + wave;  // h >= heads: stages, computes nothing kept
  const int C = heads * kD, C3 = 3 * C;
  const int g = lane >> 5, col = lane & 31;
  const int n_begin = chunk * chunk_tok;
  const int n_end = min(tokens, n_begin + chunk_tok);
  const int gch = min(kHG * kD, C - hg * kHG * kD);  // channels of this group

  // thread's four 16-byte chunks of a tile: token tid / 16 (+ 16),
  // part tid % 16 of K^ and of V^
  const int prt = tid & 15, trow = tid >> 4;
  const bool part_ok = prt * 8 < gch;
  auto issue = [&](uint4 (&d)[4], int n0) {
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(
        qkvh + ((size_t)b * tokens + n0) * C3, tile_tokens(n_end - n0) * C3 * 2);
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
  // this lane's transposed reads: lane k of its 16-lane group addresses
  // token 8 g + k / 4 (+ 4 for the second read, + 16 ks for the k-step) and
  // features 16 ((lane / 16) % 2) + 4 (k % 4) .. + 3 of head `wave`; the
  // group's lanes then hold features col of four consecutive tokens
  const int kq = lane & 15;
  const int tr_off = (8 * g + (kq >> 2)) * kKvRowB + wave * kD * 2 +
                     (16 * ((lane >> 4) & 1) + 4 * (kq & 3)) * 2;
  auto tr_read = [&](const char* T, int tv, int ks, int half) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)((lds_char*)T + tr_off + (16 * ks + 4 * half) * kKvRowB +
                     tv * kHG * kD * 2));
    return __builtin_bit_cast(uint2, v);
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
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // relu(K^)^T: row = feature col, k = tokens 16 ks + 8 g .. + 7;
      // V^: column = feature col, the same tokens
      const uint2 k0 = tr_read(T, 0, ks, 0), k1 = tr_read(T, 0, ks, 1);
      const uint2 v0 = tr_read(T, 1, ks, 0), v1 = tr_read(T, 1, ks, 1);
      const uint32_t aw[4] = {relu_bf16x2(k0.x), relu_bf16x2(k0.y), relu_bf16x2(k1.x),
                              relu_bf16x2(k1.y)};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dacc += __uint_as_float(aw[e] << 16) + __uint_as_float(aw[e] & 0xffff0000u);
      const uint4 a = {aw[0], aw[1], aw[2], aw[3]};
      const uint4 v = {v0.x, v0.y, v1.x, v1.y};
      z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, v), z, 0, 0, 0);
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

__global__ __launch_bounds__(256) void kv_partial_mfma(
    const bf16* __restrict__ qkvh, float* __restrict__ part, int tokens,
    int heads, int nchunks, int chunk_tok) {
  kv_partial_body(qkvh, part, tokens, heads, nchunks, chunk_tok, blockIdx.x, blockIdx.y,
                  blockIdx.z);
}

// The K/V state with the gate's top-k beside it (FT 3.2 selection; both
// only read the S2 conv's outputs), in the same two launches: the selection
// is latency-bound work of a few workgroups, which then overlaps the
// bandwidth-bound reduction instead of taking launches of its own.
// Launch 1: workgroups 0 .. batch * kRankParts - 1 count the rank runs of
// the gate's scores formed from its partial logits (rank_part_wg, run
// bid % kRankParts of image bid / kRankParts), the others are the
// partial-sum workgroups of kv_partial_mfma, numbered chunk fastest, then
// head group, then image.
__global__ __launch_bounds__(256) void kv_partial_rank_kernel(
    const bf16* __restrict__ qkvh, float* __restrict__ part, int tokens, int heads,
    int nchunks, int chunk_tok, int batch, const float* __restrict__ plog,
    const float* __restrict__ gb, float* __restrict__ scores, int32_t* __restrict__ rankp,
    int nblocks, int tpow, float inv_cnt) {
  __shared__ uint64_t keys[1024 / kRankParts];
  const int bid = blockIdx.x;
  if (bid < batch * kRankParts) {
    rank_part_wg<true>(plog, rankp, nblocks, tpow, gb, heads, inv_cnt, scores,
                       bid % kRankParts, bid / kRankParts, keys);
    return;
  }
  const int w = bid - batch * kRankParts;
  const int hgs = (heads + kHG - 1) / kHG;
  kv_partial_body(qkvh, part, tokens, heads, nchunks, chunk_tok, w % nchunks,
                  (w / nchunks) % hgs, w / (nchunks * hgs));
}

// Launch 2: workgroups 0 .. batch - 1 add the runs and write each image's
// ascending list (rank_final_wg; the ranks are exact counts, so the list
// equals the gate's own top-k launches'), the others combine the chunk
// partials as kv_combine_kernel: workgroup w takes entry group
// w % kCombineGroups of (image, head) w / kCombineGroups.
__global__ __launch_bounds__(256) void kv_combine_final_kernel(
    const float* __restrict__ part, float* __restrict__ kv, float* __restrict__ ksum,
    int nchunks, int batch, const int32_t* __restrict__ rankp, int32_t* __restrict__ sel,
    int nblocks, int keep, int tpow) {
  __shared__ int rank[1024];
  const int bid = blockIdx.x;
  if (bid < batch) {
    rank_final_wg(rankp, sel, nblocks, keep, tpow, bid, rank);
    return;
  }
  const int w = bid - batch;
  kv_combine_body(part, kv, ksum, nchunks, w / kCombineGroups, w % kCombineGroups);
}

// O^T = Z^T relu(Q^)^T with Z split into bf16 hi + lo parts, normalised by
// relu(q^) . D.  grid (ceil(tokens/APPLY_TOK), ceil(heads/4), batch), 256
// threads; wave = head of a 4-head group, APPLY_TOK / 32 tiles of 32 tokens
// per workgroup.  Each tile's Q^ rows (32 tokens x 4 heads x 64 bytes) are
// loaded with 16-byte loads over whole 256-byte rows into LDS, read back in
// the MFMA operand layout (lane = token), and the normalised output goes
// back through LDS to 256-byte row stores: per-lane token-major global
// accesses would touch 32-byte pieces of 32 rows per instruction.  The next
// tile's loads are in flight while a tile is computed.
constexpr int kRowB = kHG * kD * 2 + 16;  // LDS bytes per staged token row

template <int APPLY_TOK>
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
  const int n_base = blockIdx.x * APPLY_TOK;
  const int gch = min(kHG * kD, C - hg * kHG * kD);  // channels of this group
  // thread's two 16-byte chunks of a tile: token tid / 16 (+ 16), part tid % 16
  const int part = tid & 15, trow = tid >> 4;
  const bool part_ok = part * 8 < gch;
  auto tile_rows = [&](int n0) { return tile_tokens(tokens - n0); };
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
  for (int tt = 0; tt < APPLY_TOK / kTT; ++tt) {
    const int n0 = n_base + tt * kTT;
    if (tt + 1 < APPLY_TOK / kTT) issue(st[(tt + 1) & 1], n0 + kTT);
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

// tokens per bf16 partial for a call of `batch` images of `tokens` tokens
int kv_chunk_tokens(int batch, int heads, int tokens) {
  const int64_t hg = (heads + kHG - 1) / kHG;
  int ct = kChunkTok;
  while (ct > kMinChunkTok && ((tokens + ct - 1) / ct) * hg * batch < kChunkMinWgs) ct /= 2;
  return ct;
}

int kv_chunks(bool bf, int batch, int heads, int tokens) {
  if (bf) {
    const int ct = kv_chunk_tokens(batch, heads, tokens);
    return (tokens + ct - 1) / ct;
  }
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
                           int heads, hipStream_t s, int chunk_batch) {
  if (chunk_batch <= 0) chunk_batch = batch;
  if (bf && chunk_batch < batch) return hipErrorInvalidValue;
  const int chunks = kv_chunks(bf, bf ? chunk_batch : batch, heads, tokens);
  if (bf) {
    dim3 grid(chunks, (heads + kHG - 1) / kHG, batch);
    kv_partial_mfma<<<grid, 256, 0, s>>>(static_cast<const bf16*>(qkv_hat),
                                         partials, tokens, heads, chunks,
                                         kv_chunk_tokens(chunk_batch, heads, tokens));
  } else {
    const int chunk_len = (tokens + chunks - 1) / chunks;
    dim3 grid(chunks, heads, batch);
    kv_partial_kernel<float><<<grid, 256, 0, s>>>(
        static_cast<const float*>(qkv_hat), partials, tokens, heads, chunk_len);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 cgrid(batch * heads, kCombineGroups);
  kv_combine_kernel<<<cgrid, 256, 0, s>>>(partials, kv, ksum, chunks);
  return hipGetLastError();
}

hipError_t launch_kv_state_topk(const void* qkv_hat, float* kv, float* ksum, float* partials,
                                int batch, int tokens, int heads, hipStream_t s,
                                int chunk_batch, const float* plog, const float* gate_b,
                                float* scores, int32_t* sel, int32_t* rankp, int nblocks,
                                int block, int keep) {
  if (chunk_batch <= 0) chunk_batch = batch;
  if (chunk_batch < batch || nblocks <= 0 || !rankp) return hipErrorInvalidValue;
  int tpow = 2;
  while (tpow < nblocks) tpow <<= 1;
  if (tpow < 16 * kRankParts || tpow > 1024) return hipErrorInvalidValue;
  const int chunks = kv_chunks(true, chunk_batch, heads, tokens);
  const int hgs = (heads + kHG - 1) / kHG;
  kv_partial_rank_kernel<<<batch * kRankParts + chunks * hgs * batch, 256, 0, s>>>(
      static_cast<const bf16*>(qkv_hat), partials, tokens, heads, chunks,
      kv_chunk_tokens(chunk_batch, heads, tokens), batch, plog, gate_b, scores, rankp, nblocks,
      tpow, 1.f / (float)(block * block));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  kv_combine_final_kernel<<<batch + batch * heads * kCombineGroups, 256, 0, s>>>(
      partials, kv, ksum, chunks, batch, rankp, sel, nblocks, keep, tpow);
  return hipGetLastError();
}

hipError_t launch_lin_apply(bool bf, const void* qkv_hat, const float* kv,
                            const float* ksum, void* o, int batch, int tokens,
                            int heads, hipStream_t s) {
  if (bf) {
    const int hg = (heads + kHG - 1) / kHG;
    const int64_t wgs = (int64_t)((tokens + kApplyTok - 1) / kApplyTok) * hg * batch;
    if (wgs >= kApplyMinWgs) {
      dim3 grid((tokens + kApplyTok - 1) / kApplyTok, hg, batch);
      lin_apply_mfma<kApplyTok><<<grid, 256, 0, s>>>(static_cast<const bf16*>(qkv_hat), kv,
                                                     ksum, static_cast<bf16*>(o), tokens, heads);
    } else {
      constexpr int kHalf = kApplyTok / 2;
      dim3 grid((tokens + kHalf - 1) / kHalf, hg, batch);
      lin_apply_mfma<kHalf><<<grid, 256, 0, s>>>(static_cast<const bf16*>(qkv_hat), kv, ksum,
                                                 static_cast<bf16*>(o), tokens, heads);
    }
    return hipGetLastError();
  }
  dim3 grid((tokens + 63) / 64, heads, batch);
    lin_apply_kernel<float><<<grid, 64, 0, s>>>(static_cast<const float*>(qkv_hat),
                                                kv, ksum, static_cast<float*>(o),
                                                tokens, heads);
  return hipGetLastError();
}

}  // namespace hsmla
