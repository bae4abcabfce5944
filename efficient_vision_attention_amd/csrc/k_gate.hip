// Block-level gate and selection.
//
// Scores (FT 3.2 head-level score and block-level aggregation):
//   f_t^(h) = mean over the block's tokens of [Q_hat; K_hat; V_hat]^(h),
//             or, with the gate's depthwise 3x3 kernel g, of
//             DWConv3x3_g([Q_hat; K_hat; V_hat])^(h) (zero padding at the
//             image border)
//   M_t     = (1/H) sum_h sigmoid(w^(h) . f_t^(h) + b^(h))
// Selection, written in ascending block order -- the compacted tile list the
// refinement kernel runs over (FT 3.6 stage 3) -- either
//   top-k:     the keep largest M_t per image, equal scores to the lower block
//              index: each block's rank counted against every other
//              block's key (up to 1024 blocks; over several workgroups per
//              image from 128), or a bitonic sort in LDS above that (the
//              count is fixed, so the grid size is known on the host), or
//   threshold: every block with M_t > tau (FT 3.2 gating equation); the
//              per-image count goes to device memory, or
//   per head:  for each head h the blocks with G^(h)_t > tau (FT 3.2 per-head
//              output routing), one list and count per (image, head).
#include <math.h>

#include "common.h"
#include "gate_select.h"
#include "kernels.h"

namespace hsmla {
namespace {

constexpr int kD = 32;
constexpr int kXcds = 8;

// Per-head logits from the channel sums of one block (fsum[3C], already in
// LDS), then M_t; one wave per head, wave reduction in fixed lane order.
// score (optional) receives M_t, head_score (optional) G^(h) of the block
// for h = 0 .. heads-1.
__device__ void gate_tail(const float* fsum, float* gsig,
                          const float* __restrict__ gw,
                          const float* __restrict__ gb, int heads, int C,
                          float inv_cnt, float* score, float* head_score) {
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  for (int h = wave; h < heads; h += blockDim.x / 64) {
    float p = 0.f;
    for (int f = lane; f < 3 * kD; f += 64) {
      const int s = f / kD, j = f % kD;
      p = fmaf(gw[h * 3 * kD + f], fsum[s * C + h * kD + j] * inv_cnt, p);
    }
    p = wave_sum(p);
    if (lane == 0) {
      const float g = 1.f / (1.f + expf(-(p + gb[h])));
      gsig[h] = g;
      if (head_score) head_score[h] = g;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && score) {
    float m = 0.f;
    for (int h = 0; h < heads; ++h) m += gsig[h];
    *score = m / (float)heads;
  }
}

// grid (blocks per image, batch), 256 threads.  Channel sums over the
// block's tokens go to LDS (fixed token order per channel), then one wave
// forms each head's logit with a wave reduction in fixed lane order.
template <typename T>
__global__ __launch_bounds__(256) void gate_scores_kernel(
    const T* __restrict__ qkvh, const float* __restrict__ gw,
    const float* __restrict__ gb, float* __restrict__ scores,
    float* __restrict__ head_scores, int gh, int gwid, int heads, int block) {
  extern __shared__ float sh[];
  const int C = heads * kD, C3 = 3 * C;
  float* fsum = sh;          // [3C]
  float* gsig = sh + C3;     // [heads]
  const int t = blockIdx.x, b = blockIdx.y;
  const int nbc = gwid / block;
  const int r0 = (t / nbc) * block, c0 = (t % nbc) * block;
  const size_t img = (size_t)b * gh * gwid;
  // 16-byte vectors of channels, summed over the block's tokens in row-major
  // token order
  constexpr int V = 16 / sizeof(T);
  for (int cv = threadIdx.x; cv < C3 / V; cv += blockDim.x) {
    float s[V];
#pragma unroll
    for (int j = 0; j < V; ++j) s[j] = 0.f;
    for (int yy = 0; yy < block; ++yy) {
      const T* rowp = qkvh + (img + (size_t)(r0 + yy) * gwid + c0) * C3 + cv * V;
      for (int xx = 0; xx < block; ++xx) {
        const uint4 u = *reinterpret_cast<const uint4*>(rowp + (size_t)xx * C3);
        const T* e = reinterpret_cast<const T*>(&u);
#pragma unroll
        for (int j = 0; j < V; ++j) s[j] += to_f32(e[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < V; ++j) fsum[cv * V + j] = s[j];
  }
  __syncthreads();
  gate_tail(fsum, gsig, gw, gb, heads, C, 1.f / (float)(block * block),
            scores ? scores + (size_t)b * gridDim.x + t : nullptr,
            head_scores ? head_scores + ((size_t)b * gridDim.x + t) * heads : nullptr);
}

// grid (blocks per image, batch), 256 threads: the scores from block sums
// already reduced elsewhere (bsum [b][t][3C]).
__global__ __launch_bounds__(256) void gate_from_sums_kernel(
    const float* __restrict__ bsum, const float* __restrict__ gw,
    const float* __restrict__ gb, float* __restrict__ scores,
    float* __restrict__ head_scores, int heads, float inv_cnt) {
  extern __shared__ float sh[];
  const int C = heads * kD, C3 = 3 * C;
  float* fsum = sh;       // [3C]
  float* gsig = sh + C3;  // [heads]
  const int t = blockIdx.x, b = blockIdx.y;
  const size_t row = (size_t)b * gridDim.x + t;
  const float4* src = reinterpret_cast<const float4*>(bsum + row * C3);
  for (int i = threadIdx.x; i < C3 / 4; i += blockDim.x)
    reinterpret_cast<float4*>(fsum)[i] = src[i];
  __syncthreads();
  gate_tail(fsum, gsig, gw, gb, heads, C, inv_cnt, scores ? scores + row : nullptr,
            head_scores ? head_scores + row * heads : nullptr);
}

// Four consecutive channels of one token as float32 (8-byte bf16 or 16-byte
// float32 vector load).
__device__ __forceinline__ void load4(const bf16* p, float* v) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(u.x << 16);
  v[1] = __uint_as_float(u.x & 0xffff0000u);
  v[2] = __uint_as_float(u.y << 16);
  v[3] = __uint_as_float(u.y & 0xffff0000u);
}
__device__ __forceinline__ void load4(const float* p, float* v) {
  const float4 u = *reinterpret_cast<const float4*>(p);
  v[0] = u.x;
  v[1] = u.y;
  v[2] = u.z;
  v[3] = u.w;
}

// Gate with the depthwise 3x3 inside the head score.  The block sum of the
// convolution is linear in the input, so it is formed without the
// convolved map: with the block's rows r0..r0+Bs-1 and columns c0..,
//   sum_{p in block} conv(p) = sum_{dy,dx} g[dy][dx] * S(dy, dx),
// where S(dy, dx) sums the input over the block shifted by (dy-1, dx-1)
// (zero outside the image).  Per halo row y the three column-shifted sums
// U_dx(y) are built from the row's Bs + 2 tokens, and row y feeds the
// vertical shifts dy whose shifted block contains it.  One thread owns 4
// channels and keeps their 36 taps in registers.
// Grid: 1-D over (batch, block) remapped so each XCD walks a contiguous run
// of neighbouring blocks, whose halos then hit in that XCD's L2.
template <typename T>
__global__ __launch_bounds__(1024) void gate_scores_conv_kernel(
    const T* __restrict__ qkvh, const T* __restrict__ gdw,
    const float* __restrict__ gw, const float* __restrict__ gb,
    float* __restrict__ scores, float* __restrict__ head_scores, int gh,
    int gwid, int heads, int block, int nblocks, int total, int per_xcd) {
  extern __shared__ float sh[];
  const int C = heads * kD, C3 = 3 * C;
  float* fsum = sh;       // [3C]
  float* gsig = sh + C3;  // [heads]
  const int tile = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (tile >= total) return;
  const int b = tile / nblocks, t = tile % nblocks;
  const int nbc = gwid / block;
  const int r0 = (t / nbc) * block, c0 = (t % nbc) * block;
  const size_t img = (size_t)b * gh * gwid;
  for (int cv = threadIdx.x; cv < C3 / 4; cv += blockDim.x) {
    float g[4][9];
    {
      float tmp[36];
#pragma unroll
      for (int i = 0; i < 9; ++i) load4(gdw + (size_t)cv * 36 + 4 * i, tmp + 4 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 9; ++i) g[j][i] = tmp[9 * j + i];
    }
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    const int ylo = max(r0 - 1, 0), yhi = min(r0 + block, gh - 1);
    for (int y = ylo; y <= yhi; ++y) {
      const T* rowp = qkvh + (img + (size_t)y * gwid) * C3 + cv * 4;
      float vl[4] = {0.f, 0.f, 0.f, 0.f}, vr[4] = {0.f, 0.f, 0.f, 0.f};
      float v0[4], vb1[4], inner[4] = {0.f, 0.f, 0.f, 0.f};
      if (c0 > 0) load4(rowp + (size_t)(c0 - 1) * C3, vl);
      if (c0 + block < gwid) load4(rowp + (size_t)(c0 + block) * C3, vr);
      load4(rowp + (size_t)c0 * C3, v0);
      load4(rowp + (size_t)(c0 + block - 1) * C3, vb1);
      for (int x = c0 + 1; x < c0 + block - 1; ++x) {
        float v[4];
        load4(rowp + (size_t)x * C3, v);
#pragma unroll
        for (int j = 0; j < 4; ++j) inner[j] += v[j];
      }
      // vertical shifts dy whose shifted block holds row y
      const int yl = y - r0;
      const int dylo = max(0, yl + 2 - block), dyhi = min(2, yl + 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float u0, u1, u2;
        if (block == 1) {
          u0 = vl[j];
          u1 = v0[j];
          u2 = vr[j];
        } else {
          u0 = vl[j] + v0[j] + inner[j];
          u1 = v0[j] + inner[j] + vb1[j];
          u2 = inner[j] + vb1[j] + vr[j];
        }
        float a = acc[j];
#pragma unroll
        for (int dy = 0; dy < 3; ++dy) {
          if (dy < dylo || dy > dyhi) continue;  // uniform over the workgroup
          a = fmaf(g[j][3 * dy + 0], u0, a);
          a = fmaf(g[j][3 * dy + 1], u1, a);
          a = fmaf(g[j][3 * dy + 2], u2, a);
        }
        acc[j] = a;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) fsum[cv * 4 + j] = acc[j];
  }
  __syncthreads();
  gate_tail(fsum, gsig, gw, gb, heads, C, 1.f / (float)(block * block),
            scores ? scores + (size_t)b * nblocks + t : nullptr,
            head_scores ? head_scores + ((size_t)b * nblocks + t) * heads : nullptr);
}

// Top-k of one image by counting ranks (tpow <= blockDim keys): shk[0 ..
// tpow) holds the keys (padding 0), rank[] has room for tpow ints.  rank(t)
// = #{u : key_u > key_t}, the keys being distinct; the key range is split
// into `parts` runs of at least 64 keys, one thread per (t, run), and the
// runs' counts are added in LDS.  Every thread of a wave reads the same keys
// (a broadcast).  T^2 comparisons, but no barrier between them.  The blocks
// of rank below keep are written to sel in ascending order.
__device__ void rank_select(const uint64_t* shk, int* rank, int nblocks, int tpow,
                            int keep, int32_t* __restrict__ sel) {
  const int parts = min((int)blockDim.x / tpow, max(1, tpow / 64));
  const int t = threadIdx.x % tpow, q = threadIdx.x / tpow;
  if (threadIdx.x < tpow) rank[threadIdx.x] = 0;
  __syncthreads();
  const int len = tpow / parts;
  if (q < parts && t < nblocks) {
    const uint64_t kt = shk[t];
    const uint64_t* ku = shk + q * len;
    int cnt = 0;
    if (len % 16 == 0) {
      for (int u = 0; u < len; u += 16) {
        uint64_t v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = ku[u + i];
#pragma unroll
        for (int i = 0; i < 16; ++i) cnt += v[i] > kt;
      }
    } else {
      for (int u = 0; u < len; ++u) cnt += ku[u] > kt;
    }
    atomicAdd(&rank[t], cnt);
  }
  __syncthreads();
  compact_ascending([&](int u) { return rank[u] < keep; }, nblocks, sel);
}

// grid (batch), 1024 threads.  The scores of one image are sorted in LDS by
// a bitonic network on one 64-bit key per block: the score mapped to an
// order-preserving unsigned integer (-0 taken as +0) in the high word and
// the complement of the block index in the low word, sorted descending --
// score descending, then block index ascending, a total order.  The first
// `keep` entries are therefore exactly the blocks whose rank
// #{u : s_u > s_t or (s_u == s_t and u < t)} is below keep; they are
// flagged and written out in ascending order by the ballot compaction.  The
// row is padded to a power of two with key 0, which sorts after every real
// entry.  O(T log^2 T) comparisons; exact and order-independent.  Up to
// 1024 blocks the rank is counted directly instead (same keys, same
// result): T^2 comparisons in one pass cost less than the sort's
// log^2 T / 2 barrier-separated stages.
__global__ __launch_bounds__(1024) void topk_kernel(
    const float* __restrict__ scores, float* __restrict__ scores_copy,
    int32_t* __restrict__ sel, int nblocks, int keep, int tpow) {
  extern __shared__ uint64_t shk[];  // [tpow] keys, later the kept flags
  constexpr int kMaxPerThread = 8;   // keep <= 8192 = 1024 threads x 8
  const int b = blockIdx.x;
  const float* src = scores + (size_t)b * nblocks;
  for (int t = threadIdx.x; t < tpow; t += blockDim.x) {
    if (t < nblocks) {
      const float v = src[t];
      shk[t] = topk_key(v, t);
      if (scores_copy) scores_copy[(size_t)b * nblocks + t] = v;
    } else {
      shk[t] = 0;
    }
  }
  __syncthreads();
  if (tpow <= (int)blockDim.x) {
    __shared__ int rank[1024];
    rank_select(shk, rank, nblocks, tpow, keep, sel + (size_t)b * keep);
    return;
  }
  for (int size = 2; size <= tpow; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (tpow >> 1); i += blockDim.x) {
        const int a = 2 * stride * (i / stride) + (i % stride), c = a + stride;
        const uint64_t ka = shk[a], kc = shk[c];
        // runs with (a & size) == 0 sort descending, the others ascending
        if ((kc > ka) == ((a & size) == 0)) {
          shk[a] = kc;
          shk[c] = ka;
        }
      }
      __syncthreads();
    }
  }
  // the first keep sorted entries, then the LDS is reused for byte flags
  int mine[kMaxPerThread];
#pragma unroll
  for (int q = 0; q < kMaxPerThread; ++q) {
    const int r = threadIdx.x + q * blockDim.x;
    mine[q] = r < keep ? static_cast<int>(0xffffffffu - static_cast<uint32_t>(shk[r])) : -1;
  }
  __syncthreads();
  unsigned char* kept = reinterpret_cast<unsigned char*>(shk);
  for (int t = threadIdx.x; t < nblocks; t += blockDim.x) kept[t] = 0;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kMaxPerThread; ++q)
    if (mine[q] >= 0) kept[mine[q]] = 1;
  __syncthreads();
  compact_ascending([&](int t) { return kept[t] != 0; }, nblocks,
                    sel + (size_t)b * keep);
}

// The same ranks over more CUs (up to 1024 blocks): grid (kRankParts,
// batch), tpow threads, workgroup s counting run s (rank_part_wg);
// rank_final_kernel adds the runs and compacts.  The counts are exact
// integers, so the ranks equal rank_select's.
template <bool FROM_PARTS>
__global__ __launch_bounds__(1024) void rank_part_kernel(const float* __restrict__ scores,
                                                         int32_t* __restrict__ part,
                                                         int nblocks, int tpow,
                                                         const float* __restrict__ gb,
                                                         int heads, float inv_cnt,
                                                         float* __restrict__ scores_out) {
  __shared__ uint64_t keys[1024 / kRankParts];
  rank_part_wg<FROM_PARTS>(scores, part, nblocks, tpow, gb, heads, inv_cnt, scores_out,
                           blockIdx.x, blockIdx.y, keys);
}

// Up to kDirectTopk blocks per image the same scores and ranks in one
// launch: grid (batch), 1024 threads; the scores formed from the partial
// logits go to LDS as keys and rank_select counts and compacts them inside
// the workgroup (the ranks are exact integers, so the lists equal the
// two-launch form's; measured on 4 images of 128 blocks: one launch of
// about 5 us instead of two).
constexpr int kDirectTopk = 256;
__global__ __launch_bounds__(1024) void gate_topk_direct_kernel(
    const float* __restrict__ plog, const float* __restrict__ gb,
    float* __restrict__ scores_out, int32_t* __restrict__ sel, int nblocks, int tpow,
    int heads, float inv_cnt, int keep) {
  __shared__ uint64_t shk[kDirectTopk];
  __shared__ int rank[kDirectTopk];
  const int b = blockIdx.x;
  for (int t = threadIdx.x; t < tpow; t += blockDim.x) {
    if (t < nblocks) {
      const float v = score_from_parts(plog + ((size_t)b * nblocks + t) * 3 * heads, gb,
                                       heads, inv_cnt);
      scores_out[(size_t)b * nblocks + t] = v;
      shk[t] = topk_key(v, t);
    } else {
      shk[t] = 0;
    }
  }
  __syncthreads();
  rank_select(shk, rank, nblocks, tpow, keep, sel + (size_t)b * keep);
}

// grid ceil(batch * nblocks / 16), 16 * heads threads: thread (block, h) =
// (tid / heads, tid % heads) forms G^(h); the block's first thread then
// adds its heads' values in head order, as score_from_parts does, so M_t
// equals the top-k path's bit for bit.
__global__ __launch_bounds__(1024) void gate_from_parts_kernel(
    const float* __restrict__ plog, const float* __restrict__ gb, float* __restrict__ scores,
    float* __restrict__ head_scores, int total, int heads, float inv_cnt) {
  __shared__ float gs[1024];
  const int blk = blockIdx.x * 16 + threadIdx.x / heads, h = threadIdx.x % heads;
  const bool ok = blk < total;
  float g = 0.f;
  if (ok) {
    const float* P = plog + (size_t)blk * 3 * heads;
    const float p = ((P[h] + P[heads + h]) + P[2 * heads + h]) * inv_cnt;
    g = 1.f / (1.f + expf(-(p + gb[h])));
    if (head_scores) head_scores[(size_t)blk * heads + h] = g;
  }
  gs[threadIdx.x] = g;
  __syncthreads();
  if (ok && h == 0) {
    float m = 0.f;
    for (int u = 0; u < heads; ++u) m += gs[threadIdx.x + u];
    scores[blk] = m / (float)heads;
  }
}

// grid (batch), 1024 threads: rank(t) = sum of the runs' counts, then the
// blocks of rank below keep in ascending order (rank_final_wg).
__global__ __launch_bounds__(1024) void rank_final_kernel(const int32_t* __restrict__ part,
                                                          int32_t* __restrict__ sel,
                                                          int nblocks, int keep, int tpow) {
  __shared__ int rank[1024];
  rank_final_wg(part, sel, nblocks, keep, tpow, blockIdx.x, rank);
}

// grid (batch), 1024 threads: sel[b][0 .. n) = ascending blocks with
// M_t > tau, counts[b] = n.  Float32 comparison, so a score equal to tau is
// not routed.
__global__ __launch_bounds__(1024) void threshold_kernel(
    const float* __restrict__ scores, float* __restrict__ scores_copy,
    int32_t* __restrict__ sel, int32_t* __restrict__ counts, int nblocks,
    float tau) {
  const int b = blockIdx.x;
  const float* src = scores + (size_t)b * nblocks;
  if (scores_copy)
    for (int t = threadIdx.x; t < nblocks; t += blockDim.x)
      scores_copy[(size_t)b * nblocks + t] = src[t];
  const int n = compact_ascending([&](int t) { return src[t] > tau; }, nblocks,
                                  sel + (size_t)b * nblocks);
  if (threadIdx.x == 0) counts[b] = n;
}

// Per-head routing: grid (heads, batch), 1024 threads.  sel[b][h][0 .. n) =
// ascending blocks with G^(h) > tau (head scores laid out [b][t][h]),
// counts[b][h] = n.
__global__ __launch_bounds__(1024) void threshold_heads_kernel(
    const float* __restrict__ hs, float* __restrict__ hs_copy,
    int32_t* __restrict__ sel, int32_t* __restrict__ counts, int nblocks,
    int heads, float tau) {
  const int h = blockIdx.x, b = blockIdx.y;
  const float* src = hs + (size_t)b * nblocks * heads + h;
  if (hs_copy)
    for (int t = threadIdx.x; t < nblocks; t += blockDim.x)
      hs_copy[((size_t)b * nblocks + t) * heads + h] = src[(size_t)t * heads];
  const int n = compact_ascending(
      [&](int t) { return src[(size_t)t * heads] > tau; }, nblocks,
      sel + ((size_t)b * heads + h) * nblocks);
  if (threadIdx.x == 0) counts[b * heads + h] = n;
}

}  // namespace

hipError_t launch_gate_from_sums(const float* bsum, const float* gate_w,
                                 const float* gate_b, float* scores,
                                 float* head_scores, int batch, int nblocks,
                                 int heads, int block, hipStream_t s) {
  const size_t lds = (size_t)(3 * heads * kD + heads) * sizeof(float);
  gate_from_sums_kernel<<<dim3(nblocks, batch), 256, lds, s>>>(
      bsum, gate_w, gate_b, scores, head_scores, heads,
      1.f / (float)(block * block));
  return hipGetLastError();
}

hipError_t launch_gate_scores(bool bf, const void* qkv_hat,
                              const float* gate_w, const float* gate_b,
                              const void* gate_dw, float* scores,
                              float* head_scores, int batch, int gh, int gw,
                              int heads, int block, hipStream_t s) {
  const int nblocks = (gh / block) * (gw / block);
  dim3 grid(nblocks, batch);
  const size_t lds = (size_t)(3 * heads * kD + heads) * sizeof(float);
  if (gate_dw) {
    const int total = nblocks * batch;
    const int per_xcd = (total + kXcds - 1) / kXcds;
    const int vecs = 3 * heads * kD / 4;
    const int threads = min(1024, (vecs + 63) / 64 * 64);
    if (bf)
      gate_scores_conv_kernel<bf16><<<per_xcd * kXcds, threads, lds, s>>>(
          static_cast<const bf16*>(qkv_hat), static_cast<const bf16*>(gate_dw),
          gate_w, gate_b, scores, head_scores, gh, gw, heads, block, nblocks,
          total, per_xcd);
    else
      gate_scores_conv_kernel<float><<<per_xcd * kXcds, threads, lds, s>>>(
          static_cast<const float*>(qkv_hat), static_cast<const float*>(gate_dw),
          gate_w, gate_b, scores, head_scores, gh, gw, heads, block, nblocks,
          total, per_xcd);
    return hipGetLastError();
  }
  if (bf)
    gate_scores_kernel<bf16><<<grid, 256, lds, s>>>(
        static_cast<const bf16*>(qkv_hat), gate_w, gate_b, scores, head_scores,
        gh, gw, heads, block);
  else
    gate_scores_kernel<float><<<grid, 256, lds, s>>>(
        static_cast<const float*>(qkv_hat), gate_w, gate_b, scores, head_scores,
        gh, gw, heads, block);
  return hipGetLastError();
}

size_t topk_parts_bytes(int nblocks) {
  int tpow = 2;
  while (tpow < nblocks) tpow <<= 1;
  return tpow <= 1024 ? (size_t)kRankParts * tpow * sizeof(int32_t) : 0;
}

hipError_t launch_topk(const float* scores, float* scores_copy, int32_t* sel,
                       int batch, int nblocks, int keep, hipStream_t s,
                       int32_t* parts) {
  if (keep == 0 && scores_copy == nullptr) return hipSuccess;
  int tpow = 2;
  while (tpow < nblocks) tpow <<= 1;
  if (parts && !scores_copy && tpow >= 16 * kRankParts && tpow <= 1024) {
    rank_part_kernel<false><<<dim3(kRankParts, batch), tpow, 0, s>>>(
        scores, parts, nblocks, tpow, nullptr, 0, 0.f, nullptr);
    rank_final_kernel<<<batch, 1024, 0, s>>>(parts, sel, nblocks, keep, tpow);
    return hipGetLastError();
  }
  const size_t lds = (size_t)tpow * sizeof(uint64_t);  // <= 64 KB for T <= 8192
  topk_kernel<<<batch, 1024, lds, s>>>(scores, scores_copy, sel, nblocks, keep,
                                       tpow);
  return hipGetLastError();
}

bool gate_topk_from_parts_ok(int nblocks) {
  int tpow = 2;
  while (tpow < nblocks) tpow <<= 1;
  return tpow >= 16 * kRankParts && tpow <= 1024;
}

hipError_t launch_gate_topk_parts(const float* plog, const float* gate_b, float* scores,
                                  int32_t* sel, int32_t* parts, int batch, int nblocks,
                                  int heads, int block, int keep, hipStream_t s) {
  if (!parts || !gate_topk_from_parts_ok(nblocks)) return hipErrorInvalidValue;
  int tpow = 2;
  while (tpow < nblocks) tpow <<= 1;
  if (tpow <= kDirectTopk) {
    gate_topk_direct_kernel<<<batch, 1024, 0, s>>>(plog, gate_b, scores, sel, nblocks, tpow,
                                                   heads, 1.f / (float)(block * block), keep);
    return hipGetLastError();
  }
  rank_part_kernel<true><<<dim3(kRankParts, batch), tpow, 0, s>>>(
      plog, parts, nblocks, tpow, gate_b, heads, 1.f / (float)(block * block), scores);
  rank_final_kernel<<<batch, 1024, 0, s>>>(parts, sel, nblocks, keep, tpow);
  return hipGetLastError();
}

hipError_t launch_gate_from_parts(const float* plog, const float* gate_b, float* scores,
                                  float* head_scores, int batch, int nblocks, int heads,
                                  int block, hipStream_t s) {
  const int total = batch * nblocks;
  if (total == 0) return hipSuccess;
  if (heads > 64) return hipErrorInvalidValue;  // 16 blocks x heads threads
  gate_from_parts_kernel<<<(total + 15) / 16, 16 * heads, 0, s>>>(
      plog, gate_b, scores, head_scores, total, heads, 1.f / (float)(block * block));
  return hipGetLastError();
}

hipError_t launch_threshold(const float* scores, float* scores_copy,
                            int32_t* sel, int32_t* counts, int batch,
                            int nblocks, float tau, hipStream_t s) {
  threshold_kernel<<<batch, 1024, 0, s>>>(scores, scores_copy, sel, counts,
                                          nblocks, tau);
  return hipGetLastError();
}

hipError_t launch_threshold_heads(const float* head_scores, float* copy,
                                  int32_t* sel, int32_t* counts, int batch,
                                  int nblocks, int heads, float tau,
                                  hipStream_t s) {
  threshold_heads_kernel<<<dim3(heads, batch), 1024, 0, s>>>(
      head_scores, copy, sel, counts, nblocks, heads, tau);
  return hipGetLastError();
}

}  // namespace hsmla
