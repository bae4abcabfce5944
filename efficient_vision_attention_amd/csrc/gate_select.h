// Top-k selection pieces shared by the gate's own launches (k_gate.hip) and
// by the K/V-state launch that ranks the gate's scores beside its partial
// sums (k_linear.hip): the order-preserving 64-bit block key, the block
// score formed from the gate's partial logits, the workgroup-wide ascending
// compaction, and the two phases of a top-k by exact rank counts.
// FT 3.2 (block-level aggregation of the head scores; the top fraction of
// blocks routed to the softmax path).
#pragma once

#include <math.h>

#include "common.h"

namespace hsmla {
namespace {

// The score mapped to an order-preserving unsigned integer (-0 taken as +0)
// in the high word and the complement of the block index in the low word:
// keys are distinct, and key_u > key_t exactly when s_u > s_t or (s_u == s_t
// and u < t), so ranking by keys sends equal scores to the lower index.
__device__ __forceinline__ uint64_t topk_key(float v, int t) {
  uint32_t u = __float_as_uint(v + 0.f);  // -0 -> +0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(u) << 32) | (0xffffffffu - static_cast<uint32_t>(t));
}

// M_t = mean_h sigmoid((P_0 + P_1 + P_2) inv_cnt + b_h) from the gate's
// partial logits P[s][h] of one block (s = Q^, K^, V^ component), the
// heads added in head order.
__device__ __forceinline__ float score_from_parts(const float* __restrict__ P,
                                                  const float* __restrict__ gb, int heads,
                                                  float inv_cnt) {
  float m = 0.f;
  if (heads % 4 == 0) {  // 16-byte loads of the three rows (16-byte aligned)
    for (int h = 0; h < heads; h += 4) {
      const float4 a = *reinterpret_cast<const float4*>(P + h);
      const float4 k = *reinterpret_cast<const float4*>(P + heads + h);
      const float4 v = *reinterpret_cast<const float4*>(P + 2 * heads + h);
      const float pa[4] = {a.x, a.y, a.z, a.w}, pk[4] = {k.x, k.y, k.z, k.w},
                  pv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float p = ((pa[q] + pk[q]) + pv[q]) * inv_cnt;
        m += 1.f / (1.f + expf(-(p + gb[h + q])));
      }
    }
  } else {
    for (int h = 0; h < heads; ++h) {
      const float p = ((P[h] + P[heads + h]) + P[2 * heads + h]) * inv_cnt;
      m += 1.f / (1.f + expf(-(p + gb[h])));
    }
  }
  return m / (float)heads;
}

// Workgroup-wide stream compaction (any multiple of 64 threads up to
// 1024): writes every t in [0, n) with keep(t) to out[0 ..) in ascending
// order and returns the number written (same value in every thread).  The
// slot of a kept t is the number of kept entries below it: a wave ballot
// gives the rank inside the wave, a prefix over the wave totals the offset
// of the wave.
template <typename Pred>
__device__ int compact_ascending(Pred keep, int n, int32_t* __restrict__ out) {
  __shared__ int wave_tot[16];
  __shared__ int base_all;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  if (threadIdx.x == 0) base_all = 0;
  __syncthreads();
  for (int t0 = 0; t0 < n; t0 += blockDim.x) {
    const int t = t0 + threadIdx.x;
    const bool k = t < n && keep(t);
    const uint64_t m = __ballot(k);
    const int below = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wave_tot[wave] = __popcll(m);
    __syncthreads();
    int off = base_all;
    for (int w2 = 0; w2 < wave; ++w2) off += wave_tot[w2];
    if (k) out[off + below] = t;
    __syncthreads();
    if (threadIdx.x == 0) {
      int tot = 0;
      for (int w2 = 0; w2 < nwaves; ++w2) tot += wave_tot[w2];
      base_all += tot;
    }
    __syncthreads();
  }
  return base_all;
}

// Ranks over several workgroups per image (up to 1024 blocks): the key
// range [0, tpow) is split into kRankParts runs of tpow / kRankParts keys.
constexpr int kRankParts = 8;

// Workgroup s of image b (any multiple of 64 threads up to 1024): for every
// block t of the image, the number of keys of run s above key_t, written to
// part[b][s][t].  With FROM_PARTS the scores are formed from the gate's
// partial logits (plog[b][t][s][h], written by the S2 conv) and workgroup 0
// of each image stores them to scores_out; otherwise they are read from
// scores.  keys holds tpow / kRankParts keys.  The counts are exact
// integers: the ranks their sums give equal those of any other count.
template <bool FROM_PARTS>
__device__ void rank_part_wg(const float* __restrict__ scores, int32_t* __restrict__ part,
                             int nblocks, int tpow, const float* __restrict__ gb, int heads,
                             float inv_cnt, float* __restrict__ scores_out, int s, int b,
                             uint64_t* keys) {
  const int len = tpow / kRankParts;
  auto score = [&](int u) {
    if constexpr (FROM_PARTS)
      return score_from_parts(scores + ((size_t)b * nblocks + u) * 3 * heads, gb, heads,
                              inv_cnt);
    else
      return scores[(size_t)b * nblocks + u];
  };
  for (int i = threadIdx.x; i < len; i += blockDim.x) {
    const int u = s * len + i;
    keys[i] = u < nblocks ? topk_key(score(u), u) : 0;
  }
  __syncthreads();
  for (int t = threadIdx.x; t < nblocks; t += blockDim.x) {
    const float st = score(t);
    if (FROM_PARTS && s == 0) scores_out[(size_t)b * nblocks + t] = st;
    const uint64_t kt = topk_key(st, t);
    int cnt = 0;
    for (int i = 0; i < len; i += 16) {  // len is a multiple of 16
      uint64_t v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = keys[i + q];
#pragma unroll
      for (int q = 0; q < 16; ++q) cnt += v[q] > kt;
    }
    part[((size_t)b * kRankParts + s) * tpow + t] = cnt;
  }
}

// One workgroup per image (any multiple of 64 threads up to 1024): rank(t)
// = the sum of the runs' counts, then the blocks of rank below keep to
// sel[b][0 .. keep) in ascending order.  rank holds nblocks ints.
__device__ void rank_final_wg(const int32_t* __restrict__ part, int32_t* __restrict__ sel,
                              int nblocks, int keep, int tpow, int b, int* rank) {
  for (int t = threadIdx.x; t < nblocks; t += blockDim.x) {
    int r = 0;
#pragma unroll
    for (int q = 0; q < kRankParts; ++q) r += part[((size_t)b * kRankParts + q) * tpow + t];
    rank[t] = r;
  }
  __syncthreads();
  compact_ascending([&](int u) { return rank[u] < keep; }, nblocks, sel + (size_t)b * keep);
}

}  // namespace
}  // namespace hsmla
