// Local softmax refinement over the compacted block list with the two-path
// residual (FT 3.3 local-neighbourhood, lin-local and residual equations;
// FT 3.6 stages 4-5).  For a selected block t, head h and query i of t:
//
//   O_local_i   = sum_{j in W} softmax_j(q_i . k_j / sqrt(d)) v_j   (raw q,k,v)
//   O_linloc_i  = sum_{j in W} (phi(q^_i).phi(k^_j)) v^_j / sum_{j in W} phi(q^_i).phi(k^_j)
//   O_i        <- O_lin_i + O_local_i - O_linloc_i
//
// With per-block weights w (the training-time differentiable mixture of
// FT 3.3, w = M_b) every block is refined and the residual is scaled:
//   O_i        <- O_lin_i + w_b (O_local_i - O_linloc_i).
//
// W is the window x window square centred on the block, clipped to the grid.
// The lin-local ratio is evaluated in its pairwise form, which equals
// phi(q^) Z_W / phi(q^) D_W by associativity.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace hsmla {
namespace {

constexpr int kD = 32;
constexpr int kKT = 64;  // window keys staged per LDS tile

// grid (entries, batch, heads); one thread per query of the block.
template <typename T>
__global__ __launch_bounds__(256) void sparse_valu_kernel(
    const T* __restrict__ qkv, const T* __restrict__ qkvh,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ counts,
    const float* __restrict__ wts, T* __restrict__ o, int gh, int gw,
    int heads, int block, int window, SelLayout lay) {
  __shared__ float ks[kKT][kD];
  __shared__ float vs[kKT][kD];
  __shared__ float fks[kKT][kD];
  __shared__ float vhs[kKT][kD];
  const int b = blockIdx.y, h = blockIdx.z;
  const int C = heads * kD, C3 = 3 * C;
  if (counts && (int)blockIdx.x >= counts[b * lay.cnt_b + h * lay.cnt_h])
    return;  // beyond the routed set
  // without a list every block is refined (entry x is block x)
  const int t = sel ? sel[(size_t)b * lay.sel_b + (size_t)h * lay.sel_h + blockIdx.x]
                    : (int)blockIdx.x;
  const int nbc = gw / block;
  if (t < 0 || t >= (gh / block) * nbc) return;  // invalid entry: no access
  const int r0 = (t / nbc) * block, c0 = (t % nbc) * block;
  const int p = (window - block) / 2;
  const int rlo = max(0, r0 - p), rhi = min(gh, r0 + block + p);
  const int clo = max(0, c0 - p), chi = min(gw, c0 + block + p);
  const int wcols = chi - clo;
  const int nwin = (rhi - rlo) * wcols;
  const int nthr = blockDim.x;
  const int tid = threadIdx.x;
  const size_t img = (size_t)b * gh * gw;

  const int qn = (r0 + tid / block) * gw + c0 + tid % block;
  const T* qrow = qkv + (img + qn) * C3 + h * kD;
  const T* qhrow = qkvh + (img + qn) * C3 + h * kD;
  const float scale = 1.f / sqrtf((float)kD);
  float q[kD], fq[kD], acc[kD], num[kD];
#pragma unroll
  for (int j = 0; j < kD; ++j) {
    q[j] = to_f32(qrow[j]) * scale;
    fq[j] = relu(to_f32(qhrow[j]));
    acc[j] = 0.f;
    num[j] = 0.f;
  }
  float m = -INFINITY, l = 0.f, den = 0.f;

  for (int w0 = 0; w0 < nwin; w0 += kKT) {
    const int cnt = min(kKT, nwin - w0);
    for (int e = tid; e < cnt * kD; e += nthr) {
      const int r = e / kD, c = e % kD;
      const int wi = w0 + r;
      const size_t tok = img + (size_t)(rlo + wi / wcols) * gw + clo + wi % wcols;
      const T* row = qkv + tok * C3 + h * kD;
      const T* rowh = qkvh + tok * C3 + h * kD;
      ks[r][c] = to_f32(row[C + c]);
      vs[r][c] = to_f32(row[2 * C + c]);
      fks[r][c] = relu(to_f32(rowh[C + c]));
      vhs[r][c] = to_f32(rowh[2 * C + c]);
    }
    __syncthreads();
    for (int r = 0; r < cnt; ++r) {
      float s = 0.f, a = 0.f;
#pragma unroll
      for (int j = 0; j < kD; ++j) {
        s = fmaf(q[j], ks[r][j], s);
        a = fmaf(fq[j], fks[r][j], a);
      }
      const float mn = fmaxf(m, s);
      const float corr = expf(m - mn);
      const float pr = expf(s - mn);
      l = l * corr + pr;
#pragma unroll
      for (int j = 0; j < kD; ++j) {
        acc[j] = fmaf(pr, vs[r][j], acc[j] * corr);
        num[j] = fmaf(a, vhs[r][j], num[j]);
      }
      den += a;
      m = mn;
    }
    __syncthreads();
  }

  T* orow = o + (img + qn) * C + h * kD;
  const float inv_l = 1.f / l;
  const float inv_den = den > 0.f ? 1.f / den : 0.f;
  const float w = wts ? wts[(size_t)b * (gh / block) * nbc + t] : 1.f;
#pragma unroll
  for (int j = 0; j < kD; ++j) {
    const float lin = den > 0.f ? num[j] * inv_den : 0.f;
    const float v = wts ? fmaf(w, acc[j] * inv_l - lin, to_f32(orow[j]))
                        : to_f32(orow[j]) + acc[j] * inv_l - lin;
    orow[j] = from_f32<T>(v);
  }
}

// ---------------------------------------------------------------------------
// bfloat16 MFMA kernel
//
// Workgroup = one (selected block, head); 2 * nqt waves for nqt tiles of 32
// queries.  Wave w works on query tile w % nqt along one of two paths:
//   path 0 (softmax): S^T = K Q^T tile by tile, online softmax per query,
//                     O_local^T += V^T P^T;
//   path 1 (linear):  A^T = relu(K^) relu(Q^)^T, den += column sums,
//                     O_linloc^T += V^^T A^T.
// Every 32x32 accumulator tile holds one query per lane column, so row
// statistics of a query live in one lane pair (l, l ^ 32).  The P^T / A^T
// accumulator registers are fed back as the B operand of the next MFMA with
// the key order they already have; V and V^ are staged transposed in LDS in
// that same order.  Keys are streamed in tiles of 64 through double-buffered
// LDS.  Path 1 hands its normalised result to path 0 through LDS, and path 0
// writes O_lin + O_local - O_linloc.
// ---------------------------------------------------------------------------

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int KT = 64;            // keys per LDS tile
constexpr int KS = kD + 8;        // bf16 stride of key-major rows
constexpr int VS = KT + 8;        // bf16 stride of channel-major rows

struct __attribute__((aligned(16))) SparseTile {
  bf16 k[KT * KS];    // raw K,   [key][channel]
  bf16 kh[KT * KS];   // K_hat,   [key][channel]
  bf16 vt[kD * VS];   // raw V,   [channel][key]
  bf16 vht[kD * VS];  // V_hat,   [channel][key]
};

__device__ __forceinline__ uint16_t relu_bits(uint16_t u) {
  return (u & 0x8000u) ? 0 : u;  // bf16 max(x, 0); -0 and negatives -> +0
}

template <int NQT>
__global__ __launch_bounds__(64 * 2 * NQT) void sparse_mfma_kernel(
    const bf16* __restrict__ qkv, const bf16* __restrict__ qkvh,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ counts,
    const float* __restrict__ wts, bf16* __restrict__ o, int gh, int gw,
    int heads, int block, int window, SelLayout lay) {
  constexpr int NT = 64 * 2 * NQT;
  __shared__ SparseTile tiles[2];
  __shared__ float linloc[NQT * 32][kD + 1];

  const int b = blockIdx.y, h = blockIdx.z;
  const int C = heads * kD, C3 = 3 * C;
  if (counts && (int)blockIdx.x >= counts[b * lay.cnt_b + h * lay.cnt_h])
    return;  // beyond the routed set
  // without a list every block is refined (entry x is block x)
  const int t = sel ? sel[(size_t)b * lay.sel_b + (size_t)h * lay.sel_h + blockIdx.x]
                    : (int)blockIdx.x;
  const int nbc = gw / block;
  if (t < 0 || t >= (gh / block) * nbc) return;  // invalid entry: no access
  const int r0 = (t / nbc) * block, c0 = (t % nbc) * block;
  const int p = (window - block) / 2;
  const int rlo = max(0, r0 - p), rhi = min(gh, r0 + block + p);
  const int clo = max(0, c0 - p), chi = min(gw, c0 + block + p);
  const int wcols = chi - clo;
  const int nwin = (rhi - rlo) * wcols;
  const int nq = block * block;
  const size_t img = (size_t)b * gh * gw;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qt = wave % NQT, path = wave / NQT;
  const int g = lane >> 5;           // lane group (0/1)
  const int ql = qt * 32 + (lane & 31);  // query index within the block
  const bool q_ok = ql < nq;
  const int qn = q_ok ? (r0 + ql / block) * gw + c0 + ql % block : 0;

  // B operand of S^T: this lane's query, channels 8g..8g+7 and 16+8g..
  bf16x8 qf[2];
  {
    const bf16* src = (path == 0 ? qkv : qkvh) + (img + qn) * C3 + h * kD;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 u = q_ok ? *reinterpret_cast<const uint4*>(src + 16 * ks + 8 * g)
                     : uint4{0, 0, 0, 0};
      if (path == 1) {  // relu on the hatted query
        uint16_t* hv = reinterpret_cast<uint16_t*>(&u);
#pragma unroll
        for (int i = 0; i < 8; ++i) hv[i] = relu_bits(hv[i]);
      }
      qf[ks] = __builtin_bit_cast(bf16x8, u);
    }
  }

  // tile loader: 64 keys x (K, K^, V, V^) x 32 channels = 1024 chunks of 8.
  // Loads are unconditional (keys past the window re-read its last key and
  // are zeroed when staged), so no load sits under a branch and the wait
  // before staging covers exactly one tile.  Each thread's keys advance by
  // 64 window positions per tile, so their (row, column) in the window is
  // stepped instead of divided.
  constexpr int kLoads = (1024 + NT - 1) / NT;
  uint4 stg[kLoads];
  const int step_r = KT / wcols, step_c = KT % wcols;
  int kr[kLoads], kc[kLoads];  // window row / column of this thread's keys
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int key = (min(tid + NT * i, 1023) >> 2) & 63;
    kr[i] = key / wcols;
    kc[i] = key % wcols;
  }
  const size_t tok_last = img + (size_t)(rhi - 1) * gw + chi - 1;
  auto issue = [&](int w0) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int cidx = min(tid + NT * i, 1023);
      const int tensor = cidx >> 8;      // 0 K, 1 K^, 2 V, 3 V^
      const int key = (cidx >> 2) & 63, cg = cidx & 3;
      const size_t tok = w0 + key < nwin
                             ? img + (size_t)(rlo + kr[i]) * gw + clo + kc[i]
                             : tok_last;
      const bf16* base = (tensor & 1) ? qkvh : qkv;
      const int comp = (tensor < 2) ? 1 : 2;
      stg[i] = *reinterpret_cast<const uint4*>(base + tok * C3 + comp * C + h * kD + 8 * cg);
      // advance to the same key of the next tile
      kr[i] += step_r;
      kc[i] += step_c;
      if (kc[i] >= wcols) {
        kc[i] -= wcols;
        ++kr[i];
      }
    }
  };
  auto commit = [&](int buf, int w0) {
    SparseTile& T = tiles[buf];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int cidx = tid + NT * i;
      if (cidx >= 1024) break;
      const int tensor = cidx >> 8;
      const int key = (cidx >> 2) & 63, cg = cidx & 3;
      uint4 u = w0 + key < nwin ? stg[i] : uint4{0, 0, 0, 0};
      if (tensor == 0) {
        *reinterpret_cast<uint4*>(&T.k[key * KS + 8 * cg]) = u;
      } else if (tensor == 1) {
        uint16_t* hv = reinterpret_cast<uint16_t*>(&u);
#pragma unroll
        for (int j = 0; j < 8; ++j) hv[j] = relu_bits(hv[j]);
        *reinterpret_cast<uint4*>(&T.kh[key * KS + 8 * cg]) = u;
      } else {
        bf16* dst = tensor == 2 ? T.vt : T.vht;
        const uint16_t* hv = reinterpret_cast<const uint16_t*>(&u);
#pragma unroll
        for (int j = 0; j < 8; ++j) dst[(8 * cg + j) * VS + key].u = hv[j];
      }
    }
  };

  f32x16 oacc;
#pragma unroll
  for (int r = 0; r < 16; ++r) oacc[r] = 0.f;
  float run_max = -INFINITY;  // softmax path: running max (shared by l, l^32)
  float run_sum = 0.f;        // this lane's share of the column sum
  const float sc = 1.4426950408889634f / sqrtf((float)kD);  // log2(e)/sqrt(d)

  const int ntiles = (nwin + KT - 1) / KT;
  issue(0);
  commit(0, 0);
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    if (it + 1 < ntiles) issue((it + 1) * KT);
    const SparseTile& T = tiles[buf];
    const bf16* kmat = path == 0 ? T.k : T.kh;
    const bf16* vmat = path == 0 ? T.vt : T.vht;
#pragma unroll
    for (int sub = 0; sub < KT / 32; ++sub) {
      const int kbase = it * KT + sub * 32;
      if (kbase >= nwin) break;
      // S^T (or A^T) tile: rows = 32 keys, columns = 32 queries
      f32x16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 kf = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(
                        &kmat[(sub * 32 + (lane & 31)) * KS + 16 * ks + 8 * g]));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s, 0, 0, 0);
      }
      // lane holds keys kbase + 8(r/4) + 4g + r%4 of its query
      if (path == 0) {
        float mx = -INFINITY;
        if (kbase + 32 <= nwin) {  // a whole tile of keys (uniform)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            s[r] *= sc;
            mx = fmaxf(mx, s[r]);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kbase + 8 * (r >> 2) + 4 * g + (r & 3);
            s[r] = key < nwin ? s[r] * sc : -INFINITY;
            mx = fmaxf(mx, s[r]);
          }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mnew = fmaxf(run_max, mx);
        // arguments are <= 0: the hardware exp2 (results below 2^-126, i.e.
        // probabilities negligible against the row maximum's 1, flush to 0;
        // -inf gives 0) instead of the library's denormal-preserving form
        const float corr = __builtin_amdgcn_exp2f(run_max - mnew);
        run_max = mnew;
        float ps = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[r] = __builtin_amdgcn_exp2f(s[r] - mnew);
          ps += s[r];
        }
        run_sum = run_sum * corr + ps;
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[r] *= corr;
      } else {
        float ps = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) ps += s[r];
        run_sum += ps;
      }
      // O^T += V^T P^T over two 16-key slabs, keys in accumulator order
#pragma unroll
      for (int slab = 0; slab < 2; ++slab) {
        uint4 pb;
        pb.x = pack_bf16x2(s[8 * slab + 0], s[8 * slab + 1]);
        pb.y = pack_bf16x2(s[8 * slab + 2], s[8 * slab + 3]);
        pb.z = pack_bf16x2(s[8 * slab + 4], s[8 * slab + 5]);
        pb.w = pack_bf16x2(s[8 * slab + 6], s[8 * slab + 7]);
        const bf16* vrow = &vmat[(lane & 31) * VS + sub * 32 + 16 * slab + 4 * g];
        uint4 va;
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
        va.x = lo.x; va.y = lo.y; va.z = hi.x; va.w = hi.y;
        oacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, va), __builtin_bit_cast(bf16x8, pb), oacc,
            0, 0, 0);
      }
    }
    // tiles[buf ^ 1] was last read before the previous barrier
    if (it + 1 < ntiles) commit(buf ^ 1, (it + 1) * KT);
    __syncthreads();
  }

  // column totals over both lane groups
  const float total = run_sum + __shfl_xor(run_sum, 32, 64);
  // lane holds channels 8(r/4) + 4g + r%4 of query ql
  if (path == 1) {
    const float inv = total > 0.f ? 1.f / total : 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      linloc[ql][8 * (r >> 2) + 4 * g + (r & 3)] = total > 0.f ? oacc[r] * inv : 0.f;
  }
  __syncthreads();
  if (path == 0 && q_ok) {
    const float inv = 1.f / total;
    const float w = wts ? wts[(size_t)b * (gh / block) * nbc + t] : 1.f;
    bf16* orow = o + (img + qn) * C + h * kD;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ch = 8 * j + 4 * g;
      const uint2 prev = *reinterpret_cast<const uint2*>(orow + ch);
      float v[4];
      v[0] = __uint_as_float(prev.x << 16);
      v[1] = __uint_as_float(prev.x & 0xffff0000u);
      v[2] = __uint_as_float(prev.y << 16);
      v[3] = __uint_as_float(prev.y & 0xffff0000u);
      if (wts) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[i] = fmaf(w, oacc[4 * j + i] * inv - linloc[ql][ch + i], v[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] += oacc[4 * j + i] * inv - linloc[ql][ch + i];
      }
      uint2 outv;
      outv.x = pack_bf16x2(v[0], v[1]);
      outv.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(orow + ch) = outv;
    }
  }
}

template <typename T>
hipError_t run(const void* qkv, const void* qkvh, const int32_t* sel,
               const int32_t* counts, const float* wts, void* o, int batch,
               int gh, int gw, int heads, int block, int window, int entries,
               SelLayout lay, hipStream_t s) {
  dim3 grid(entries, batch, heads);
  sparse_valu_kernel<T><<<grid, block * block, 0, s>>>(
      static_cast<const T*>(qkv), static_cast<const T*>(qkvh), sel, counts, wts,
      static_cast<T*>(o), gh, gw, heads, block, window, lay);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse(bool bf, const void* qkv, const void* qkv_hat,
                         const int32_t* sel, const int32_t* counts,
                         const float* wts, void* o, int batch, int gh, int gw,
                         int heads, int block, int window, int entries,
                         SelLayout lay, hipStream_t s) {
  if (entries == 0) return hipSuccess;
  const int nqt = (block * block + 31) / 32;
  if (bf && nqt <= 4) {
    dim3 grid(entries, batch, heads);
    const bf16* q = static_cast<const bf16*>(qkv);
    const bf16* qh = static_cast<const bf16*>(qkv_hat);
    bf16* out = static_cast<bf16*>(o);
    switch (nqt) {
      case 1: sparse_mfma_kernel<1><<<grid, 128, 0, s>>>(q, qh, sel, counts, wts, out, gh, gw, heads, block, window, lay); break;
      case 2: sparse_mfma_kernel<2><<<grid, 256, 0, s>>>(q, qh, sel, counts, wts, out, gh, gw, heads, block, window, lay); break;
      case 3: sparse_mfma_kernel<3><<<grid, 384, 0, s>>>(q, qh, sel, counts, wts, out, gh, gw, heads, block, window, lay); break;
      default: sparse_mfma_kernel<4><<<grid, 512, 0, s>>>(q, qh, sel, counts, wts, out, gh, gw, heads, block, window, lay); break;
    }
    return hipGetLastError();
  }
  return bf ? run<bf16>(qkv, qkv_hat, sel, counts, wts, o, batch, gh, gw, heads,
                        block, window, entries, lay, s)
            : run<float>(qkv, qkv_hat, sel, counts, wts, o, batch, gh, gw, heads,
                         block, window, entries, lay, s);
}

}  // namespace hsmla
