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

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace hsmla {
namespace {

constexpr int kD = 32;
constexpr int kKT = 64;  // window keys staged per LDS tile
constexpr int kXcds = 8;
constexpr int kCusPerXcd = 32;
// resident workgroups per CU of the MFMA kernel (22.5 KB of LDS and one wave
// of at most 128 VGPRs per SIMD each)
constexpr int kSparseWgsPerCu = 4;

// grid (entries, batch, heads); block^2 x G threads: thread (q, g) =
// (tid % block^2, tid / block^2) takes query q and the window keys r with
// r % G == g, keeping its own online-softmax state; the G states of a query
// are merged at the end (maxima first, then the rescaled sums through LDS).
// G = 1 is one thread per query.  Splitting the keys shortens each thread's
// dependent chain of 32-term dot products G-fold: the kernel serves the
// float32 path and large bf16 blocks, whose launches are small.
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
  __shared__ float st_m[256], st_l[256], st_d[256];
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
  const int nq = block * block, G = nthr / nq;
  const int qi = tid % nq, g = tid / nq;
  const size_t img = (size_t)b * gh * gw;

  const int qn = (r0 + qi / block) * gw + c0 + qi % block;
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
    for (int r = g; r < cnt; r += G) {
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

  // merge the G states of each query (in g order): the maxima, then the
  // sums rescaled to the common maximum, the vectors through LDS (the key
  // tiles are free now)
  float L = l, Dn = den;
  if (G > 1) {
    st_m[tid] = m;
    st_l[tid] = l;
    st_d[tid] = den;
    __syncthreads();
    float mx = -INFINITY;
    for (int u = 0; u < G; ++u) mx = fmaxf(mx, st_m[qi + nq * u]);
    L = 0.f;
    Dn = 0.f;
    for (int u = 0; u < G; ++u) {
      const float mu = st_m[qi + nq * u];
      L += mu == -INFINITY ? 0.f : st_l[qi + nq * u] * expf(mu - mx);
      Dn += st_d[qi + nq * u];
    }
    const float c = m == -INFINITY ? 0.f : expf(m - mx);
    float* buf = &ks[0][0];  // 64 x 32 floats: 256 threads x 8, per pass
    static_assert(kKT * kD == 256 * 8, "merge buffer");
    // unrolled, so every register index is static
#pragma unroll
    for (int part = 0; part < 2 * kD / 8; ++part) {  // 8 of the 64 values per pass
      const bool is_num = part >= kD / 8;
      const int j0 = (part % (kD / 8)) * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        buf[tid * 8 + j] = is_num ? num[j0 + j] : acc[j0 + j] * c;
      __syncthreads();
      if (g == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float sm = 0.f;
          for (int u = 0; u < G; ++u) sm += buf[(qi + nq * u) * 8 + j];
          if (is_num)
            num[j0 + j] = sm;
          else
            acc[j0 + j] = sm;
        }
      }
      __syncthreads();
    }
  }
  if (g != 0) return;

  T* orow = o + (img + qn) * C + h * kD;
  const float inv_l = 1.f / L;
  const float inv_den = Dn > 0.f ? 1.f / Dn : 0.f;
  const float w = wts ? wts[(size_t)b * (gh / block) * nbc + t] : 1.f;
#pragma unroll
  for (int j = 0; j < kD; ++j) {
    const float lin = Dn > 0.f ? num[j] * inv_den : 0.f;
    const float v = wts ? fmaf(w, acc[j] * inv_l - lin, to_f32(orow[j]))
                        : to_f32(orow[j]) + acc[j] * inv_l - lin;
    orow[j] = from_f32<T>(v);
  }
}

// ---------------------------------------------------------------------------
// bfloat16 MFMA kernel
//
// A workgroup refines one (selected block, head) at a time (a grid of at
// most four workgroups per CU walks the work items, see the kernel); 2 *
// nqt waves for nqt tiles of 32 queries.  Wave w works on query tile
// w % nqt along one of two paths:
//   path 0 (softmax): S^T = K Q^T tile by tile, online softmax per query,
//                     O_local^T += V^T P^T;
//   path 1 (linear):  A^T = relu(K^) relu(Q^)^T, den += column sums,
//                     O_linloc^T += V^^T A^T.
// Every 32x32 accumulator tile holds one query per lane column, so row
// statistics of a query live in one lane pair (l, l ^ 32).  The P^T / A^T
// accumulator registers are fed back as the B operand of the next MFMA with
// the key order they already have; V and V^ are staged key-major in LDS (as
// they lie in HBM) and read as the A operand V^T in that same key order with
// gfx950's transposing LDS read (ds_read_b64_tr_b16: within each group of
// 16 lanes, lane j receives element j % 4 of the four 16-bit values that
// lane 4e + j / 4 addresses, e = 0..3; so when lane k addresses channels
// f0 + 4 (k % 4) .. + 3 of key t0 + k / 4, lane j receives channel f0 + j of
// keys t0 .. t0 + 3).  Keys are streamed in tiles of 32 through
// double-buffered LDS.  Path 1 hands its normalised result to path 0 through LDS, and path 0
// writes O_lin + O_local - O_linloc.
// ---------------------------------------------------------------------------

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// keys per LDS tile: 32 keys (two buffers, 22.5 KB) let four workgroups
// share a CU where 64 (45 KB) allowed three (measured on the block
// workload: keep 50% 102.3 -> 99.2 us, keep 10% unchanged)
constexpr int KT = 32;
constexpr int KS = kD + 8;        // bf16 stride of K rows (80 bytes)
constexpr int VS = kD + 16;       // bf16 stride of V rows (96 bytes: a transposing
                                  // read's four 32-byte pieces in distinct banks)

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

struct __attribute__((aligned(16))) SparseTile {
  bf16 k[KT * KS];    // raw K,   [key][channel]
  bf16 kh[KT * KS];   // K_hat,   [key][channel]
  bf16 v[KT * VS];    // raw V,   [key][channel]
  bf16 vh[KT * VS];   // V_hat,   [key][channel]
};

// bf16 max(x, 0) on two packed values: a packed 16-bit integer max with 0
// (a bf16 with the sign bit set is a negative int16; -0 and negatives -> +0)
typedef short s16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t relu_bf16x2(uint32_t u) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s16x2, u),
                                                                s16x2{0, 0}));
}
__device__ __forceinline__ uint4 relu_bf16x8(uint4 u) {
  return uint4{relu_bf16x2(u.x), relu_bf16x2(u.y), relu_bf16x2(u.z), relu_bf16x2(u.w)};
}

// The two-query-tile form (8x8 blocks, the workloads' shape) is compiled for
// five waves per SIMD (at most 102 VGPRs; the compiler spills a few values
// to scratch) so that five workgroups share a CU: on the block workload at
// keep 10%, 1248 work items then fit in one round of 1280 workgroups
// (28.1 -> 26.5 us; keep 50% unchanged).  The other forms keep four.  Two
// key tiles are in flight; the item's O_lin rows are read at its end (read
// with the queries, they cost the registers of the second tile: 26.7 ->
// 26.1 us at keep 10%, 98.1 -> 95.6 at keep 50%).
template <int NQT>
__global__ __launch_bounds__(64 * 2 * NQT)
__attribute__((amdgpu_waves_per_eu(NQT == 2 ? 5 : 4))) void sparse_mfma_kernel(
    const bf16* __restrict__ qkv, const bf16* __restrict__ qkvh,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ counts,
    const float* __restrict__ wts, bf16* __restrict__ o, int gh, int gw,
    int heads, int block, int window, SelLayout lay, int entries, int n_items,
    int per_xcd, int wgs_per_xcd) {
  constexpr int NT = 64 * 2 * NQT;
  __shared__ SparseTile tiles[2];
  // path 1's normalised result for path 0, written after the key loop has
  // ended (its last barrier passed): it reuses the tile buffers
  static_assert(sizeof(float) * NQT * 32 * (kD + 1) <= sizeof(SparseTile) * 2, "linloc fits");
  float (*linloc)[kD + 1] = reinterpret_cast<float (*)[kD + 1]>(&tiles[0]);

  // Work items (image b, list entry e, head h), walked by a grid of at most
  // four workgroups per CU; workgroup blockIdx.x runs on XCD
  // blockIdx.x % 8 and takes that XCD's local items lw, lw + wgs_per_xcd, ...
  // Fixed-length lists: each XCD takes a contiguous run of items numbered
  // with h fastest, so the heads of a block (which share the cache lines of
  // every window row) and the neighbouring selected blocks (whose windows
  // overlap) meet in that XCD's L2.  Counted lists (threshold routings),
  // whose valid entries are the first count of each list: the entries are
  // dealt to the XCDs in turn (entry e on XCD e % 8, its heads together), so
  // the routed work spreads over the whole chip, and a workgroup stops at
  // the largest count instead of every surplus entry taking a workgroup.
  const int xcd = blockIdx.x % kXcds, lw = blockIdx.x / kXcds;
  const int batch = n_items / (entries * heads);
  const int C = heads * kD, C3 = 3 * C;
  const int nbc = gw / block;
  int max_cnt = entries;
  if (counts) {
    max_cnt = 0;
    for (int b = 0; b < batch; ++b)
      for (int h = 0; h < (lay.cnt_h ? heads : 1); ++h)
        max_cnt = max(max_cnt, counts[b * lay.cnt_b + h * lay.cnt_h]);
    max_cnt = min(max_cnt, entries);
  }
  for (int j = lw;; j += wgs_per_xcd) {
    int h, e, b;
    if (counts) {
      h = j % heads;
      b = (j / heads) % batch;
      e = (j / heads / batch) * kXcds + xcd;
      if (e >= max_cnt) break;
    } else {
      const int item = xcd * per_xcd + j;
      if (j >= per_xcd || item >= n_items) break;
      h = item % heads;
      e = (item / heads) % entries;
      b = item / heads / entries;
    }
    if (counts && e >= counts[b * lay.cnt_b + h * lay.cnt_h])
      continue;  // beyond the routed set
    // without a list every block is refined (entry x is block x)
    const int t = sel ? sel[(size_t)b * lay.sel_b + (size_t)h * lay.sel_h + e] : e;
    if (t < 0 || t >= (gh / block) * nbc) continue;  // invalid entry: no access
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
        if (path == 1) u = relu_bf16x8(u);  // relu on the hatted query
        qf[ks] = __builtin_bit_cast(bf16x8, u);
      }
    }

    // tile loader: KT keys x (K, K^, V, V^) x 32 channels = 16 KT chunks of 8.
    // Loads are unconditional (keys past the window re-read its last key and
    // are zeroed when staged), so no load sits under a branch and the wait
    // before staging covers exactly one tile.  Each chunk keeps a pointer to
    // its tensor's head slice in the image and the 32-bit element offset of its
    // key's token, both formed once: a tile advances every key by KT window
    // positions, i.e. a fixed offset step plus one row's wrap when its column
    // passes the window's edge (the launcher keeps an image's offsets below
    // 2^31 elements).
    constexpr int kChunks = KT * 16;  // KT keys x 4 tensors x 4 chunks of 8
    constexpr int kLoads = (kChunks + NT - 1) / NT;
    __builtin_assume(tid < NT);
    uint4 stg[2][kLoads];  // two tiles in flight: tile t in set t % 2
    const int step_r = KT / wcols, step_c = KT % wcols;
    const uint32_t d_off = (uint32_t)((step_r * gw + step_c) * C3);
    const uint32_t wrap_off = (uint32_t)((gw - wcols) * C3);
    const uint32_t off_last = (uint32_t)(((rhi - 1) * gw + chi - 1) * C3);
    int kc[kLoads];            // window column of this thread's keys
    uint32_t koff[kLoads];     // element offset of their token in the image
    const bf16* kptr[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int cidx = min(tid + NT * i, kChunks - 1);
      const int tensor = cidx / (KT * 4);  // 0 K, 1 K^, 2 V, 3 V^
      const int key = (cidx >> 2) % KT, cg = cidx & 3;
      const int kr = key / wcols;
      kc[i] = key % wcols;
      koff[i] = (uint32_t)(((rlo + kr) * gw + clo + kc[i]) * C3);
      kptr[i] = ((tensor & 1) ? qkvh : qkv) + img * C3 + (tensor < 2 ? 1 : 2) * C + h * kD + 8 * cg;
    }
    auto issue = [&](auto set_c, int w0) {
      constexpr int set = decltype(set_c)::value;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int key = (min(tid + NT * i, kChunks - 1) >> 2) % KT;
        stg[set][i] = *reinterpret_cast<const uint4*>(kptr[i] + (w0 + key < nwin ? koff[i] : off_last));
        // advance to the same key of the next tile
        koff[i] += d_off;
        kc[i] += step_c;
        if (kc[i] >= wcols) {
          kc[i] -= wcols;
          koff[i] += wrap_off;
        }
      }
    };
    auto commit = [&](auto set_c, int buf, int w0) {
      constexpr int set = decltype(set_c)::value;
      SparseTile& T = tiles[buf];
      const bool whole = w0 + KT <= nwin;  // uniform: no key past the window
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int cidx = tid + NT * i;
        if (cidx >= kChunks) break;
        const int tensor = cidx / (KT * 4);
        const int key = (cidx >> 2) % KT, cg = cidx & 3;
        uint4 u = stg[set][i];
        if (!whole && w0 + key >= nwin) u = uint4{0, 0, 0, 0};
        if (tensor == 0) {
          *reinterpret_cast<uint4*>(&T.k[key * KS + 8 * cg]) = u;
        } else if (tensor == 1) {
          *reinterpret_cast<uint4*>(&T.kh[key * KS + 8 * cg]) = relu_bf16x8(u);
        } else {
          bf16* dst = tensor == 2 ? T.v : T.vh;
          *reinterpret_cast<uint4*>(&dst[key * VS + 8 * cg]) = u;
        }
      }
    };

    f32x16 oacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[r] = 0.f;
    float run_max = -INFINITY;  // softmax path: running max (shared by l, l^32)
    float run_sum = 0.f;        // this lane's share of the column sum
    const float sc = 1.4426950408889634f / sqrtf((float)kD);  // log2(e)/sqrt(d)

    // Two tiles in flight: while tile it is computed from LDS buffer it % 2,
    // tiles it + 1 and it + 2 load into the two register sets; after the
    // compute, tile it + 1 is staged into the other buffer and tile it + 3
    // issued into the set it leaves.  Issues past the window re-read its
    // last key (in bounds, never staged), so none sits under a branch.
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    const int ntiles = (nwin + KT - 1) / KT;
    issue(S0{}, 0);
    issue(S1{}, KT);
    commit(S0{}, 0, 0);
    issue(S0{}, 2 * KT);
    __syncthreads();
    auto step = [&](auto par_c, int it) {
      constexpr int par = decltype(par_c)::value;  // it % 2
      using Next = std::integral_constant<int, 1 - par>;
      const int buf = par;
      const SparseTile& T = tiles[buf];
      const bf16* kmat = path == 0 ? T.k : T.kh;
      const bf16* vmat = path == 0 ? T.v : T.vh;
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
          // the maximum of the raw scores, scaled once (sc > 0, and rounding
          // is monotonic, so this is the maximum of the scaled scores)
          float mx = -INFINITY;
          if (kbase + 32 <= nwin) {  // a whole tile of keys (uniform)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kbase + 8 * (r >> 2) + 4 * g + (r & 3);
              s[r] = key < nwin ? s[r] : -INFINITY;
              mx = fmaxf(mx, s[r]);
            }
          }
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * sc;
          const float mnew = fmaxf(run_max, mx);
          // arguments are <= 0: the hardware exp2 (results below 2^-126, i.e.
          // probabilities negligible against the row maximum's 1, flush to 0;
          // -inf gives 0) instead of the library's denormal-preserving form
          const float corr = __builtin_amdgcn_exp2f(run_max - mnew);
          run_max = mnew;
          float ps = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], sc, -mnew));
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
          // V^T operand: channel lane % 32, keys sub*32 + 16 slab + 4 g + 0..3
          // and + 8 .. + 11 (two transposing reads, see above)
          const bf16* vrow = &vmat[(sub * 32 + 16 * slab + 4 * g + ((lane & 15) >> 2)) * VS +
                                   16 * ((lane >> 4) & 1) + 4 * (lane & 3)];
          const uint2 lo = __builtin_bit_cast(
              uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_char*)vrow));
          const uint2 hi = __builtin_bit_cast(
              uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_char*)(vrow + 8 * VS)));
          uint4 va;
          va.x = lo.x; va.y = lo.y; va.z = hi.x; va.w = hi.y;
          oacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, va), __builtin_bit_cast(bf16x8, pb), oacc,
              0, 0, 0);
        }
      }
      // tiles[buf ^ 1] was last read before the previous barrier
      if (it + 1 < ntiles) commit(Next{}, buf ^ 1, (it + 1) * KT);
      issue(Next{}, (it + 3) * KT);
      __syncthreads();
    };
    // in pairs, so that the register sets are static; a step past the last
    // tile computes and stages nothing
    for (int it = 0; it < ntiles; it += 2) {
      step(S0{}, it);
      step(S1{}, it + 1);
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
        const uint2 pv = *reinterpret_cast<const uint2*>(orow + ch);
        float v[4];
        v[0] = __uint_as_float(pv.x << 16);
        v[1] = __uint_as_float(pv.x & 0xffff0000u);
        v[2] = __uint_as_float(pv.y << 16);
        v[3] = __uint_as_float(pv.y & 0xffff0000u);
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
    // the next item stages its first key tile over linloc
    __syncthreads();
  }
}

template <typename T>
hipError_t run(const void* qkv, const void* qkvh, const int32_t* sel,
               const int32_t* counts, const float* wts, void* o, int batch,
               int gh, int gw, int heads, int block, int window, int entries,
               SelLayout lay, hipStream_t s) {
  dim3 grid(entries, batch, heads);
  // key groups per query: as many as fit 256 threads, at most 16 (a
  // power of two, so that block^2 x G divides into whole merge passes)
  const int nq = block * block;
  int G = 1;
  while (G < 16 && nq * G * 2 <= 256) G *= 2;
  sparse_valu_kernel<T><<<grid, nq * G, 0, s>>>(
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
  // the MFMA kernel forms an image's token offsets in 32 bits
  if (bf && nqt <= 4 && (int64_t)gh * gw * 3 * heads * kD < INT32_MAX) {
    if ((int64_t)entries * batch * heads > INT32_MAX / 2) return hipErrorInvalidValue;
    const int total = entries * batch * heads;
    const int per_xcd = (total + kXcds - 1) / kXcds;
    // local items per XCD: a contiguous run, or (counted lists) the entries
    // e = xcd, xcd + 8, ... of every (image, head)
    const int local = counts ? (entries + kXcds - 1) / kXcds * batch * heads : per_xcd;
    const int per_cu = nqt == 2 ? kSparseWgsPerCu + 1 : kSparseWgsPerCu;
    const int wgs_per_xcd = std::min(local, per_cu * kCusPerXcd);
    const dim3 grid(wgs_per_xcd * kXcds);
    const bf16* q = static_cast<const bf16*>(qkv);
    const bf16* qh = static_cast<const bf16*>(qkv_hat);
    bf16* out = static_cast<bf16*>(o);
    switch (nqt) {
      case 1: sparse_mfma_kernel<1><<<grid, 128, 0, s>>>(q, qh, sel, counts, wts, out, gh, gw, heads, block, window, lay, entries, total, per_xcd, wgs_per_xcd); break;
      case 2: sparse_mfma_kernel<2><<<grid, 256, 0, s>>>(q, qh, sel, counts, wts, out, gh, gw, heads, block, window, lay, entries, total, per_xcd, wgs_per_xcd); break;
      case 3: sparse_mfma_kernel<3><<<grid, 384, 0, s>>>(q, qh, sel, counts, wts, out, gh, gw, heads, block, window, lay, entries, total, per_xcd, wgs_per_xcd); break;
      default: sparse_mfma_kernel<4><<<grid, 512, 0, s>>>(q, qh, sel, counts, wts, out, gh, gw, heads, block, window, lay, entries, total, per_xcd, wgs_per_xcd); break;
    }
    return hipGetLastError();
  }
  return bf ? run<bf16>(qkv, qkv_hat, sel, counts, wts, o, batch, gh, gw, heads,
                        block, window, entries, lay, s)
            : run<float>(qkv, qkv_hat, sel, counts, wts, o, batch, gh, gw, heads,
                         block, window, entries, lay, s);
}

}  // namespace hsmla
