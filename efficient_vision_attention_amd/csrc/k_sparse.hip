// Local softmax refinement over the compacted block list with the two-path
// residual (FT 3.3 local-neighbourhood, lin-local and residual equations;
// FT 3.6 stages 4-5).  For a selected block t, head h and query i of t:
//
//   O_local_i   = sum_{j in W} softmax_j(q_i . k_j / sqrt(d)) v_j   (raw q,k,v)
//   O_linloc_i  = sum_{j in W} (phi(q^_i).phi(k^_j)) v^_j / sum_{j in W} phi(q^_i).phi(k^_j)
//   O_i        <- O_lin_i + O_local_i - O_linloc_i
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

// grid (keep, batch, heads); one thread per query of the block.
template <typename T>
__global__ __launch_bounds__(256) void sparse_valu_kernel(
    const T* __restrict__ qkv, const T* __restrict__ qkvh,
    const int32_t* __restrict__ sel, T* __restrict__ o, int gh, int gw,
    int heads, int block, int window, int keep) {
  __shared__ float ks[kKT][kD];
  __shared__ float vs[kKT][kD];
  __shared__ float fks[kKT][kD];
  __shared__ float vhs[kKT][kD];
  const int b = blockIdx.y, h = blockIdx.z;
  const int C = heads * kD, C3 = 3 * C;
  const int t = sel[(size_t)b * keep + blockIdx.x];
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
#pragma unroll
  for (int j = 0; j < kD; ++j) {
    const float lin = den > 0.f ? num[j] * inv_den : 0.f;
    const float v = to_f32(orow[j]) + acc[j] * inv_l - lin;
    orow[j] = from_f32<T>(v);
  }
}

template <typename T>
hipError_t run(const void* qkv, const void* qkvh, const int32_t* sel, void* o,
               int batch, int gh, int gw, int heads, int block, int window,
               int keep, hipStream_t s) {
  dim3 grid(keep, batch, heads);
  sparse_valu_kernel<T><<<grid, block * block, 0, s>>>(
      static_cast<const T*>(qkv), static_cast<const T*>(qkvh), sel,
      static_cast<T*>(o), gh, gw, heads, block, window, keep);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse(bool bf, const void* qkv, const void* qkv_hat,
                         const int32_t* sel, void* o, int batch, int gh,
                         int gw, int heads, int block, int window, int keep,
                         hipStream_t s) {
  if (keep == 0) return hipSuccess;
  return bf ? run<bf16>(qkv, qkv_hat, sel, o, batch, gh, gw, heads, block,
                        window, keep, s)
            : run<float>(qkv, qkv_hat, sel, o, batch, gh, gw, heads, block,
                         window, keep, s);
}

}  // namespace hsmla
