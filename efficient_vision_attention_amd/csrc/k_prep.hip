// Preparation of constant operands, in one launch: the folded depthwise tap
// sets and the projection weights in the layout the GEMM reads.
//
// Folded taps (abstract and EX section 2: the identity plus depthwise
// kernels of several sizes; FT 3.5 block equation for the FFN's 3x3): every
// branch is linear, so weff[tap][c] = identity (centre tap, when set) + the
// sum of the branch kernels zero-padded to kmax x kmax, in branch order.
//
// Weights: a projection y = x . W takes W as [in][out] row-major; the GEMM
// reads eight consecutive input channels of one output column per lane, so
// the copy is the transpose [out][in], stored row-major or tile-blocked
// (one K step of one tile as one contiguous block, see launch_gemm).  Both
// are plain permutations of the elements.
#include "common.h"
#include "kernels.h"

namespace hsmla {
namespace {

constexpr int kMaxTapSets = 2;
constexpr int kMaxBlockJobs = 4;

struct TapSet {
  const void* p[3];
  int k[3];
  int nk, kmax, ch, identity;
  float* weff;
};

struct PrepArgs {
  TapSet taps[kMaxTapSets];
  BlockJob jobs[kMaxBlockJobs];
  int ntaps, njobs;
  int tap_end[kMaxTapSets];   // running thread counts
  int job_end[kMaxBlockJobs];
};

template <typename T>
__device__ void fold_tap(const TapSet& ks, int idx) {
  const int kmax = ks.kmax, ch = ks.ch;
  const int c = idx % ch, tap = idx / ch;
  const int dy = tap / kmax, dx = tap % kmax;
  const int rmax = (kmax - 1) / 2;
  float v = (ks.identity && dy == rmax && dx == rmax) ? 1.f : 0.f;
  for (int i = 0; i < ks.nk; ++i) {
    const int k = ks.k[i], r = (k - 1) / 2;
    const int ky = dy - rmax + r, kx = dx - rmax + r;
    if (ky >= 0 && ky < k && kx >= 0 && kx < k)
      v += to_f32(static_cast<const T*>(ks.p[i])[((size_t)c * k + ky) * k + kx]);
  }
  ks.weff[idx] = v;
}

// Eight consecutive input channels k0..k0+7 of output column n of the
// transposed copy per thread; consecutive threads take consecutive n, so
// each of the eight source reads is one contiguous run across the wave.
template <typename T>
__device__ void weight_chunk(const BlockJob& j, int idx) {
  const int n = idx % j.rows, k0 = (idx / j.rows) * 8;
  const T* src = static_cast<const T*>(j.src) + (size_t)k0 * j.rows + n;
  T v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = src[(size_t)i * j.rows];
  const size_t dst =
      j.tile_rows ? ((size_t)(n / j.tile_rows) * (j.cols / kGemmTileK) + k0 / kGemmTileK) *
                            ((size_t)j.tile_rows * kGemmTileK) +
                        (size_t)(n % j.tile_rows) * kGemmTileK + k0 % kGemmTileK
                  : (size_t)n * j.cols + k0;
  T* d = static_cast<T*>(j.dst) + dst;
#pragma unroll
  for (int i = 0; i < 8; ++i) d[i] = v[i];
}

// Threads [0, tap_end[0]) fold the first tap set, the next range the
// second, then the block jobs in order.
template <typename T>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
  int idx = blockIdx.x * blockDim.x + threadIdx.x;
  int base = 0;
  for (int t = 0; t < a.ntaps; ++t) {
    if (idx < a.tap_end[t]) {
      fold_tap<T>(a.taps[t], idx - base);
      return;
    }
    base = a.tap_end[t];
  }
  for (int t = 0; t < a.njobs; ++t) {
    if (idx < a.job_end[t]) {
      weight_chunk<T>(a.jobs[t], idx - base);
      return;
    }
    base = a.job_end[t];
  }
}

}  // namespace

hipError_t launch_prep(bool bf, const TapSpec* taps, int ntaps,
                       const BlockJob* jobs, int njobs, hipStream_t s) {
  if (ntaps > kMaxTapSets || njobs > kMaxBlockJobs) return hipErrorInvalidValue;
  PrepArgs a{};
  int total = 0;
  for (int t = 0; t < ntaps; ++t) {
    TapSet& ts = a.taps[t];
    for (int i = 0; i < taps[t].nk; ++i) {
      ts.p[i] = taps[t].kernels[i];
      ts.k[i] = taps[t].ks[i];
    }
    ts.nk = taps[t].nk;
    ts.kmax = taps[t].kmax;
    ts.ch = taps[t].ch;
    ts.identity = taps[t].identity;
    ts.weff = taps[t].weff;
    total += ts.kmax * ts.kmax * ts.ch;
    a.tap_end[t] = total;
  }
  for (int t = 0; t < njobs; ++t) {
    if (jobs[t].cols % (jobs[t].tile_rows ? kGemmTileK : 8) ||
        (jobs[t].tile_rows && (!bf || jobs[t].rows % jobs[t].tile_rows)))
      return hipErrorInvalidValue;
    a.jobs[t] = jobs[t];
    total += jobs[t].rows * (jobs[t].cols / 8);
    a.job_end[t] = total;
  }
  a.ntaps = ntaps;
  a.njobs = njobs;
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (bf)
    prep_kernel<bf16><<<blocks, 256, 0, s>>>(a);
  else
    prep_kernel<float><<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_dw_taps(bool bf, const void* const* kernels, const int* ks,
                          int nk, int kmax, int ch, int identity, float* weff,
                          hipStream_t s) {
  TapSpec t{{nullptr, nullptr, nullptr}, {0, 0, 0}, nk, kmax, ch, identity, weff};
  for (int i = 0; i < nk; ++i) {
    t.kernels[i] = kernels[i];
    t.ks[i] = ks[i];
  }
  return launch_prep(bf, &t, 1, nullptr, 0, s);
}

}  // namespace hsmla
