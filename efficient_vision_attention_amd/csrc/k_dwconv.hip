// Depthwise convolutions on the NHWC token grid.
//
// Multi-scale branches: T_hat = T + sum_s DWConv_{k_s}(T) for every channel
// of Q, K and V (abstract and EX section 2: depthwise kernels of several
// sizes enrich the tokens).  Because every branch is linear in T, the
// identity and all branches are folded into one kmax x kmax tap set per
// channel before the convolution runs.  The FFN's 3x3 depthwise conv (FT 3.5
// block equation) uses the same kernel with a GELU epilogue.
#include "common.h"
#include "kernels.h"

namespace hsmla {
namespace {

struct KernelSet {
  const void* p[3];
  int k[3];
};

template <typename T>
__global__ void dw_taps_kernel(KernelSet ks, int nk, int kmax, int ch,
                               int identity, float* __restrict__ weff) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= ch) return;
  const int rmax = (kmax - 1) / 2;
  for (int dy = 0; dy < kmax; ++dy) {
    for (int dx = 0; dx < kmax; ++dx) {
      float v = (identity && dy == rmax && dx == rmax) ? 1.f : 0.f;
      for (int i = 0; i < nk; ++i) {
        const int k = ks.k[i], r = (k - 1) / 2;
        const int ky = dy - rmax + r, kx = dx - rmax + r;
        if (ky >= 0 && ky < k && kx >= 0 && kx < k)
          v += to_f32(static_cast<const T*>(ks.p[i])[((size_t)c * k + ky) * k + kx]);
      }
      weff[(size_t)(dy * kmax + dx) * ch + c] = v;
    }
  }
}

__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.f + erff(x * 0.70710678118654752f));
}

// One thread per output element, channels fastest (coalesced).
template <typename T, bool GELU>
__global__ __launch_bounds__(256) void dwconv_simple(
    const T* __restrict__ in, T* __restrict__ out,
    const float* __restrict__ weff, int kmax, int batch, int gh, int gw,
    int ch) {
  const size_t total = (size_t)batch * gh * gw * ch;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int c = idx % ch;
  size_t rest = idx / ch;
  const int x = rest % gw;
  rest /= gw;
  const int y = rest % gh;
  const int b = rest / gh;
  const int r = (kmax - 1) / 2;
  float acc = 0.f;
  for (int dy = 0; dy < kmax; ++dy) {
    const int yy = y + dy - r;
    if (yy < 0 || yy >= gh) continue;
    for (int dx = 0; dx < kmax; ++dx) {
      const int xx = x + dx - r;
      if (xx < 0 || xx >= gw) continue;
      acc = fmaf(weff[(size_t)(dy * kmax + dx) * ch + c],
                 to_f32(in[(((size_t)b * gh + yy) * gw + xx) * ch + c]), acc);
    }
  }
  if (GELU) acc = gelu_erf(acc);
  out[idx] = from_f32<T>(acc);
}

template <typename T, bool GELU>
hipError_t run_dw(const void* in, void* out, const float* weff, int kmax,
                  int batch, int gh, int gw, int ch, hipStream_t s) {
  const size_t total = (size_t)batch * gh * gw * ch;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  dwconv_simple<T, GELU><<<blocks, 256, 0, s>>>(
      static_cast<const T*>(in), static_cast<T*>(out), weff, kmax, batch, gh,
      gw, ch);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dw_taps(bool bf, const void* const* kernels, const int* ks,
                          int nk, int kmax, int ch, int identity, float* weff,
                          hipStream_t s) {
  KernelSet set{};
  for (int i = 0; i < nk; ++i) {
    set.p[i] = kernels[i];
    set.k[i] = ks[i];
  }
  const unsigned blocks = (unsigned)((ch + 255) / 256);
  if (bf)
    dw_taps_kernel<bf16><<<blocks, 256, 0, s>>>(set, nk, kmax, ch, identity, weff);
  else
    dw_taps_kernel<float><<<blocks, 256, 0, s>>>(set, nk, kmax, ch, identity, weff);
  return hipGetLastError();
}

hipError_t launch_dwconv(bool bf, const void* in, void* out, const float* weff,
                         int kmax, int batch, int gh, int gw, int ch,
                         bool gelu, hipStream_t s) {
  if (bf)
    return gelu ? run_dw<bf16, true>(in, out, weff, kmax, batch, gh, gw, ch, s)
                : run_dw<bf16, false>(in, out, weff, kmax, batch, gh, gw, ch, s);
  return gelu ? run_dw<float, true>(in, out, weff, kmax, batch, gh, gw, ch, s)
              : run_dw<float, false>(in, out, weff, kmax, batch, gh, gw, ch, s);
}

}  // namespace hsmla
