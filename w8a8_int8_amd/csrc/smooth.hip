// Smoothing factors s_j = amax_x[j]^alpha / amax_w[j]^(1 - alpha) and inv_s_j = 1 / s_j
// (the rounding is that of smooth_factor in smooth_factor.h).
//
// Method: jisaku.com glossary page "SmoothQuant", section "ハイパーパラメータ α".
//
// K is at most a few tens of thousands: one thread per channel, launch bound.
#include "common.h"
#include "smooth_factor.h"

namespace w8a8 {

namespace {

__global__ __launch_bounds__(256) void k_smooth_factors(const float* __restrict__ ax,
                                                        const float* __restrict__ aw, int64_t K,
                                                        double alpha, float* __restrict__ s,
                                                        float* __restrict__ inv_s) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= K) return;
  smooth_factor(ax[j], aw[j], alpha, s[j], inv_s[j]);
}

// out_j = a_j * b_j, one fp32 rounding: the folded weight of a per-channel
// scale (the smoothing's inv_s) and the per-channel weight it folds into.
__global__ __launch_bounds__(256) void k_fold(const float* __restrict__ a,
                                              const float* __restrict__ b, int64_t n,
                                              float* __restrict__ out) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j < n) out[j] = a[j] * b[j];
}

}  // namespace

hipError_t launch_fold(const float* a, const float* b, int64_t n, float* out, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fold, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a, b, n, out);
  return hipGetLastError();
}

hipError_t launch_smooth_factors(const float* ax, const float* aw, int64_t K, double alpha,
                                 float* s, float* inv_s, hipStream_t st) {
  if (K == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((K + 255) / 256);
  hipLaunchKernelGGL(k_smooth_factors, dim3(blocks), dim3(256), 0, st, ax, aw, K, alpha, s, inv_s);
  return hipGetLastError();
}

}  // namespace w8a8
