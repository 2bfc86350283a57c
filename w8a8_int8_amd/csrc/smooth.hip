// Smoothing factors s_j = amax_x[j]^alpha / amax_w[j]^(1 - alpha) and inv_s_j = 1 / s_j.
//
// Method: jisaku.com glossary page "SmoothQuant", section "ハイパーパラメータ α".
// The factor is formed in fp64 (device pow and one IEEE division) and rounded
// once to fp32; the reciprocal is one IEEE fp32 division.  alpha = 1 and
// alpha = 0 take the formula's exact values (s = amax_x, s = 1 / amax_w) so
// those limits do not depend on the accuracy of pow.  A channel with a zero
// maximum on either side is left unscaled (s = 1).
//
// K is at most a few tens of thousands: one thread per channel, launch bound.
#include "common.h"

namespace w8a8 {

namespace {

__global__ __launch_bounds__(256) void k_smooth_factors(const float* __restrict__ ax,
                                                        const float* __restrict__ aw, int64_t K,
                                                        double alpha, float* __restrict__ s,
                                                        float* __restrict__ inv_s) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= K) return;
  const double a = ax[j], b = aw[j];
  float sj;
  if (a == 0.0 || b == 0.0) {
    sj = 1.0f;
  } else if (alpha == 1.0) {
    sj = (float)a;
  } else if (alpha == 0.0) {
    sj = (float)(1.0 / b);
  } else {
    sj = (float)(pow(a, alpha) / pow(b, 1.0 - alpha));
  }
  s[j] = sj;
  inv_s[j] = 1.0f / sj;
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
