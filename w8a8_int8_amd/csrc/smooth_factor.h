// The smoothing factor of one channel, shared by k_smooth_factors and the
// fused calibration kernel so that both round it identically.
//
// Method: jisaku.com glossary page "SmoothQuant", section "ハイパーパラメータ α":
// s_j = max|X_j|^alpha / max|W_j|^(1 - alpha).  It is formed in fp64 (device
// pow and one IEEE division) and rounded once to fp32; the reciprocal is one
// IEEE fp32 division.  alpha = 1 and alpha = 0 take the formula's exact values
// (s = amax_x, s = 1 / amax_w) so those limits do not depend on the accuracy
// of pow.  A channel with a zero maximum on either side is left unscaled
// (s = 1).
#pragma once

#include <hip/hip_runtime.h>

namespace w8a8 {

__device__ __forceinline__ void smooth_factor(float ax, float aw, double alpha, float& s,
                                              float& inv_s) {
  const double a = ax, b = aw;
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
  s = sj;
  inv_s = 1.0f / sj;
}

}  // namespace w8a8
