// Internal declarations shared by the HIP sources of libw8a8 (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Launchers: arguments are validated by the C ABI layer before these run.
hipError_t launch_channel_amax(const void* x, bool bf16, int64_t rows, int64_t cols, float* amax,
                               hipStream_t st);
hipError_t launch_smooth_factors(const float* ax, const float* aw, int64_t K, double alpha,
                                 float* s, float* inv_s, hipStream_t st);
// Scratch of launch_calibrate_smooth: the weight maximum accumulator (K
// floats, padded to 256 bytes) and one arrival counter per 256 channels.
size_t calibrate_smooth_scratch_bytes(int64_t K);
hipError_t launch_calibrate_smooth(const void* xc, int64_t cal_rows, const void* w,
                                   int64_t w_rows, bool bf16, int64_t K, double alpha,
                                   float* amax_x, float* amax_w, float* s, float* inv_s,
                                   void* scratch, hipStream_t st);
// Several layers' launch_calibrate_smooth in one launch (same dtype); each
// entry as that call's arguments, with n = the weight's rows and k = K.
struct CalibLayerArgs {
  const void* x_cal;
  int64_t cal_rows;
  const void* w;
  int64_t n, k;
  double alpha;
  float *amax_x, *amax_w, *s, *inv_s;
  void* scratch;
};
hipError_t launch_calibrate_smooth_layers(int n, const CalibLayerArgs* a, bool bf16,
                                          hipStream_t st);
// fmt: 0 = symmetric INT8 codes, 1 = FP8 E4M3 codes.  norm (INT8 only): the
// rows are RMS-norm inputs and col_scale the folded norm weight; the row scale
// is divided by the row's rms (with eps).  The same launch sets the nzero
// words at `zero` to 0 (the split-K counters of the product that follows).
hipError_t launch_scale_quant_rows(const void* x, bool bf16, int64_t rows, int64_t cols,
                                   const float* col_scale, bool norm, float eps, void* q,
                                   float* row_scale, int fmt, hipStream_t st,
                                   unsigned* zero = nullptr, int nzero = 0);
// The weight (n rows, col_scale s) and the activations (m rows, col_scale
// inv_s) of one layer, both with k columns, quantized to INT8 in one launch.
hipError_t launch_scale_quant_pair(const void* w, int64_t n, const float* s, void* qw, float* sw,
                                   const void* x, int64_t m, const float* inv_s, void* qx,
                                   float* sx, bool bf16, int64_t k, hipStream_t st);
hipError_t launch_fold(const float* a, const float* b, int64_t n, float* out, hipStream_t st);
// LayerNorm fold (fp16 rows): per-token INT8 of LayerNorm(x; gamma, beta) * inv_s
// given g = RN32(gamma * inv_s) and b = RN32(beta * inv_s).
hipError_t launch_layernorm_quant_rows(const void* x, int64_t rows, int64_t cols, const float* g,
                                       const float* b, float eps, void* q, float* row_scale,
                                       hipStream_t st);
// Split-K few-token GEMM with the dequant epilogue (3 <= M <= 32 on narrow
// layers with long rows; splitk_plan): one launch over groups x splits
// blocks.  Each block stores an int32 partial slice of M x N in `partials`
// (splits slices) and counts itself on counters[group] (groups of them, zero
// on entry, left at S); the last block of a group adds the slices and
// dequantizes.
constexpr int kSplitkCG = 4;  // 16-channel groups per block
struct SplitkPlan {
  int splits;  // 0: shape not served (the unsplit kernels take it)
  int groups;  // blocks per split, one counter each
};
SplitkPlan splitk_plan(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_splitk(const int8_t* qa, const int8_t* qb, int64_t M, int64_t N, int64_t K,
                              const float* sa, const float* sb, void* y, bool bf16,
                              int32_t* partials, unsigned* counters, hipStream_t st);
// out_mode: 0 = int32 accumulators, 1 = fp16 dequant, 2 = bf16 dequant (int8
// operands, K in bytes); 3 = fp16, 4 = bf16 dense product (16-bit operands,
// K in elements, fp32 accumulation); 5 = fp16, 6 = bf16 dequant of FP8 E4M3
// operands (K in bytes, fp32 accumulation)
hipError_t launch_gemm(const int8_t* qa, const int8_t* qb, int64_t M, int64_t N, int64_t K,
                       const float* sa, const float* sb, void* out, int out_mode,
                       hipStream_t st);

// Widening of one 16-bit storage value to fp32 (exact).
__device__ __forceinline__ float widen16(unsigned short h, bool bf16) {
  if (bf16) return __uint_as_float(((unsigned)h) << 16);
  return (float)__builtin_bit_cast(_Float16, h);
}

}  // namespace w8a8
