// C ABI of libw8a8: argument validation and dispatch to the kernels.
//
// Every check runs on the host before any HIP call, so a rejected call
// enqueues nothing and touches no device state.  The entry points, their
// arguments and their error codes are documented in include/w8a8.h.
#include "../../include/w8a8.h"

#include <math.h>

#include <mutex>

#include "common.h"

// The scratch of w8a8_linear_noalloc: one file-scope device array, which
// every GPU the library runs on holds (at its own address) until the process
// ends.  Host code never uses the name itself, which is only a host-side
// stand-in: it takes the array's device address per device from
// hipGetSymbolAddress and passes that to the kernels.
static __device__ __align__(256) char scratch[W8A8_NOALLOC_SCRATCH_BYTES];

namespace {

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

inline w8a8_status_t hip_status(hipError_t e) { return e == hipSuccess ? W8A8_OK : W8A8_ERR_HIP; }

inline bool valid_dtype(int dt) { return dt == W8A8_F16 || dt == W8A8_BF16; }

constexpr int64_t kMaxRows = (int64_t)1 << 31;  // 32-bit row indices in the kernels
constexpr int64_t kMaxQuantCols = 65536;         // 1024 threads x 8 chunks x 8 values
constexpr size_t kWsAlign = 256;

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Device address of `scratch` on the current device, resolved once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

w8a8_status_t scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return W8A8_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return W8A8_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return W8A8_OK;
}

w8a8_status_t check_gemm(const void* qa, const void* qb, const void* out, int64_t M, int64_t N,
                         int64_t K) {
  if (M < 0 || N < 0 || K < 0 || M >= kMaxRows || N >= kMaxRows || K > W8A8_MAX_K ||
      K % 16 != 0 || N % 8 != 0)
    return W8A8_ERR_SHAPE;
  // a pointer may be NULL only when its array is empty
  if ((!qa && M * K) || (!qb && N * K) || (!out && M * N)) return W8A8_ERR_NULL;
  // the kernels address each operand tile with 32-bit offsets: BM x K bytes
  if (!aligned(qa, 16) || !aligned(qb, 16) || !aligned(out, 16)) return W8A8_ERR_ALIGN;
  return W8A8_OK;
}

w8a8_status_t check_quant(const void* x, int dtype, int64_t rows, int64_t cols,
                          const float* col_scale, const int8_t* q, const float* row_scale) {
  if (!valid_dtype(dtype)) return W8A8_ERR_DTYPE;
  if (rows < 0 || cols < 0 || rows >= kMaxRows || cols > kMaxQuantCols || cols % 16 != 0)
    return W8A8_ERR_SHAPE;
  // a pointer may be NULL only when its array is empty
  if ((!x && rows * cols) || (!q && rows * cols) || (!col_scale && cols) || (!row_scale && rows))
    return W8A8_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(col_scale, 16) || !aligned(row_scale, 4))
    return W8A8_ERR_ALIGN;
  return W8A8_OK;
}

// Argument checks of the runtime forward (workspace as w8a8_linear takes it).
w8a8_status_t check_linear(const void* x, int dtype, const float* inv_s, const int8_t* qw,
                           const float* sw, const void* y, int64_t M, int64_t N, int64_t K,
                           const void* workspace, size_t ws_bytes);

// Enqueue the runtime forward on checked arguments.
w8a8_status_t launch_linear(const void* x, int dtype, const float* inv_s, const int8_t* qw,
                            const float* sw, void* y, int64_t M, int64_t N, int64_t K,
                            void* workspace, hipStream_t stream);

}  // namespace

extern "C" {

int w8a8_abi_version(void) { return W8A8_ABI_VERSION; }

const char* w8a8_status_str(int status) {
  switch (status) {
    case W8A8_OK: return "ok";
    case W8A8_ERR_NULL: return "a required pointer is NULL";
    case W8A8_ERR_SHAPE: return "invalid shape (negative, too large, or not a required multiple)";
    case W8A8_ERR_ALIGN: return "pointer not aligned as required (16 bytes for matrices)";
    case W8A8_ERR_DTYPE: return "unknown dtype code";
    case W8A8_ERR_ARG: return "argument out of range";
    case W8A8_ERR_HIP: return "HIP launch failed";
    case W8A8_ERR_TOO_LARGE:
      return "the call needs more scratch than the library's static array holds "
             "(W8A8_NOALLOC_SCRATCH_BYTES); use w8a8_linear with a workspace";
    default: return "unknown status";
  }
}

w8a8_status_t w8a8_channel_amax(const void* x, int dtype, int64_t rows, int64_t cols,
                                float* amax, hipStream_t stream) {
  if (!valid_dtype(dtype)) return W8A8_ERR_DTYPE;
  if (rows < 0 || cols < 1 || cols % 8 != 0 || rows >= ((int64_t)1 << 40)) return W8A8_ERR_SHAPE;
  if ((!x && rows) || !amax) return W8A8_ERR_NULL;
  if (!aligned(x, 16) || !aligned(amax, 4)) return W8A8_ERR_ALIGN;
  return hip_status(w8a8::launch_channel_amax(x, dtype == W8A8_BF16, rows, cols, amax, stream));
}

w8a8_status_t w8a8_smooth_factors(const float* amax_x, const float* amax_w, int64_t K,
                                  double alpha, float* s, float* inv_s, hipStream_t stream) {
  if (K < 0 || K >= kMaxRows) return W8A8_ERR_SHAPE;
  if (K && (!amax_x || !amax_w || !s || !inv_s)) return W8A8_ERR_NULL;
  if (!(alpha >= 0.0 && alpha <= 1.0)) return W8A8_ERR_ARG;  // also rejects NaN
  if (!aligned(amax_x, 4) || !aligned(amax_w, 4) || !aligned(s, 4) || !aligned(inv_s, 4))
    return W8A8_ERR_ALIGN;
  return hip_status(w8a8::launch_smooth_factors(amax_x, amax_w, K, alpha, s, inv_s, stream));
}

size_t w8a8_calibrate_smooth_scratch_bytes(int64_t K) {
  if (K < 1 || K % 8 != 0 || K >= kMaxRows) return 0;
  return w8a8::calibrate_smooth_scratch_bytes(K);
}

namespace {

// The checks of one w8a8_calibrate_smooth call (dtype checked by the caller).
w8a8_status_t check_calibrate(const void* x_cal, int64_t cal_rows, const void* w, int64_t N,
                              int64_t K, double alpha, const float* amax_x, const float* amax_w,
                              const float* s, const float* inv_s, const void* scratch,
                              size_t scratch_bytes) {
  if (cal_rows < 0 || N < 0 || cal_rows >= ((int64_t)1 << 40) || N >= ((int64_t)1 << 40) ||
      K < 1 || K % 8 != 0 || K >= kMaxRows)
    return W8A8_ERR_SHAPE;
  if ((!x_cal && cal_rows) || (!w && N) || !amax_x || !amax_w || !s || !inv_s || !scratch)
    return W8A8_ERR_NULL;
  if (!(alpha >= 0.0 && alpha <= 1.0)) return W8A8_ERR_ARG;  // also rejects NaN
  if (scratch_bytes < w8a8::calibrate_smooth_scratch_bytes(K)) return W8A8_ERR_ARG;
  if (!aligned(x_cal, 16) || !aligned(w, 16) || !aligned(amax_x, 4) || !aligned(amax_w, 4) ||
      !aligned(s, 4) || !aligned(inv_s, 4) || !aligned(scratch, 16))
    return W8A8_ERR_ALIGN;
  return W8A8_OK;
}

}  // namespace

w8a8_status_t w8a8_calibrate_smooth_layers(const w8a8_calib_layer_t* layers, int n, int dtype,
                                           hipStream_t stream) {
  if (!valid_dtype(dtype)) return W8A8_ERR_DTYPE;
  if (n < 0) return W8A8_ERR_SHAPE;
  if (n == 0) return W8A8_OK;
  if (!layers) return W8A8_ERR_NULL;
  for (int i = 0; i < n; ++i) {
    const w8a8_calib_layer_t& l = layers[i];
    const w8a8_status_t st = check_calibrate(l.x_cal, l.cal_rows, l.w, l.N, l.K, l.alpha, l.amax_x,
                                             l.amax_w, l.s, l.inv_s, l.scratch, l.scratch_bytes);
    if (st != W8A8_OK) return st;
  }
  // the kernel arguments of one launch, in chunks of up to 8 entries
  w8a8::CalibLayerArgs a[8];
  for (int i0 = 0; i0 < n; i0 += 8) {
    const int m = n - i0 < 8 ? n - i0 : 8;
    for (int i = 0; i < m; ++i) {
      const w8a8_calib_layer_t& l = layers[i0 + i];
      a[i] = w8a8::CalibLayerArgs{l.x_cal, l.cal_rows, l.w, l.N, l.K, l.alpha,
                                  l.amax_x, l.amax_w, l.s, l.inv_s, l.scratch};
    }
    const w8a8_status_t st =
        hip_status(w8a8::launch_calibrate_smooth_layers(m, a, dtype == W8A8_BF16, stream));
    if (st != W8A8_OK) return st;
  }
  return W8A8_OK;
}

w8a8_status_t w8a8_calibrate_smooth(const void* x_cal, int64_t cal_rows, const void* w, int64_t N,
                                    int dtype, int64_t K, double alpha, float* amax_x,
                                    float* amax_w, float* s, float* inv_s, void* scratch,
                                    size_t scratch_bytes, hipStream_t stream) {
  if (!valid_dtype(dtype)) return W8A8_ERR_DTYPE;
  const w8a8_status_t st = check_calibrate(x_cal, cal_rows, w, N, K, alpha, amax_x, amax_w, s,
                                           inv_s, scratch, scratch_bytes);
  if (st != W8A8_OK) return st;
  return hip_status(w8a8::launch_calibrate_smooth(x_cal, cal_rows, w, N, dtype == W8A8_BF16, K,
                                                  alpha, amax_x, amax_w, s, inv_s, scratch,
                                                  stream));
}

w8a8_status_t w8a8_scale_quant_rows(const void* x, int dtype, int64_t rows, int64_t cols,
                                    const float* col_scale, int8_t* q, float* row_scale,
                                    hipStream_t stream) {
  const w8a8_status_t st = check_quant(x, dtype, rows, cols, col_scale, q, row_scale);
  if (st != W8A8_OK) return st;
  return hip_status(w8a8::launch_scale_quant_rows(x, dtype == W8A8_BF16, rows, cols, col_scale,
                                                  false, 0.0f, q, row_scale, 0, stream));
}

w8a8_status_t w8a8_scale_quant_pair(const void* w, int64_t N, const float* s, int8_t* qw,
                                    float* sw, const void* x, int64_t M, const float* inv_s,
                                    int8_t* qx, float* sx, int dtype, int64_t K,
                                    hipStream_t stream) {
  w8a8_status_t st = check_quant(w, dtype, N, K, s, qw, sw);
  if (st == W8A8_OK) st = check_quant(x, dtype, M, K, inv_s, qx, sx);
  if (st != W8A8_OK) return st;
  if (M + N >= kMaxRows) return W8A8_ERR_SHAPE;
  return hip_status(w8a8::launch_scale_quant_pair(w, N, s, qw, sw, x, M, inv_s, qx, sx,
                                                  dtype == W8A8_BF16, K, stream));
}

w8a8_status_t w8a8_scale_quant_rows_e4m3(const void* x, int dtype, int64_t rows, int64_t cols,
                                         const float* col_scale, uint8_t* q, float* row_scale,
                                         hipStream_t stream) {
  const w8a8_status_t st = check_quant(x, dtype, rows, cols, col_scale, (const int8_t*)q, row_scale);
  if (st != W8A8_OK) return st;
  return hip_status(w8a8::launch_scale_quant_rows(x, dtype == W8A8_BF16, rows, cols, col_scale,
                                                  false, 0.0f, q, row_scale, 1, stream));
}

w8a8_status_t w8a8_fold_norm_weight(const float* gamma, const float* inv_s, int64_t K, float* g,
                                    hipStream_t stream) {
  if (K < 0 || K >= kMaxRows) return W8A8_ERR_SHAPE;
  if (K && (!gamma || !inv_s || !g)) return W8A8_ERR_NULL;
  if (!aligned(gamma, 4) || !aligned(inv_s, 4) || !aligned(g, 4)) return W8A8_ERR_ALIGN;
  return hip_status(w8a8::launch_fold(gamma, inv_s, K, g, stream));
}

w8a8_status_t w8a8_rmsnorm_quant_rows(const void* h, int dtype, int64_t rows, int64_t cols,
                                      const float* g, float eps, int8_t* q, float* row_scale,
                                      hipStream_t stream) {
  const w8a8_status_t st = check_quant(h, dtype, rows, cols, g, q, row_scale);
  if (st != W8A8_OK) return st;
  if (!(eps >= 0.0f && eps <= 3.0e38f)) return W8A8_ERR_ARG;  // also rejects NaN and +inf
  if (cols == 0 && rows) return W8A8_ERR_SHAPE;                // the mean of an empty row
  return hip_status(w8a8::launch_scale_quant_rows(h, dtype == W8A8_BF16, rows, cols, g, true, eps,
                                                  q, row_scale, 0, stream));
}

w8a8_status_t w8a8_layernorm_quant_rows(const void* x, int dtype, int64_t rows, int64_t cols,
                                        const float* g, const float* b, float eps, int8_t* q,
                                        float* row_scale, hipStream_t stream) {
  const w8a8_status_t st = check_quant(x, dtype, rows, cols, g, q, row_scale);
  if (st != W8A8_OK) return st;
  if (dtype != W8A8_F16) return W8A8_ERR_DTYPE;  // exact row sums need fp16's range
  if (!b && cols) return W8A8_ERR_NULL;
  if (!aligned(b, 16)) return W8A8_ERR_ALIGN;
  if (!(eps >= 0.0f && eps <= 3.0e38f)) return W8A8_ERR_ARG;  // also rejects NaN and +inf
  if (cols == 0 && rows) return W8A8_ERR_SHAPE;                // the mean of an empty row
  return hip_status(w8a8::launch_layernorm_quant_rows(x, rows, cols, g, b, eps, q, row_scale,
                                                      stream));
}

w8a8_status_t w8a8_gemm_i32(const int8_t* qa, const int8_t* qb, int32_t* c, int64_t M, int64_t N,
                            int64_t K, hipStream_t stream) {
  const w8a8_status_t st = check_gemm(qa, qb, c, M, N, K);
  if (st != W8A8_OK) return st;
  return hip_status(w8a8::launch_gemm(qa, qb, M, N, K, nullptr, nullptr, c, 0, stream));
}

w8a8_status_t w8a8_gemm_dequant(const int8_t* qa, const float* sa, const int8_t* qb,
                                const float* sb, void* y, int out_dtype, int64_t M, int64_t N,
                                int64_t K, hipStream_t stream) {
  w8a8_status_t st = check_gemm(qa, qb, y, M, N, K);
  if (st != W8A8_OK) return st;
  if ((!sa && M) || (!sb && N)) return W8A8_ERR_NULL;
  if (!valid_dtype(out_dtype)) return W8A8_ERR_DTYPE;
  if (!aligned(sa, 4) || !aligned(sb, 16)) return W8A8_ERR_ALIGN;
  return hip_status(w8a8::launch_gemm(qa, qb, M, N, K, sa, sb, y, out_dtype == W8A8_BF16 ? 2 : 1,
                                      stream));
}

w8a8_status_t w8a8_gemm_dequant_e4m3(const uint8_t* qa, const float* sa, const uint8_t* qb,
                                     const float* sb, void* y, int out_dtype, int64_t M, int64_t N,
                                     int64_t K, hipStream_t stream) {
  w8a8_status_t st = check_gemm((const int8_t*)qa, (const int8_t*)qb, y, M, N, K);
  if (st != W8A8_OK) return st;
  if ((!sa && M) || (!sb && N)) return W8A8_ERR_NULL;
  if (!valid_dtype(out_dtype)) return W8A8_ERR_DTYPE;
  if (!aligned(sa, 4) || !aligned(sb, 16)) return W8A8_ERR_ALIGN;
  return hip_status(w8a8::launch_gemm((const int8_t*)qa, (const int8_t*)qb, M, N, K, sa, sb, y,
                                      out_dtype == W8A8_BF16 ? 6 : 5, stream));
}

w8a8_status_t w8a8_gemm_float(const void* a, const void* b, void* y, int dtype, int64_t M,
                              int64_t N, int64_t K, hipStream_t stream) {
  if (!valid_dtype(dtype)) return W8A8_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0 || M >= kMaxRows || N >= kMaxRows || K > ((int64_t)1 << 20) ||
      K % 8 != 0 || N % 8 != 0)
    return W8A8_ERR_SHAPE;
  if ((!a && M * K) || (!b && N * K) || (!y && M * N)) return W8A8_ERR_NULL;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(y, 16)) return W8A8_ERR_ALIGN;
  return hip_status(w8a8::launch_gemm((const int8_t*)a, (const int8_t*)b, M, N, K, nullptr,
                                      nullptr, y, dtype == W8A8_BF16 ? 4 : 3, stream));
}

// Shapes that take the split-K path (splitk_plan): its int32 partial slices
// and the arrival counters of its channel groups follow the INT8 activations
// and their scales in the workspace.
static bool linear_splitk(int64_t M, int64_t N, int64_t K) {
  return w8a8::splitk_plan(M, N, K).splits > 0;
}

size_t w8a8_linear_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return 0;
  size_t b = round_up((size_t)M * (size_t)K, kWsAlign) + round_up((size_t)M * 4, kWsAlign);
  if (linear_splitk(M, N, K)) {
    const w8a8::SplitkPlan p = w8a8::splitk_plan(M, N, K);
    b += round_up((size_t)p.splits * (size_t)M * (size_t)N * 4, kWsAlign);
    b += round_up((size_t)p.groups * 4, kWsAlign);
  }
  return b;
}

w8a8_status_t w8a8_linear(const void* x, int dtype, const float* inv_s, const int8_t* qw,
                          const float* sw, void* y, int64_t M, int64_t N, int64_t K,
                          void* workspace, size_t ws_bytes, hipStream_t stream) {
  const w8a8_status_t st = check_linear(x, dtype, inv_s, qw, sw, y, M, N, K, workspace, ws_bytes);
  if (st != W8A8_OK) return st;
  return launch_linear(x, dtype, inv_s, qw, sw, y, M, N, K, workspace, stream);
}

w8a8_status_t w8a8_linear_noalloc(const void* x, int dtype, const float* inv_s, const int8_t* qw,
                                  const float* sw, void* y, int64_t M, int64_t N, int64_t K,
                                  hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0) return W8A8_ERR_SHAPE;
  if (w8a8_linear_workspace_bytes(M, N, K) > (size_t)W8A8_NOALLOC_SCRATCH_BYTES)
    return W8A8_ERR_TOO_LARGE;
  // every argument check first, with a stand-in for the scratch's address
  // (any 256-byte aligned value), so a rejected call makes no HIP call at all
  w8a8_status_t st = check_linear(x, dtype, inv_s, qw, sw, y, M, N, K, (void*)kWsAlign,
                                  W8A8_NOALLOC_SCRATCH_BYTES);
  if (st != W8A8_OK) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != W8A8_OK) return st;
  return launch_linear(x, dtype, inv_s, qw, sw, y, M, N, K, ws, stream);
}

}  // extern "C"

namespace {

struct LinearWs {
  int8_t* qx;
  float* sx;
  int32_t* part;      // split-K partial slices (splits x M x N)
  unsigned* counters;  // split-K arrival counters (one per channel group)
};

LinearWs linear_ws(const void* workspace, int64_t M, int64_t N, int64_t K) {
  char* base = (char*)workspace;
  const size_t off_sx = round_up((size_t)M * (size_t)K, kWsAlign);
  const size_t off_part = off_sx + round_up((size_t)M * 4, kWsAlign);
  size_t off_cnt = off_part;
  if (linear_splitk(M, N, K))
    off_cnt += round_up((size_t)w8a8::splitk_plan(M, N, K).splits * (size_t)M * (size_t)N * 4,
                        kWsAlign);
  return LinearWs{(int8_t*)base, (float*)(base + off_sx), (int32_t*)(base + off_part),
                  (unsigned*)(base + off_cnt)};
}

w8a8_status_t check_linear(const void* x, int dtype, const float* inv_s, const int8_t* qw,
                           const float* sw, const void* y, int64_t M, int64_t N, int64_t K,
                           const void* workspace, size_t ws_bytes) {
  if (!valid_dtype(dtype)) return W8A8_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0) return W8A8_ERR_SHAPE;
  if (!workspace || (!sw && N)) return W8A8_ERR_NULL;
  if (!aligned(workspace, kWsAlign)) return W8A8_ERR_ALIGN;
  if (ws_bytes < w8a8_linear_workspace_bytes(M, N, K)) return W8A8_ERR_ARG;
  const LinearWs ws = linear_ws(workspace, M, N, K);
  w8a8_status_t st = check_quant(x, dtype, M, K, inv_s, ws.qx, ws.sx);
  if (st != W8A8_OK) return st;
  st = check_gemm(ws.qx, qw, y, M, N, K);
  if (st != W8A8_OK) return st;
  if (!aligned(sw, 16)) return W8A8_ERR_ALIGN;
  return W8A8_OK;
}

w8a8_status_t launch_linear(const void* x, int dtype, const float* inv_s, const int8_t* qw,
                            const float* sw, void* y, int64_t M, int64_t N, int64_t K,
                            void* workspace, hipStream_t stream) {
  const LinearWs ws = linear_ws(workspace, M, N, K);
  const bool bf16 = dtype == W8A8_BF16;
  const bool split = linear_splitk(M, N, K);
  // the quantization launch also clears the split-K counters
  const int ncnt = split ? w8a8::splitk_plan(M, N, K).groups : 0;
  hipError_t e = w8a8::launch_scale_quant_rows(x, bf16, M, K, inv_s, false, 0.0f, ws.qx, ws.sx, 0,
                                               stream, ws.counters, ncnt);
  if (e != hipSuccess) return W8A8_ERR_HIP;
  if (split)
    return hip_status(w8a8::launch_gemm_splitk(ws.qx, qw, M, N, K, ws.sx, sw, y, bf16, ws.part,
                                               ws.counters, stream));
  return hip_status(w8a8::launch_gemm(ws.qx, qw, M, N, K, ws.sx, sw, y, bf16 ? 2 : 1, stream));
}

}  // namespace
