/*
 * w8a8.h -- C ABI of the SmoothQuant W8A8 linear-layer path on MI355X (gfx950).
 *
 * Source of the method: the jisaku.com glossary page "SmoothQuant"
 * (アクティベーション平滑化量子化).  Each entry point names the section of that
 * page that defines its operation.
 *
 * The path, for one linear layer Y = X W (X: M x K activations, W: the
 * layer's weight with K input and N output channels):
 *   1. channel amax over calibration activations      w8a8_channel_amax
 *   2. smoothing factors s, their reciprocals          w8a8_smooth_factors
 *      1 (one last batch) + weight maxima + 2 at once   w8a8_calibrate_smooth
 *      fold s into W and quantize W per output channel w8a8_channel_amax (on W)
 *                                                       + w8a8_scale_quant_rows
 *   3. X diag(s)^-1 and per-token INT8 quantization    w8a8_scale_quant_rows
 *      2 (weight fold + quant) and 3 in one launch      w8a8_scale_quant_pair
 *      ... folded into the RMS norm that produces X     w8a8_fold_norm_weight (offline)
 *                                                       + w8a8_rmsnorm_quant_rows
 *      ... or into a LayerNorm (fp16)                   w8a8_layernorm_quant_rows
 *   4. INT8 x INT8 -> INT32 product                    w8a8_gemm_i32 (diagnostic)
 *   5. dequantize with per-token x per-channel scales  w8a8_gemm_dequant (fuses 4+5)
 *   runtime forward = 3 + 4 + 5                         w8a8_linear
 *   FP8 (E4M3) form of 2/3 and 4+5                      w8a8_scale_quant_rows_e4m3,
 *                                                       w8a8_gemm_dequant_e4m3
 *
 * Conventions shared by every entry point
 *   - Layout: all matrices are row-major and contiguous.  Activations are
 *     M x K (token major).  Weights are stored N x K (output channel major),
 *     so the page's "W_j" (input channel j) is column j of that array.
 *   - Memory: pointers are DEVICE pointers on the current HIP device unless a
 *     comment says otherwise.  The caller allocates and owns every buffer; the
 *     library allocates nothing and keeps no mutable state (the one exception
 *     is the static scratch of w8a8_linear_noalloc, at the end), so concurrent
 *     calls on different streams are safe when their buffers do not overlap.
 *   - Asynchrony: device work is enqueued on `stream` (0 = the null stream)
 *     and the call returns without synchronizing.
 *   - Errors: every check below runs on the host before any HIP call; a failed
 *     check returns its status and enqueues nothing.  W8A8_ERR_HIP means the
 *     launch itself failed (hipGetLastError).  No entry point aborts.
 *   - NULL: a pointer may be NULL only when the array it points to is empty
 *     (zero elements); otherwise NULL is W8A8_ERR_NULL.
 *   - Alignment: matrix base pointers must be 16-byte aligned and row lengths
 *     multiples of 16 bytes, so that every row starts on a 16-byte boundary.
 *   - Arithmetic: fp32 steps are single IEEE operations with round to nearest
 *     even (no fused multiply-add); integer results are exact.  Inputs must be
 *     finite; outputs for non-finite inputs are unspecified.
 */
#ifndef W8A8_H
#define W8A8_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

#define W8A8_ABI_VERSION 7

/* Largest K for which 127 * 127 * K fits int32, so that every accumulator
 * (and every partial sum) of the INT8 product is exact in int32. */
#define W8A8_MAX_K 131072

typedef enum {
  W8A8_OK = 0,
  W8A8_ERR_NULL = 1,      /* a required pointer is NULL */
  W8A8_ERR_SHAPE = 2,     /* a size is negative, too large, or breaks a multiple-of rule */
  W8A8_ERR_ALIGN = 3,     /* a pointer is not aligned as required */
  W8A8_ERR_DTYPE = 4,     /* unknown dtype code */
  W8A8_ERR_ARG = 5,       /* another argument is out of range (alpha, workspace size) */
  W8A8_ERR_HIP = 6,       /* the HIP launch failed */
  W8A8_ERR_TOO_LARGE = 7, /* w8a8_linear_noalloc: needs more than its static scratch */
} w8a8_status_t;

/* Storage type of activations, weights and outputs. */
typedef enum {
  W8A8_F16 = 0, /* IEEE binary16 */
  W8A8_BF16 = 1 /* bfloat16 */
} w8a8_dtype_t;

/* ABI version of the loaded library (W8A8_ABI_VERSION it was built with). */
int w8a8_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* w8a8_status_str(int status);

/*
 * Step 1 (and the weight half of step 2): per-column running maximum of |x|.
 * Page section "ハイパーパラメータ α": the smoothing factor uses max(|X_j|)
 * over the calibration tokens and max(|W_j|) over the output channels; the
 * usage example collects the former with `get_act_scales`.
 *
 *   x     [rows x cols] fp16/bf16 (dtype), row-major, 16-byte aligned.
 *   amax  [cols] fp32, in/out: amax[j] = max(amax[j], max_t |x[t, j]|).
 *         Before the first call the caller fills it with +0.0f; later calls
 *         (further calibration batches, in any order) keep folding into it.
 *         Every value in it must be a non-negative finite float.
 *   rows >= 0 (0 leaves amax unchanged), 1 <= cols, cols % 8 == 0.
 * For a weight stored N x K, rows = N and cols = K give max|W_j|.
 * Errors: NULL, SHAPE, ALIGN (x not 16-byte, amax not 4-byte aligned), DTYPE, HIP.
 */
w8a8_status_t w8a8_channel_amax(const void* x, int dtype, int64_t rows, int64_t cols,
                                float* amax, hipStream_t stream);

/*
 * Step 2: smoothing factors.  Page section "ハイパーパラメータ α":
 * s_j = max(|X_j|)^alpha / max(|W_j|)^(1 - alpha).
 *
 *   amax_x, amax_w  [K] fp32 channel maxima of the activations and weights.
 *   alpha           migration strength, 0 <= alpha <= 1 (the page's default is 0.5).
 *   s, inv_s        [K] fp32 outputs: s_j evaluated in fp64 and rounded once to
 *                   fp32; inv_s_j = 1 / s_j as one fp32 division.  A channel whose
 *                   amax_x or amax_w is zero gets s_j = inv_s_j = 1.
 *   K >= 0.
 * Errors: NULL, SHAPE, ARG (alpha outside [0, 1] or NaN), HIP.
 */
w8a8_status_t w8a8_smooth_factors(const float* amax_x, const float* amax_w, int64_t K,
                                  double alpha, float* s, float* inv_s, hipStream_t stream);

/*
 * Steps 1 and 2 of one layer in one launch: fold one calibration batch into
 * the running max|X_j|, take max|W_j| over the weight's output channels, and
 * form s and inv_s from the two.  Page section "ハイパーパラメータ α", as
 * w8a8_channel_amax (twice) followed by w8a8_smooth_factors, with the same
 * results bit for bit; the usage example's `smooth_lm(model, act_scales,
 * alpha)` is this call after the other calibration batches went through
 * w8a8_channel_amax (or with cal_rows = 0).
 *
 *   x_cal    [cal_rows x K] fp16/bf16 (dtype) calibration batch, 16-byte
 *            aligned; cal_rows may be 0 (then amax_x is only read).
 *   w        [N x K] weight, same dtype, 16-byte aligned; N may be 0 (then
 *            amax_w = 0 and s = 1).
 *   amax_x   [K] fp32, in/out running maximum as in w8a8_channel_amax.
 *   amax_w   [K] fp32 output, max_k |w[k, j]| (overwritten, not folded).
 *   s, inv_s [K] fp32 outputs as in w8a8_smooth_factors (alpha in [0, 1]).
 *   scratch  device memory of at least w8a8_calibrate_smooth_scratch_bytes(K)
 *            bytes, 16-byte aligned, zero-filled by the caller before its
 *            first use.  Every call leaves it zero again, so it is filled
 *            once, not per call.  Calls that share a scratch must not run
 *            concurrently (they would mix their weight maxima).
 *   K >= 8, K % 8 == 0; cal_rows, N >= 0.
 * The blocks meet through device-scope atomics only (no host round trip, no
 * second launch): the last block over each 256 channels forms their s.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, ARG (alpha outside [0, 1] or NaN,
 * scratch_bytes too small), HIP.
 */
size_t w8a8_calibrate_smooth_scratch_bytes(int64_t K); /* 0 for an invalid K */
w8a8_status_t w8a8_calibrate_smooth(const void* x_cal, int64_t cal_rows, const void* w, int64_t N,
                                    int dtype, int64_t K, double alpha, float* amax_x,
                                    float* amax_w, float* s, float* inv_s, void* scratch,
                                    size_t scratch_bytes, hipStream_t stream);

/*
 * w8a8_calibrate_smooth for several layers in one launch: the usage example's
 * `smooth_lm(model, act_scales, alpha)` smooths every linear layer of the
 * model (page section "インストール・使用例"), and the layers are independent,
 * so their calibration folds, weight maxima and smoothing factors can share a
 * grid.  Each entry's results are the same bits as w8a8_calibrate_smooth with
 * its arguments.  One launch covers up to 8 entries (more are split into
 * several launches, in order).
 *
 *   layers   HOST array of n entries, read during the call only (the library
 *            keeps no pointer to it).  Each entry: x_cal, cal_rows, w, N, K,
 *            alpha, amax_x, amax_w, s, inv_s, scratch, scratch_bytes, with the
 *            meaning, layout and rules of the w8a8_calibrate_smooth arguments
 *            of the same names (device pointers).  The entries must not share
 *            an output array or a scratch.
 *   n        number of entries, n >= 0 (0: nothing is enqueued).
 *   dtype    one dtype for every entry's x_cal and w.
 * Errors: NULL (layers NULL with n > 0, or an entry's pointer), SHAPE (n < 0
 * or an entry's sizes), ALIGN, DTYPE, ARG (an entry's alpha or scratch size),
 * HIP.  Every entry is checked before anything is enqueued.
 */
typedef struct {
  const void* x_cal;
  int64_t cal_rows;
  const void* w;
  int64_t N;
  int64_t K;
  double alpha;
  float* amax_x;
  float* amax_w;
  float* s;
  float* inv_s;
  void* scratch;
  size_t scratch_bytes;
} w8a8_calib_layer_t;
w8a8_status_t w8a8_calibrate_smooth_layers(const w8a8_calib_layer_t* layers, int n, int dtype,
                                           hipStream_t stream);

/*
 * Steps 2 (weights) and 3 (activations): scale every column, then quantize
 * every row to symmetric INT8.  Page section "平滑化変換の数学": X~ = X s^-1
 * and W~ = s W; with (x = W, col_scale = s) this folds s into the weight and
 * quantizes it per output channel, with (x = X, col_scale = inv_s) it smooths
 * the activations and quantizes them per token.  For each row t:
 *   v_j = fp32(x[t, j]) * col_scale[j]
 *   m   = max_j |v_j|;  row_scale[t] = m / 127;  r = 127 / m
 *   q[t, j] = clamp(round_half_even(v_j * r), -127, 127)
 * A row with m == 0 gets row_scale 0 and all-zero codes.
 *
 *   x          [rows x cols] fp16/bf16, 16-byte aligned.
 *   col_scale  [cols] fp32, 16-byte aligned.
 *   q          [rows x cols] int8 output, 16-byte aligned.
 *   row_scale  [rows] fp32 output (the dequantization scale of each row).
 *   rows >= 0, cols >= 0, cols % 16 == 0, cols <= 65536.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, HIP.
 */
w8a8_status_t w8a8_scale_quant_rows(const void* x, int dtype, int64_t rows, int64_t cols,
                                    const float* col_scale, int8_t* q, float* row_scale,
                                    hipStream_t stream);

/*
 * Steps 2 (weights) and 3 (activations) of one layer in a single launch, as
 * soon as the layer's s and inv_s exist.  Page section "平滑化変換の数学": the
 * smoothed product is (X s^-1)(s W), so with K input channels
 *   (qw, sw) = w8a8_scale_quant_rows(w [N x K], col_scale = s)
 *   (qx, sx) = w8a8_scale_quant_rows(x [M x K], col_scale = inv_s)
 * with every output bit identical to those two calls.  One grid covers the
 * rows of both matrices (a block takes rows of one of them only), which saves
 * one launch's ramp and tail.
 *
 *   w, qw, sw  [N x K] fp16/bf16 input, [N x K] int8 codes, [N] fp32 scales.
 *   x, qx, sx  [M x K] input of the same dtype, [M x K] codes, [M] scales.
 *   s, inv_s   [K] fp32 column scales.
 *   Alignment, cols (= K) and row limits as in w8a8_scale_quant_rows, and
 *   M + N < 2^31.  The two matrices' outputs must not overlap.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, HIP (the checks of both matrices).
 */
w8a8_status_t w8a8_scale_quant_pair(const void* w, int64_t N, const float* s, int8_t* qw,
                                    float* sw, const void* x, int64_t M, const float* inv_s,
                                    int8_t* qx, float* sx, int dtype, int64_t K,
                                    hipStream_t stream);

/*
 * Offline half of folding step 3 into the RMS normalisation that produces X
 * (LLaMA-family decoders normalise the hidden state h before each projection:
 * X = h / rms(h) * gamma).  Page section "平滑化変換の数学": X~ = X s^-1 is a
 * per-channel factor, so it folds into the norm's per-channel weight (the fold
 * is an extension beyond the page): g_j = gamma_j * inv_s_j, one fp32
 * rounding, computed once per layer like the weight fold.
 *
 *   gamma, inv_s  [K] fp32; g [K] fp32 output; it may be the same array as
 *                 either input (each element is read before it is written).
 *   K >= 0.
 * Errors: NULL, SHAPE, ALIGN (4-byte), HIP.
 */
w8a8_status_t w8a8_fold_norm_weight(const float* gamma, const float* inv_s, int64_t K, float* g,
                                    hipStream_t stream);

/*
 * Runtime half: RMS normalisation with the folded weight g, smoothing and
 * per-token INT8 in one pass over h.  The per-token quantizer is unchanged by
 * a positive factor common to a row, so 1 / rms only enters the row scale.
 * For each row t (fp32, each step one rounding):
 *   v_j = fp32(h[t, j]) * g[j];  m = max_j |v_j|;  r = 127 / m
 *   q[t, j] = round_half_even(v_j * r)
 *   ms = (sum_j h[t, j]^2) / cols   (fp32 sum, order unspecified)
 *   row_scale[t] = (m / 127) * (1 / sqrt(ms + eps))      (0 when m == 0)
 * so that q[t, j] * row_scale[t] approximates (h / rms(h) * gamma)[t, j] * inv_s[j].
 * The codes equal those of w8a8_scale_quant_rows(h, g) bit for bit;
 * row_scale is within (cols / 2 + 6) * 2^-24 relative of its value with an
 * exact sum of squares.  Traffic: that of w8a8_scale_quant_rows; the
 * normalised activations are never written.
 *
 *   h          [rows x cols] fp16/bf16 (dtype), 16-byte aligned: the norm's input.
 *   g          [cols] fp32 folded norm weight (w8a8_fold_norm_weight), 16-byte aligned.
 *   eps        finite, >= 0.
 *   q, row_scale  outputs as in w8a8_scale_quant_rows.
 *   rows >= 0, cols % 16 == 0, cols <= 65536, cols >= 16 when rows > 0.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, ARG (eps negative, NaN or infinite), HIP.
 */
w8a8_status_t w8a8_rmsnorm_quant_rows(const void* h, int dtype, int64_t rows, int64_t cols,
                                      const float* g, float eps, int8_t* q, float* row_scale,
                                      hipStream_t stream);

/*
 * The same fold for a LayerNorm (the norm in front of the projections of
 * OPT-family decoders), y = (x - mean) / sqrt(var + eps) * gamma + beta:
 * y * inv_s = (x - mean) r g + b with g = RN32(gamma * inv_s) and
 * b = RN32(beta * inv_s), both from w8a8_fold_norm_weight.  The pages give no
 * normalisation; the fold extends their X diag(s)^-1 (section
 * "平滑化変換の数学").  The additive b keeps the row statistics in every
 * element, so they are defined without a summation order: every fp16 value
 * is an integer multiple of 2^-24, and with X = x * 2^24, K = cols,
 * S1 = sum X and S2 = sum X^2 (exact integers),
 *   mean = f32(f64(f64(S1) / (K * 2^24)))
 *   var  = f32(f64(f64(K * S2 - S1^2) / (K^2 * 2^48)))   (population variance)
 *   r    = 1 / sqrt(var + eps) in fp32 (each step one rounding), 0 when var + eps == 0
 *   v_j  = ((x[t, j] - mean) * r) * g[j] + b[j]           (fp32, left to right)
 * where f64() / f32() round to nearest even.  Then the per-row quantizer of
 * w8a8_scale_quant_rows on v: codes and row_scale = m / 127.  Results are
 * bit-reproducible.  One pass over x; y is never written.
 *
 *   x          [rows x cols] fp16 (dtype must be W8A8_F16; bf16's exponent
 *              range does not allow exact integer sums), 16-byte aligned.
 *   g, b       [cols] fp32 folded weight and bias, 16-byte aligned.
 *   eps        finite, >= 0.
 *   q, row_scale  outputs as in w8a8_scale_quant_rows.
 *   rows >= 0, cols % 16 == 0, cols <= 65536, cols >= 16 when rows > 0.
 * Errors: NULL, SHAPE, ALIGN, DTYPE (bf16 or unknown), ARG (eps negative, NaN or
 * infinite), HIP.
 */
w8a8_status_t w8a8_layernorm_quant_rows(const void* x, int dtype, int64_t rows, int64_t cols,
                                        const float* g, const float* b, float eps, int8_t* q,
                                        float* row_scale, hipStream_t stream);

/*
 * Step 4 alone (a diagnostic / test entry point): C = qa qb^T in exact int32.
 * Page section comparing GPTQ / AWQ / SmoothQuant: the INT8 operands are
 * multiplied directly, without dequantizing first.
 *
 *   qa  [M x K] int8 (per-token codes), 16-byte aligned.
 *   qb  [N x K] int8 (per-output-channel weight codes), 16-byte aligned.
 *   c   [M x N] int32 output, c[t, k] = sum_j qa[t, j] * qb[k, j], 16-byte aligned.
 *   M >= 0, N >= 0, 0 <= K <= W8A8_MAX_K, K % 16 == 0, N % 8 == 0.
 *   K == 0 writes zeros.  Codes must lie in [-127, 127] (as produced by
 *   w8a8_scale_quant_rows); a -128 code could overflow int32 at the largest K.
 * Errors: NULL, SHAPE, ALIGN, HIP.
 */
w8a8_status_t w8a8_gemm_i32(const int8_t* qa, const int8_t* qb, int32_t* c, int64_t M,
                            int64_t N, int64_t K, hipStream_t stream);

/*
 * Steps 4 + 5 fused: y[t, k] = out(fp32(fp32(C[t, k]) * sa[t]) * sb[k]) with C
 * as in w8a8_gemm_i32, each product one fp32 rounding, out() the round to
 * nearest even conversion to fp16 / bf16 (out_dtype).  The per-token and
 * per-channel scales factor out of the K sum, so the product stays in INT8.
 *
 *   sa  [M] fp32 per-token scales; sb [N] fp32 per-output-channel scales,
 *       16-byte aligned.
 *   y   [M x N] fp16/bf16 output, 16-byte aligned.
 *   Shape rules as w8a8_gemm_i32.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, HIP.
 */
w8a8_status_t w8a8_gemm_dequant(const int8_t* qa, const float* sa, const int8_t* qb,
                                const float* sb, void* y, int out_dtype, int64_t M, int64_t N,
                                int64_t K, hipStream_t stream);

/*
 * Dense 16-bit baseline: y = a b^T with fp16 or bf16 operands (dtype), fp32
 * accumulation and a round-to-nearest-even conversion of every accumulator
 * to dtype.  This is the FP16 product that the page measures W8A8 against
 * (section "パフォーマンスベンチマーク(A100-80GB)", speed table); it runs on the
 * 16-bit matrix cores with the same tiling as the INT8 kernel, so the two can
 * be timed against each other on the same shapes.
 *
 *   a  [M x K], b [N x K] (weight layout), y [M x N], all of dtype, 16-byte aligned.
 *   M >= 0, N >= 0, 0 <= K <= 1048576, K % 8 == 0, N % 8 == 0.  K == 0 writes zeros.
 *   The order of the fp32 accumulation is unspecified: before the final
 *   rounding each output is within K * 2^-24 * sum_j |a[t, j] b[k, j]| of the
 *   exact sum.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, HIP.
 */
w8a8_status_t w8a8_gemm_float(const void* a, const void* b, void* y, int dtype, int64_t M,
                              int64_t N, int64_t K, hipStream_t stream);

/*
 * FP8 variant of steps 2 and 3: as w8a8_scale_quant_rows, but each row is
 * quantized to OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits, largest finite value 448, no infinity) instead of INT8.  The jisaku.com
 * glossary page on quantization calibration (GPTQ / AWQ / SmoothQuant / QuaRot)
 * lists "FP8 SmoothQuant" among its methods, and the SmoothQuant page's FAQ
 * (FP4 and the Blackwell generation) notes that the smoothing transform
 * carries over to low-bit float formats.  For each row t:
 *   v_j = fp32(x[t, j]) * col_scale[j]
 *   m   = max_j |v_j|;  row_scale[t] = m / 448;  r = 448 / m
 *   q[t, j] = E4M3(v_j * r), round to nearest, ties to even
 * (|v_j * r| never exceeds 448 by more than fp32 rounding, so no code
 * saturates or is NaN).  A row with m == 0 gets row_scale 0 and +0 codes
 * (0x00, or 0x80 where v_j is -0).
 *
 *   q  [rows x cols] uint8 E4M3 codes, 16-byte aligned; other arguments and
 *      rules as w8a8_scale_quant_rows.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, HIP.
 */
w8a8_status_t w8a8_scale_quant_rows_e4m3(const void* x, int dtype, int64_t rows, int64_t cols,
                                         const float* col_scale, uint8_t* q, float* row_scale,
                                         hipStream_t stream);

/*
 * FP8 variant of steps 4 + 5: y[t, k] = out(fp32(fp32(C[t, k]) * sa[t]) * sb[k])
 * with C[t, k] = sum_j e4m3(qa[t, j]) * e4m3(qb[k, j]) accumulated in fp32 on
 * the FP8 matrix cores (pages as w8a8_scale_quant_rows_e4m3).  Each product of
 * two E4M3 values is exact; the order of the fp32 accumulation is
 * unspecified, so C is within K * 2^-24 * sum_j |a_j b_j| of the exact sum.
 *
 *   qa [M x K], qb [N x K] uint8 E4M3 codes (from w8a8_scale_quant_rows_e4m3;
 *   no NaN codes), 16-byte aligned; sa, sb, y, out_dtype and the shape rules
 *   as w8a8_gemm_dequant.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, HIP.
 */
w8a8_status_t w8a8_gemm_dequant_e4m3(const uint8_t* qa, const float* sa, const uint8_t* qb,
                                     const float* sb, void* y, int out_dtype, int64_t M, int64_t N,
                                     int64_t K, hipStream_t stream);

/* Bytes of workspace w8a8_linear needs for M tokens, K input and N output
 * channels: the INT8 activations and their per-token scales, then, where the
 * product is split along K (17 <= M <= 32 on fewer than 12288 output
 * channels with rows of 32 or more 256-byte pieces, K > 7936; 3 <= M <= 16 on
 * fewer than 2048 channels with rows of 64 or more, K > 16128), the int32
 * partial sums (S x M x N) and one 4-byte counter
 * per 64 output channels; each part 256-byte aligned.  0 for negative
 * sizes. */
size_t w8a8_linear_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * Runtime forward of one smoothed W8A8 linear layer (steps 3 + 4 + 5):
 * (qX, sx) = scale_quant_rows(x, inv_s) into the workspace, then
 * y = gemm_dequant(qX, sx, qw, sw).  No host sync.  On the split shapes
 * (decode batches on narrow layers with long rows; see
 * w8a8_linear_workspace_bytes) the product is split along K over more blocks
 * in the same launch: each block stores its exact int32 partial sums in the
 * workspace and the last block of each 64-channel group adds the S slices
 * (integer addition, exact) and applies the same epilogue, so y is
 * bit-identical to gemm_dequant's.  The quantization launch clears the
 * group counters, so the workspace needs no initialisation.
 *
 *   x          [M x K] fp16/bf16 activations (dtype; y has the same dtype).
 *   inv_s      [K] fp32 reciprocal smoothing factors, 16-byte aligned.
 *   qw, sw     [N x K] int8 folded weight codes and [N] fp32 scales (16-byte aligned).
 *   y          [M x N] output.
 *   workspace  device buffer of ws_bytes >= w8a8_linear_workspace_bytes(M, N, K),
 *              256-byte aligned; its contents on return are the INT8
 *              activations (M x K) followed by their scales.
 *   Shape rules: those of both steps (K % 16 == 0, K <= 65536, N % 8 == 0).
 * Errors: NULL, SHAPE, ALIGN, DTYPE, ARG (workspace too small), HIP.
 */
w8a8_status_t w8a8_linear(const void* x, int dtype, const float* inv_s, const int8_t* qw,
                          const float* sw, void* y, int64_t M, int64_t N, int64_t K,
                          void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * w8a8_linear without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation.  It computes exactly what w8a8_linear computes
 * (the same kernels, bit-identical y) and takes its scratch (the INT8
 * activations, their scales and the split-K partial sums) from a static
 * device array of W8A8_NOALLOC_SCRATCH_BYTES inside the library.  It calls
 * no allocating routine.  Every GPU the library runs on holds one such array
 * until the process ends.
 *
 *   Arguments and shape rules as w8a8_linear, without workspace / ws_bytes.
 *   Limit: w8a8_linear_workspace_bytes(M, N, K) <= W8A8_NOALLOC_SCRATCH_BYTES
 *   (for example 2048 tokens at K = 28672, or 4096 tokens at K = 8192, and
 *   every few-token call of up to 32 tokens at K <= 65536); larger calls return
 *   W8A8_ERR_TOO_LARGE and enqueue nothing.
 *   Sharing: all calls on one GPU share its array, which keeps the last
 *   call's contents (nothing in it needs to start at zero).  Calls that
 *   overlap on one GPU (concurrent streams, or host threads with the same
 *   current device) race on it: the caller serialises them, for example by
 *   issuing them on one stream.
 *   The first call on each device looks up the array's device address
 *   (hipGetSymbolAddress) and keeps it; make that first call outside graph
 *   capture.
 * Errors: those of w8a8_linear (ARG cannot occur), TOO_LARGE.
 */
#define W8A8_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
w8a8_status_t w8a8_linear_noalloc(const void* x, int dtype, const float* inv_s, const int8_t* qw,
                                  const float* sw, void* y, int64_t M, int64_t N, int64_t K,
                                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
