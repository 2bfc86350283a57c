// Per-column running max|x| over a row-major fp16/bf16 matrix.
//
// Method: jisaku.com glossary page "SmoothQuant", section "ハイパーパラメータ α"
// (the smoothing factor needs max|X_j| over calibration tokens and max|W_j|
// over output channels).
//
// HBM-bound streaming kernel.  The absolute value of an fp16 or bf16 number is
// its bit pattern with the sign bit cleared, and for non-negative finite
// values the order of the bit patterns (as unsigned integers) is the order of
// the values.  So the reduction runs on integers: AND with 0x7fff7fff and a
// packed unsigned 16-bit max per pair of elements, exact by construction.
// The block result is widened to fp32 (exact) and folded into the output with
// an unsigned atomic max on the fp32 bit pattern, which orders non-negative
// floats the same way.
//
// Work split: a block owns a strip of 256 columns (512 bytes of every row)
// and a tall range of rows.  One wave load covers 2 rows x 512 B (32 lanes
// per row); the 4 waves take interleaved pairs of rows and each lane keeps U
// loads in flight.  At the end the two lanes that hold the same columns are
// folded with a cross-lane max, then the 4 waves through LDS, and the block
// issues one coalesced atomic max per column.  Row ranges are sized so the
// grid has about 1024 blocks while each column receives at most 128 atomics.
// Measured on fp16 weights of 4096 to 57344 rows: 512-byte row pieces stream
// at 5.5-6.4 TB/s where 128-byte pieces (a strip of 64 columns) reached
// 5.0-5.6 TB/s.
//
// k_calibrate_smooth runs the same strip code over a calibration batch and a
// weight in one grid and forms the smoothing factors at the end of each strip
// (its comment gives the cross-block protocol); k_calibrate_smooth_layers
// does that for several layers in one flat grid.
#include "common.h"
#include "smooth_factor.h"

namespace w8a8 {

namespace {

constexpr int kAmaxThreads = 256;
constexpr int kAmaxWaves = kAmaxThreads / kWave;
constexpr int kAmaxUnroll = 8;                                      // loads in flight per lane
constexpr int kFusedUnroll = 16;                                    // ... in k_calibrate_smooth
constexpr int kLanesPerRow = 32;                                    // 16-byte chunks of a row piece
constexpr int kStripCols = kLanesPerRow * 8;                        // 256 columns per block
constexpr int kRowsPerLoad = kWave / kLanesPerRow;                  // 2 rows per wave load
constexpr int kRowsPerGroup = kRowsPerLoad * kAmaxWaves;            // 8 rows per block step
constexpr int kMaxRowRanges = 128;                                  // atomics per column
static_assert(kStripCols == kAmaxThreads, "one column per thread in the fold");

__device__ __forceinline__ unsigned pmax16(unsigned a, unsigned b) {
  u16x2 x = __builtin_bit_cast(u16x2, a);
  u16x2 y = __builtin_bit_cast(u16x2, b);
  return __builtin_bit_cast(unsigned, __builtin_elementwise_max(x, y));
}

__device__ __forceinline__ v4u vmax(v4u m, v4u v) {
  return v4u{pmax16(m.x, v.x & 0x7fff7fffu), pmax16(m.y, v.y & 0x7fff7fffu),
             pmax16(m.z, v.z & 0x7fff7fffu), pmax16(m.w, v.w & 0x7fff7fffu)};
}

// The maximum of |x| over rows [r_begin, r_end) of the block's 256-column
// strip, as a 16-bit magnitude pattern, for the column of this thread
// (column blockIdx.x * 256 + threadIdx.x); 0 for columns past the end.
// U loads in flight per lane, U * kRowsPerGroup rows per batch.
template <bool BF16, int U>
__device__ __forceinline__ unsigned short strip_max(const v4u* __restrict__ x, int64_t cols8,
                                                    int64_t strip, int64_t r_begin, int64_t r_end) {
  constexpr int kRowsPerBatch = kRowsPerGroup * U;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int sub = lane / kLanesPerRow;  // row within a wave load
  const int64_t chunk = strip * kLanesPerRow + (lane % kLanesPerRow);  // 16-byte chunk
  const bool active = chunk < cols8;

  v4u m = {0u, 0u, 0u, 0u};
  if (active) {
    const v4u* p = x + chunk;
    int64_t r = r_begin + wave * kRowsPerLoad + sub;
    // full batches: U loads per lane in flight, no per-load bounds test
    for (; r + (int64_t)(U - 1) * kRowsPerGroup < r_end; r += kRowsPerBatch) {
      v4u v[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        v[u] = __builtin_nontemporal_load(p + (r + (int64_t)u * kRowsPerGroup) * cols8);
#pragma unroll
      for (int u = 0; u < U; ++u) m = vmax(m, v[u]);
    }
    // the last partial batch: all of its loads issued together as well (a
    // row-by-row tail would pay one memory round trip per row group)
    if (r < r_end) {
      v4u v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t ru = r + (int64_t)u * kRowsPerGroup;
        v[u] = ru < r_end ? __builtin_nontemporal_load(p + ru * cols8) : v4u{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) m = vmax(m, v[u]);
    }
  }
  // fold the lanes that hold the same chunk (lanes l and l ^ 32)
#pragma unroll
  for (int off = kLanesPerRow; off < kWave; off <<= 1) {
    m.x = pmax16(m.x, (unsigned)__shfl_xor((int)m.x, off, kWave));
    m.y = pmax16(m.y, (unsigned)__shfl_xor((int)m.y, off, kWave));
    m.z = pmax16(m.z, (unsigned)__shfl_xor((int)m.z, off, kWave));
    m.w = pmax16(m.w, (unsigned)__shfl_xor((int)m.w, off, kWave));
  }
  // fold the waves through LDS: wave w's lanes 0..31 hold its 256 column maxima
  __shared__ unsigned short part[kAmaxWaves][kStripCols];
  if (lane < kLanesPerRow) {
    const unsigned w4[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      part[wave][lane * 8 + 2 * i] = (unsigned short)(w4[i] & 0xffffu);
      part[wave][lane * 8 + 2 * i + 1] = (unsigned short)(w4[i] >> 16);
    }
  }
  __syncthreads();
  // one column per thread (kStripCols == kAmaxThreads)
  const int c = threadIdx.x;
  unsigned short b = part[0][c];
#pragma unroll
  for (int w = 1; w < kAmaxWaves; ++w) b = max(b, part[w][c]);
  return b;
}

template <bool BF16>
__global__ __launch_bounds__(kAmaxThreads) void k_channel_amax(const v4u* __restrict__ x,
                                                               int64_t rows, int64_t cols8,
                                                               int64_t rows_per_block,
                                                               unsigned* __restrict__ amax_bits) {
  const int64_t r_begin = (int64_t)blockIdx.y * rows_per_block;
  const unsigned short b =
      strip_max<BF16, kAmaxUnroll>(x, cols8, blockIdx.x, r_begin, min(rows, r_begin + rows_per_block));
  const int64_t col = (int64_t)blockIdx.x * kStripCols + threadIdx.x;
  if (col < cols8 * 8 && b != 0)  // +0 never raises a non-negative running max
    atomicMax(amax_bits + col, __float_as_uint(widen16(b, BF16)));
}

// One launch for a layer's calibration fold, weight maxima and smoothing
// factors.  Row blocks y < rb_x take rows of the calibration batch xc and
// fold into the running amax_x; the others take rows of the weight w and fold
// into the accumulator acc_w (zero on entry).  Each strip counts its arriving
// blocks; the last block of a strip forms s and inv_s of its 256 channels.
//
// Cross-block order without fences: every maximum and every count is a
// device-scope atomic, performed at the one point of coherence that all eight
// XCDs share (the same property the running max of k_channel_amax relies on).
// A thread waits for its maximum's returned value before the block counts
// itself, so when the count reaches the strip's total every maximum of the
// strip has been performed; the last block then reads the maxima with atomic
// read-modify-writes at that same point: amax_x by a compare-and-swap that
// never matches, and acc_w by an exchange with 0, which also leaves the
// accumulator zero for the next call.
// It resets its counter the same way.  Its plain stores (amax_w, s, inv_s)
// are for later kernels.
// One layer's part of a calibrate-smooth launch: the two matrices, their row
// split and the outputs.  Row blocks yb < rb_x take rows of the calibration
// batch, the others rows of the weight; the layer has strips x rb blocks.
struct CalLayer {
  const v4u* xc;
  const v4u* w;
  unsigned* amax_x_bits;
  unsigned* acc_w_bits;
  unsigned* arrivals;
  float* amax_w;
  float* s;
  float* inv_s;
  int64_t cal_rows, w_rows, cols8, rows_per_block, rb_x, rb, strips, block0;
  double alpha;
};

template <bool BF16>
__device__ __forceinline__ void calibrate_block(const CalLayer& g, int64_t strip, int64_t yb) {
  const bool cal = yb < g.rb_x;
  const v4u* x = cal ? g.xc : g.w;
  const int64_t rows = cal ? g.cal_rows : g.w_rows;
  const int64_t r_begin = (cal ? yb : yb - g.rb_x) * g.rows_per_block;
  const unsigned short b = strip_max<BF16, kFusedUnroll>(x, g.cols8, strip, r_begin,
                                                         min(rows, r_begin + g.rows_per_block));
  const int c = threadIdx.x;
  const int64_t col = strip * kStripCols + c;
  const bool live = col < g.cols8 * 8;
  unsigned seen = 0u;
  if (live && b != 0)
    seen = atomicMax((cal ? g.amax_x_bits : g.acc_w_bits) + col, __float_as_uint(widen16(b, BF16)));
  // the returned value has arrived, so this thread's maximum has been
  // performed, before the block is counted
  asm volatile("s_waitcnt vmcnt(0)" : : "v"(seen) : "memory");
  __shared__ unsigned last;
  __syncthreads();
  if (c == 0) last = atomicAdd(g.arrivals + strip, 1u) == (unsigned)g.rb - 1 ? 1u : 0u;
  __syncthreads();
  if (!last) return;
  if (live) {
    // a compare-and-swap that never matches (the pattern is a NaN, never
    // stored) reads the value as a read-modify-write, like the maxima
    const float ax = __uint_as_float(atomicCAS(g.amax_x_bits + col, 0xffffffffu, 0xffffffffu));
    const float aw = __uint_as_float(atomicExch(g.acc_w_bits + col, 0u));
    g.amax_w[col] = aw;
    float sj, ij;
    smooth_factor(ax, aw, g.alpha, sj, ij);
    g.s[col] = sj;
    g.inv_s[col] = ij;
  }
  if (c == 0) atomicExch(g.arrivals + strip, 0u);
}

template <bool BF16>
__global__ __launch_bounds__(kAmaxThreads) void k_calibrate_smooth(const CalLayer g) {
  calibrate_block<BF16>(g, blockIdx.x, blockIdx.y);
}

// Several layers in one launch: a flat grid, the layers' blocks one after
// another in the order of the one-layer grid (strip fastest), so every layer
// gets the same blocks, rows and protocol as its own launch would.  The
// layers are independent (their own inputs, outputs and scratch), so their
// blocks run side by side and one layer's tail (the last block of each strip
// forming s) overlaps the others' streaming.
constexpr int kMaxCalLayers = 8;
struct CalLayers {
  CalLayer l[kMaxCalLayers];
  int n;
};

template <bool BF16>
__global__ __launch_bounds__(kAmaxThreads) void k_calibrate_smooth_layers(const CalLayers gs) {
  const int64_t b = blockIdx.x;
  int i = 0;
  while (i + 1 < gs.n && b >= gs.l[i + 1].block0) ++i;
  const CalLayer& g = gs.l[i];
  const int64_t local = b - g.block0;
  calibrate_block<BF16>(g, local % g.strips, local / g.strips);
}

}  // namespace

hipError_t launch_channel_amax(const void* x, bool bf16, int64_t rows, int64_t cols, float* amax,
                               hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int64_t cols8 = cols / 8;
  const int64_t strips = (cols8 + kLanesPerRow - 1) / kLanesPerRow;
  // about 1024 blocks, at most kMaxRowRanges row ranges per strip, at least
  // one block step of rows each
  int64_t row_blocks = (1024 + strips - 1) / strips;
  if (row_blocks > kMaxRowRanges) row_blocks = kMaxRowRanges;
  const int64_t max_rb = (rows + kRowsPerGroup - 1) / kRowsPerGroup;
  if (row_blocks > max_rb) row_blocks = max_rb;
  if (row_blocks < 1) row_blocks = 1;
  int64_t rpb = (rows + row_blocks - 1) / row_blocks;
  rpb = (rpb + kRowsPerGroup - 1) / kRowsPerGroup * kRowsPerGroup;
  row_blocks = (rows + rpb - 1) / rpb;
  dim3 grid((unsigned)strips, (unsigned)row_blocks);
  if (bf16)
    hipLaunchKernelGGL(k_channel_amax<true>, grid, dim3(kAmaxThreads), 0, st,
                       (const v4u*)x, rows, cols8, rpb, (unsigned*)amax);
  else
    hipLaunchKernelGGL(k_channel_amax<false>, grid, dim3(kAmaxThreads), 0, st,
                       (const v4u*)x, rows, cols8, rpb, (unsigned*)amax);
  return hipGetLastError();
}

size_t calibrate_smooth_scratch_bytes(int64_t K) {
  if (K <= 0) return 0;
  const int64_t strips = (K / 8 + kLanesPerRow - 1) / kLanesPerRow;
  return (size_t)((4 * K + 255) / 256 * 256 + 4 * strips);
}

namespace {

// The grid of one layer: about 448 blocks over both matrices, the same rows
// per block for both, with 16 loads in flight per lane.  Measured on the
// Llama-2-7B layers: more blocks lose time to the arrival protocol (each
// strip's counter and each column's maximum take one atomic per row block,
// one after another), fewer lose streaming rate on the larger weights.
CalLayer plan_calibrate(const void* xc, int64_t cal_rows, const void* w, int64_t w_rows, int64_t K,
                        double alpha, float* amax_x, float* amax_w, float* s, float* inv_s,
                        void* scratch) {
  CalLayer g;
  g.cols8 = K / 8;
  g.strips = (g.cols8 + kLanesPerRow - 1) / kLanesPerRow;
  const int64_t target = (448 + g.strips - 1) / g.strips;
  int64_t rpb = (cal_rows + w_rows + target - 1) / target;
  rpb = (rpb + kRowsPerGroup - 1) / kRowsPerGroup * kRowsPerGroup;
  if (rpb < kRowsPerGroup) rpb = kRowsPerGroup;
  g.rows_per_block = rpb;
  g.rb_x = (cal_rows + rpb - 1) / rpb;
  int64_t rb_w = (w_rows + rpb - 1) / rpb;
  if (g.rb_x + rb_w == 0) rb_w = 1;  // no rows at all: one empty block per strip still forms s
  g.rb = g.rb_x + rb_w;
  g.xc = (const v4u*)xc;
  g.w = (const v4u*)w;
  g.cal_rows = cal_rows;
  g.w_rows = w_rows;
  g.alpha = alpha;
  g.amax_x_bits = (unsigned*)amax_x;
  g.acc_w_bits = (unsigned*)scratch;
  g.arrivals = g.acc_w_bits + (K + 63) / 64 * 64;
  g.amax_w = amax_w;
  g.s = s;
  g.inv_s = inv_s;
  g.block0 = 0;
  return g;
}

}  // namespace

hipError_t launch_calibrate_smooth(const void* xc, int64_t cal_rows, const void* w,
                                   int64_t w_rows, bool bf16, int64_t K, double alpha,
                                   float* amax_x, float* amax_w, float* s, float* inv_s,
                                   void* scratch, hipStream_t st) {
  if (K == 0) return hipSuccess;
  const CalLayer g = plan_calibrate(xc, cal_rows, w, w_rows, K, alpha, amax_x, amax_w, s, inv_s,
                                    scratch);
  const dim3 grid((unsigned)g.strips, (unsigned)g.rb);
  if (bf16)
    hipLaunchKernelGGL(k_calibrate_smooth<true>, grid, dim3(kAmaxThreads), 0, st, g);
  else
    hipLaunchKernelGGL(k_calibrate_smooth<false>, grid, dim3(kAmaxThreads), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_calibrate_smooth_layers(int n, const CalibLayerArgs* a, bool bf16,
                                          hipStream_t st) {
  for (int i0 = 0; i0 < n; i0 += kMaxCalLayers) {
    CalLayers gs;
    gs.n = 0;
    int64_t blocks = 0;
    for (int i = i0; i < n && i < i0 + kMaxCalLayers; ++i) {
      CalLayer g = plan_calibrate(a[i].x_cal, a[i].cal_rows, a[i].w, a[i].n, a[i].k, a[i].alpha,
                                  a[i].amax_x, a[i].amax_w, a[i].s, a[i].inv_s, a[i].scratch);
      g.block0 = blocks;
      blocks += g.strips * g.rb;
      gs.l[gs.n++] = g;
    }
    if (bf16)
      hipLaunchKernelGGL(k_calibrate_smooth_layers<true>, dim3((unsigned)blocks), dim3(kAmaxThreads),
                         0, st, gs);
    else
      hipLaunchKernelGGL(k_calibrate_smooth_layers<false>, dim3((unsigned)blocks),
                         dim3(kAmaxThreads), 0, st, gs);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace w8a8
