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
#include "common.h"

namespace w8a8 {

namespace {

constexpr int kAmaxThreads = 256;
constexpr int kAmaxWaves = kAmaxThreads / kWave;
constexpr int kAmaxUnroll = 8;
constexpr int kLanesPerRow = 32;                                    // 16-byte chunks of a row piece
constexpr int kStripCols = kLanesPerRow * 8;                        // 256 columns per block
constexpr int kRowsPerLoad = kWave / kLanesPerRow;                  // 2 rows per wave load
constexpr int kRowsPerGroup = kRowsPerLoad * kAmaxWaves;            // 8 rows per block step
constexpr int kRowsPerBatch = kRowsPerGroup * kAmaxUnroll;          // 64 rows in flight
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

template <bool BF16>
__global__ __launch_bounds__(kAmaxThreads) void k_channel_amax(const v4u* __restrict__ x,
                                                               int64_t rows, int64_t cols8,
                                                               int64_t rows_per_block,
                                                               unsigned* __restrict__ amax_bits) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int sub = lane / kLanesPerRow;  // row within a wave load
  const int64_t chunk = (int64_t)blockIdx.x * kLanesPerRow + (lane % kLanesPerRow);  // 16-byte chunk
  const int64_t r_begin = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r_end = min(rows, r_begin + rows_per_block);
  const bool active = chunk < cols8;

  v4u m = {0u, 0u, 0u, 0u};
  if (active) {
    const v4u* p = x + chunk;
    int64_t r = r_begin + wave * kRowsPerLoad + sub;
    // full batches: U loads per lane in flight, no per-load bounds test
    for (; r + (int64_t)(kAmaxUnroll - 1) * kRowsPerGroup < r_end; r += kRowsPerBatch) {
      v4u v[kAmaxUnroll];
#pragma unroll
      for (int u = 0; u < kAmaxUnroll; ++u)
        v[u] = __builtin_nontemporal_load(p + (r + (int64_t)u * kRowsPerGroup) * cols8);
#pragma unroll
      for (int u = 0; u < kAmaxUnroll; ++u) m = vmax(m, v[u]);
    }
    // the last partial batch: all of its loads issued together as well (a
    // row-by-row tail would pay one memory round trip per row group)
    if (r < r_end) {
      v4u v[kAmaxUnroll];
#pragma unroll
      for (int u = 0; u < kAmaxUnroll; ++u) {
        const int64_t ru = r + (int64_t)u * kRowsPerGroup;
        v[u] = ru < r_end ? __builtin_nontemporal_load(p + ru * cols8) : v4u{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kAmaxUnroll; ++u) m = vmax(m, v[u]);
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
  const int64_t col = (int64_t)blockIdx.x * kStripCols + c;
  if (col < cols8 * 8 && b != 0)  // +0 never raises a non-negative running max
    atomicMax(amax_bits + col, __float_as_uint(widen16(b, BF16)));
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

}  // namespace w8a8
