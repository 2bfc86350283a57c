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
// Work split: a block owns a strip of 64 columns (128 bytes of every row) and
// a tall range of rows.  One wave load covers 8 rows x 128 B (8 lanes per row,
// full cache lines); the 4 waves take interleaved groups of 8 rows and each
// lane keeps U loads in flight.  At the end the lanes that hold the same
// columns are folded with cross-lane max, then the 4 waves through LDS, and
// 64 lanes issue one coalesced atomic max each (one per column).  Row ranges
// are sized so the grid has about 1024 blocks while each column receives at
// most a few dozen atomics: the atomics, not the loads, are what a finer
// split would pay for.
#include "common.h"

namespace w8a8 {

namespace {

constexpr int kAmaxThreads = 256;
constexpr int kAmaxWaves = kAmaxThreads / kWave;
constexpr int kAmaxUnroll = 8;
constexpr int kRowsPerLoad = 8;                                     // rows per wave load
constexpr int kRowsPerGroup = kRowsPerLoad * kAmaxWaves;            // 32 rows per block step
constexpr int kRowsPerBatch = kRowsPerGroup * kAmaxUnroll;          // 256 rows in flight

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
  const int sub = lane / 8;                                   // row within a wave load
  const int64_t chunk = (int64_t)blockIdx.x * 8 + (lane % 8);  // 16-byte column chunk
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
  // fold the 8 row lanes that hold the same chunk (lanes l, l^8, l^16, l^32)
#pragma unroll
  for (int off = 8; off < kWave; off <<= 1) {
    m.x = pmax16(m.x, (unsigned)__shfl_xor((int)m.x, off, kWave));
    m.y = pmax16(m.y, (unsigned)__shfl_xor((int)m.y, off, kWave));
    m.z = pmax16(m.z, (unsigned)__shfl_xor((int)m.z, off, kWave));
    m.w = pmax16(m.w, (unsigned)__shfl_xor((int)m.w, off, kWave));
  }
  // fold the waves through LDS: wave w's lanes 0..7 hold its 64 column maxima
  __shared__ unsigned short part[kAmaxWaves][64];
  if (lane < 8) {
    const unsigned w4[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      part[wave][lane * 8 + 2 * i] = (unsigned short)(w4[i] & 0xffffu);
      part[wave][lane * 8 + 2 * i + 1] = (unsigned short)(w4[i] >> 16);
    }
  }
  __syncthreads();
  if (wave != 0) return;
  unsigned short b = part[0][lane];
#pragma unroll
  for (int w = 1; w < kAmaxWaves; ++w) b = max(b, part[w][lane]);
  const int64_t col = (int64_t)blockIdx.x * 64 + lane;
  if (col < cols8 * 8 && b != 0)  // +0 never raises a non-negative running max
    atomicMax(amax_bits + col, __float_as_uint(widen16(b, BF16)));
}

}  // namespace

hipError_t launch_channel_amax(const void* x, bool bf16, int64_t rows, int64_t cols, float* amax,
                               hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int64_t cols8 = cols / 8;
  const int64_t strips = (cols8 + 7) / 8;
  // about 1024 blocks, at most 32 row ranges per strip, at least one 32-row step each
  int64_t row_blocks = (1024 + strips - 1) / strips;
  if (row_blocks > 32) row_blocks = 32;
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
