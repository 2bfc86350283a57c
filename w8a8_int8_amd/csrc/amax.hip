// Per-column running max|x| over a row-major fp16/bf16 matrix.
//
// Method: jisaku.com glossary page "SmoothQuant", section "ハイパーパラメータ α"
// (the smoothing factor needs max|X_j| over calibration tokens and max|W_j|
// over output channels).
//
// HBM-bound streaming kernel.  The absolute value of an fp16 or bf16 number is
// its bit pattern with the sign bit cleared, and for non-negative finite
// values the order of the bit patterns (as unsigned integers) is the order of
// the values.  So the whole reduction runs on integers: AND with 0x7fff7fff
// and a packed unsigned 16-bit max per pair of elements, exact by construction.
// The block result is widened to fp32 (exact) and folded into the output with
// an unsigned atomic max on the fp32 bit pattern, which orders non-negative
// floats the same way.
//
// Work split: a wave reads 64 lanes x 16 B = 512 consecutive columns of one
// row per load (fully coalesced 1 KiB), the 4 waves of a block take
// interleaved rows of the same 512-column strip, and each lane keeps U loads
// in flight.  Blocks split the rows so the grid has a few thousand blocks.
#include "common.h"

namespace w8a8 {

namespace {

constexpr int kAmaxThreads = 256;
constexpr int kAmaxWaves = kAmaxThreads / kWave;
constexpr int kAmaxUnroll = 8;

__device__ __forceinline__ unsigned pmax16(unsigned a, unsigned b) {
  u16x2 x = __builtin_bit_cast(u16x2, a);
  u16x2 y = __builtin_bit_cast(u16x2, b);
  return __builtin_bit_cast(unsigned, __builtin_elementwise_max(x, y));
}

template <bool BF16>
__global__ __launch_bounds__(kAmaxThreads) void k_channel_amax(const v4u* __restrict__ x,
                                                               int64_t rows, int64_t cols8,
                                                               int64_t rows_per_block,
                                                               unsigned* __restrict__ amax_bits) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int64_t chunk = (int64_t)blockIdx.x * kWave + lane;  // 16-byte column chunk
  const int64_t r_begin = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r_end = min(rows, r_begin + rows_per_block);
  const bool active = chunk < cols8;

  unsigned m0 = 0, m1 = 0, m2 = 0, m3 = 0;
  if (active) {
    const v4u* p = x + chunk;
    int64_t r = r_begin + wave;
    // full groups of U rows per wave, no per-load bounds test
    for (; r + (int64_t)(kAmaxUnroll - 1) * kAmaxWaves < r_end; r += kAmaxUnroll * kAmaxWaves) {
      v4u v[kAmaxUnroll];
#pragma unroll
      for (int u = 0; u < kAmaxUnroll; ++u)
        v[u] = __builtin_nontemporal_load(p + (r + (int64_t)u * kAmaxWaves) * cols8);
#pragma unroll
      for (int u = 0; u < kAmaxUnroll; ++u) {
        m0 = pmax16(m0, v[u].x & 0x7fff7fffu);
        m1 = pmax16(m1, v[u].y & 0x7fff7fffu);
        m2 = pmax16(m2, v[u].z & 0x7fff7fffu);
        m3 = pmax16(m3, v[u].w & 0x7fff7fffu);
      }
    }
    for (; r < r_end; r += kAmaxWaves) {
      v4u v = __builtin_nontemporal_load(p + r * cols8);
      m0 = pmax16(m0, v.x & 0x7fff7fffu);
      m1 = pmax16(m1, v.y & 0x7fff7fffu);
      m2 = pmax16(m2, v.z & 0x7fff7fffu);
      m3 = pmax16(m3, v.w & 0x7fff7fffu);
    }
  }

  // combine the waves of the block through LDS
  __shared__ uint4 part[kAmaxWaves][kWave];
  part[wave][lane] = make_uint4(m0, m1, m2, m3);
  __syncthreads();
  if (wave != 0 || !active) return;
#pragma unroll
  for (int w = 1; w < kAmaxWaves; ++w) {
    uint4 o = part[w][lane];
    m0 = pmax16(m0, o.x);
    m1 = pmax16(m1, o.y);
    m2 = pmax16(m2, o.z);
    m3 = pmax16(m3, o.w);
  }
  const unsigned m[4] = {m0, m1, m2, m3};
  unsigned* out = amax_bits + chunk * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const unsigned short bits = (unsigned short)(m[i] >> (16 * h));
      if (bits == 0) continue;  // +0 never raises a non-negative running max
      const float f = widen16(bits, BF16);
      atomicMax(out + 2 * i + h, __float_as_uint(f));
    }
  }
}

}  // namespace

hipError_t launch_channel_amax(const void* x, bool bf16, int64_t rows, int64_t cols, float* amax,
                               hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int64_t cols8 = cols / 8;
  const int64_t strips = (cols8 + kWave - 1) / kWave;
  // aim for ~4096 blocks; each block covers at least one unrolled group of rows
  const int64_t min_rows = (int64_t)kAmaxUnroll * kAmaxWaves;
  int64_t row_blocks = (4096 + strips - 1) / strips;
  int64_t rpb = (rows + row_blocks - 1) / row_blocks;
  rpb = ((rpb + min_rows - 1) / min_rows) * min_rows;
  row_blocks = (rows + rpb - 1) / rpb;
  if (row_blocks > 65535) {
    row_blocks = 65535;
    rpb = (rows + row_blocks - 1) / row_blocks;
    rpb = ((rpb + min_rows - 1) / min_rows) * min_rows;
    row_blocks = (rows + rpb - 1) / rpb;
  }
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
