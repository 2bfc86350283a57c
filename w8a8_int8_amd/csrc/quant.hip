// Per-column scale followed by per-row symmetric INT8 quantization.
//
// Method: jisaku.com glossary page "SmoothQuant", section "平滑化変換の数学"
// (X~ = X s^-1, W~ = s W) and section "Activation外れ値問題" (INT8 range); the
// symmetric grid [-127, 127], per-row scales and round-half-even are the
// readings stated in the library header.  Per row t:
//   v_j = fp32(x[t, j]) * c_j;  m = max_j |v_j|;  delta = m / 127;  r = 127 / m;
//   q_j = clamp(rint(v_j * r), -127, 127)
// Each arrow is one IEEE fp32 operation (no contraction; there is no add to
// fuse), divisions are the correctly rounded ones, rint is round-half-even.
//
// HBM-bound: 2 B read + 1 B written per element (+ 4 B per row).  A group of
// G threads (a multiple of the 64-wide wavefront, at most 1024) owns a row:
// thread g holds the 16-byte chunks g, g + G, ... (CPT of them), so every wave
// load is 1 KiB of consecutive bytes and every wave store 512 B.  The row is
// kept in registers between the max pass and the quantize pass, so x is read
// from HBM exactly once.  A block handles R consecutive rows with the same
// column ownership: the column scales are loaded once per block (they stay
// L2 resident) and the R rows' loads are all in flight before the first
// reduction.  The row max is a wave-level butterfly followed by one LDS round
// across the waves of the block.
#include "common.h"

namespace w8a8 {

namespace {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ unsigned pack4(float a, float b, float c, float d) {
  const unsigned q0 = (unsigned)(int)a & 0xffu, q1 = (unsigned)(int)b & 0xffu;
  const unsigned q2 = (unsigned)(int)c & 0xffu, q3 = (unsigned)(int)d & 0xffu;
  return q0 | (q1 << 8) | (q2 << 16) | (q3 << 24);
}

__device__ __forceinline__ float code(float v, float r) {
  return fminf(fmaxf(rintf(v * r), -127.0f), 127.0f);
}

template <int CPT, int R, bool BF16>
__global__ __launch_bounds__(1024) void k_scale_quant_rows(const v4u* __restrict__ x, int64_t rows,
                                                           int cols8,
                                                           const float4* __restrict__ col_scale,
                                                           uint2* __restrict__ q,
                                                           float* __restrict__ row_scale) {
  const int tid = threadIdx.x;
  const int G = blockDim.x;
  const int lane = tid % kWave, wave = tid / kWave, nwaves = G / kWave;
  const int64_t row0 = (int64_t)blockIdx.x * R;

  v4u xv[R][CPT];
  float sc[CPT][8];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = i * G + tid;
    if (c < cols8) {
      const float4 lo = col_scale[2 * c], hi = col_scale[2 * c + 1];
      sc[i][0] = lo.x; sc[i][1] = lo.y; sc[i][2] = lo.z; sc[i][3] = lo.w;
      sc[i][4] = hi.x; sc[i][5] = hi.y; sc[i][6] = hi.z; sc[i][7] = hi.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) sc[i][e] = 0.0f;
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = i * G + tid;
      if (c < cols8 && row0 + r < rows)
        xv[r][i] = __builtin_nontemporal_load(x + (row0 + r) * cols8 + c);
      else
        xv[r][i] = v4u{0u, 0u, 0u, 0u};
    }
  }

  // pass 1: row max of |x * c|
  float m[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float mr = 0.0f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const unsigned short h = (unsigned short)(xv[r][i][e / 2] >> (16 * (e % 2)));
        mr = fmaxf(mr, fabsf(widen16(h, BF16) * sc[i][e]));
      }
    }
    m[r] = wave_max(mr);
  }
  __shared__ float red[R][16];
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) red[r][wave] = m[r];
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float mr = red[r][0];
    for (int w = 1; w < nwaves; ++w) mr = fmaxf(mr, red[r][w]);
    m[r] = mr;
  }

  // pass 2: codes
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = row0 + r;
    if (row >= rows) break;
    const float mr = m[r];
    const float rcp = mr > 0.0f ? 127.0f / mr : 0.0f;
    if (tid == 0) row_scale[row] = mr > 0.0f ? mr / 127.0f : 0.0f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = i * G + tid;
      if (c >= cols8) continue;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const unsigned short h = (unsigned short)(xv[r][i][e / 2] >> (16 * (e % 2)));
        v[e] = code(widen16(h, BF16) * sc[i][e], rcp);
      }
      uint2 o;
      o.x = pack4(v[0], v[1], v[2], v[3]);
      o.y = pack4(v[4], v[5], v[6], v[7]);
      q[row * cols8 + c] = o;
    }
  }
}

template <int CPT, int R>
hipError_t launch_cfg(const void* x, bool bf16, int64_t rows, int cols8, int G,
                      const float* col_scale, int8_t* q, float* row_scale, hipStream_t st) {
  const unsigned blocks = (unsigned)((rows + R - 1) / R);
  if (bf16)
    hipLaunchKernelGGL((k_scale_quant_rows<CPT, R, true>), dim3(blocks), dim3(G), 0, st,
                       (const v4u*)x, rows, cols8, (const float4*)col_scale, (uint2*)q, row_scale);
  else
    hipLaunchKernelGGL((k_scale_quant_rows<CPT, R, false>), dim3(blocks), dim3(G), 0, st,
                       (const v4u*)x, rows, cols8, (const float4*)col_scale, (uint2*)q, row_scale);
  return hipGetLastError();
}

template <int CPT>
hipError_t launch_rows(const void* x, bool bf16, int64_t rows, int cols8, int G,
                       const float* col_scale, int8_t* q, float* row_scale, hipStream_t st) {
  // rows per block: amortize the column-scale loads while keeping >= ~1024 blocks
  if (rows >= 4 * 1024)
    return launch_cfg<CPT, 4>(x, bf16, rows, cols8, G, col_scale, q, row_scale, st);
  if (rows >= 2 * 1024)
    return launch_cfg<CPT, 2>(x, bf16, rows, cols8, G, col_scale, q, row_scale, st);
  return launch_cfg<CPT, 1>(x, bf16, rows, cols8, G, col_scale, q, row_scale, st);
}

}  // namespace

hipError_t launch_scale_quant_rows(const void* x, bool bf16, int64_t rows, int64_t cols,
                                   const float* col_scale, int8_t* q, float* row_scale,
                                   hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int cols8 = (int)(cols / 8);
  // threads per row: about 4 chunks each, a whole number of waves, at most 1024
  int G = (cols8 + 3) / 4;
  G = ((G + kWave - 1) / kWave) * kWave;
  if (G < kWave) G = kWave;
  if (G > 1024) G = 1024;
  const int cpt = (cols8 + G - 1) / G;
  switch (cpt <= 1 ? 1 : cpt) {
    case 1: return launch_rows<1>(x, bf16, rows, cols8, G, col_scale, q, row_scale, st);
    case 2: return launch_rows<2>(x, bf16, rows, cols8, G, col_scale, q, row_scale, st);
    case 3: return launch_rows<3>(x, bf16, rows, cols8, G, col_scale, q, row_scale, st);
    case 4: return launch_rows<4>(x, bf16, rows, cols8, G, col_scale, q, row_scale, st);
    case 5: return launch_rows<5>(x, bf16, rows, cols8, G, col_scale, q, row_scale, st);
    case 6: return launch_rows<6>(x, bf16, rows, cols8, G, col_scale, q, row_scale, st);
    case 7: return launch_rows<7>(x, bf16, rows, cols8, G, col_scale, q, row_scale, st);
    case 8: return launch_rows<8>(x, bf16, rows, cols8, G, col_scale, q, row_scale, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace w8a8
