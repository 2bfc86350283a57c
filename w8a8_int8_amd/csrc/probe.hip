// Hardware probes of the GPU, for the roofline figures of the benchmark.
// They are not part of the W8A8 path: libw8a8_probe.so is a separate
// library that only bench.py --ceilings loads.
//
//   w8a8probe_read   read-only streaming: every byte of a buffer read once
//                    with 16-byte loads, 8 in flight per lane, folded into a
//                    register (the practical ceiling of the amax kernels)
//   w8a8probe_copy   a plain copy, 16 bytes per lane (read + write)
//   w8a8probe_mfma   v_mfma_i32_32x32x32_i8 or _16x16x64_i8 back to back from registers
//                    (no memory traffic), 4 or 8 waves per block, with each block's
//                    shader-clock cycles (s_memtime) and 100 MHz wall-clock
//                    ticks (s_memrealtime) recorded around its loop, so the
//                    clock the matrix cores run at follows from the two
//
// Error convention: 0 on success, 1 for a bad argument (checked on the host
// before any launch), 2 when the launch fails.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kUnroll = 8;

// chunked = 0: grid-stride (each step of the whole grid reads one contiguous
// stripe); chunked = 1: each block reads its own contiguous share, 4 KiB per
// block load, kUnroll loads in flight.
__global__ __launch_bounds__(256) void k_read(const v4i* __restrict__ src, int64_t n16,
                                              int chunked, unsigned* __restrict__ sink) {
  v4i acc = {0, 0, 0, 0};
  int64_t i, end, stride;
  if (chunked) {
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    i = (int64_t)blockIdx.x * per + threadIdx.x;
    end = min(n16, (int64_t)(blockIdx.x + 1) * per);
    stride = 256;
  } else {
    i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    end = n16;
    stride = (int64_t)gridDim.x * 256;
  }
  for (; i + (kUnroll - 1) * stride < end; i += kUnroll * stride) {
    v4i v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  for (; i < end; i += stride) acc ^= src[i];
  const unsigned r = (unsigned)(acc.x ^ acc.y ^ acc.z ^ acc.w);
  if (r == 0x9e3779b9u) sink[0] = r;  // keeps the loads live; practically never stores
}

__global__ __launch_bounds__(256) void k_copy(const v4i* __restrict__ src, v4i* __restrict__ dst,
                                              int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// pattern 0: all-zero operands; 1: uniformly random bytes; 2: codes of
// magnitude below 32 (the typical size of smoothed, per-token quantized
// activations and per-channel quantized weights).
__device__ __forceinline__ unsigned operand_word(unsigned seed, int pattern) {
  unsigned x = seed * 0x9e3779b1u + 0x7f4a7c15u;
  x ^= x >> 15;
  x *= 0x2c1b3c6du;
  x ^= x >> 12;
  if (pattern == 0) return 0u;
  if (pattern == 2) {
    // four signed bytes in [-31, 31]
    unsigned r = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int v = (int)((x >> (8 * b)) & 63u) - 31;
      r |= ((unsigned)v & 0xffu) << (8 * b);
    }
    return r;
  }
  return x;
}

// CH independent accumulator chains per wave; the block size sets the waves
// per SIMD (512 threads: two, 256: one).  SHAPE 0: v_mfma_i32_32x32x32_i8
// (16 accumulator registers), SHAPE 1: v_mfma_i32_16x16x64_i8 (4 registers,
// half the work per instruction).
template <int SHAPE>
struct ProbeMma;
template <>
struct ProbeMma<0> {
  typedef v16i acc_t;
  __device__ static __forceinline__ acc_t mma(v4i a, v4i b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  }
};
template <>
struct ProbeMma<1> {
  typedef v4i acc_t;
  __device__ static __forceinline__ acc_t mma(v4i a, v4i b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
  }
};

template <int CH, int SHAPE>
__global__ __launch_bounds__(512) void k_mfma(int iters, int pattern, long long* __restrict__ clocks,
                                              int* __restrict__ sink) {
  typedef typename ProbeMma<SHAPE>::acc_t acc_t;
  constexpr int NE = sizeof(acc_t) / 4;
  const int tid = threadIdx.x;
  const unsigned seed = (unsigned)(blockIdx.x * blockDim.x + tid);
  v4i a, b;
  a.x = (int)operand_word(seed * 8 + 0, pattern);
  a.y = (int)operand_word(seed * 8 + 1, pattern);
  a.z = (int)operand_word(seed * 8 + 2, pattern);
  a.w = (int)operand_word(seed * 8 + 3, pattern);
  b.x = (int)operand_word(seed * 8 + 4, pattern);
  b.y = (int)operand_word(seed * 8 + 5, pattern);
  b.z = (int)operand_word(seed * 8 + 6, pattern);
  b.w = (int)operand_word(seed * 8 + 7, pattern);
  acc_t c[CH];
#pragma unroll
  for (int h = 0; h < CH; ++h) c[h] = acc_t{};
  __syncthreads();
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
    // independent accumulators, operands rotated so that successive MFMAs
    // see different data
#pragma unroll
    for (int h = 0; h < CH; h += 2) {
      c[h] = ProbeMma<SHAPE>::mma(a, b, c[h]);
      c[h + 1] = ProbeMma<SHAPE>::mma(b, a, c[h + 1]);
      a = a.yzwx;
    }
  }
  __syncthreads();
  const long long t1 = __builtin_amdgcn_s_memtime();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  if (tid == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
  int s = 0;
#pragma unroll
  for (int h = 0; h < CH; ++h)
#pragma unroll
    for (int e = 0; e < NE; ++e) s += c[h][e];
  if (s == 0x3c6ef372) sink[0] = s;  // keeps the MFMAs live
}

}  // namespace

extern "C" {

int w8a8probe_read(const void* src, size_t bytes, unsigned* sink, int blocks, int chunked,
                   hipStream_t st) {
  if (!src || !sink || bytes % 16 || ((uintptr_t)src) % 16 || blocks < 1) return 1;
  hipLaunchKernelGGL(k_read, dim3(blocks), dim3(256), 0, st, (const v4i*)src, (int64_t)(bytes / 16),
                     chunked ? 1 : 0, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int w8a8probe_copy(const void* src, void* dst, size_t bytes, int blocks, hipStream_t st) {
  if (!src || !dst || bytes % 16 || ((uintptr_t)src) % 16 || ((uintptr_t)dst) % 16 || blocks < 1)
    return 1;
  hipLaunchKernelGGL(k_copy, dim3(blocks), dim3(256), 0, st, (const v4i*)src, (v4i*)dst,
                     (int64_t)(bytes / 16));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// clocks: [blocks x 2] int64 (shader cycles, 100 MHz ticks) per block.
// waves: 8 (two per SIMD) or 4 (one per SIMD); chains: 4, 8 or 16
// accumulators per wave; shape: 0 = 32x32x32, 1 = 16x16x64 (16 chains only
// with this shape).
int w8a8probe_mfma(int blocks, int iters, int pattern, int waves, int chains, int shape,
                   long long* clocks, int* sink, hipStream_t st) {
  if (blocks < 1 || iters < 1 || pattern < 0 || pattern > 2 || !clocks || !sink) return 1;
  if ((waves != 4 && waves != 8) || (shape != 0 && shape != 1)) return 1;
  if (chains != 4 && chains != 8 && !(chains == 16 && shape == 1)) return 1;
  const dim3 block(64 * waves), grid(blocks);
#define W8A8_PROBE(CH, SH) hipLaunchKernelGGL((k_mfma<CH, SH>), grid, block, 0, st, iters, pattern, clocks, sink)
  if (shape == 0) {
    if (chains == 4) W8A8_PROBE(4, 0);
    else W8A8_PROBE(8, 0);
  } else {
    if (chains == 4) W8A8_PROBE(4, 1);
    else if (chains == 8) W8A8_PROBE(8, 1);
    else W8A8_PROBE(16, 1);
  }
#undef W8A8_PROBE
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
