// Per-column scale followed by per-row symmetric INT8 (or FP8 E4M3) quantization.
//
// Method: jisaku.com glossary page "SmoothQuant", section "平滑化変換の数学"
// (X~ = X s^-1, W~ = s W) and section "Activation外れ値問題" (INT8 range); the
// symmetric grid [-127, 127], per-row scales and round-half-even are the
// readings stated in the library header.  Per row t:
//   v_j = fp32(x[t, j]) * c_j;  m = max_j |v_j|;  delta = m / 127;  r = 127 / m;
//   q_j = round_half_even(v_j * r)   (always within [-127, 127])
// Each step is one IEEE fp32 operation (no contraction), the divisions are
// the correctly rounded ones, and the rounding to an integer is done by an
// fp32 add of 1.5 * 2^23, which rounds to nearest even like rint does.
//
// HBM-bound: 2 B read + 1 B written per element (+ 4 B per row).  A group of
// G threads (a multiple of the 64-wide wavefront, at most 1024) owns a row:
// thread g holds the 16-byte chunks g, g + G, ... (CPT of them, normally 2),
// so every wave load is 1 KiB of consecutive bytes and every wave store
// 512 B.  The row slice stays in registers between the max pass and the
// quantize pass (scaled, or as its 16-bit inputs), so x is read from HBM
// exactly once.  A block handles R
// consecutive rows with the same column ownership (the column scales are
// loaded once per block and stay L2 resident) and issues all of its row loads
// before the first reduction.  The row max is a wave reduction by DPP moves
// within 16-lane rows and four lane reads, followed by one LDS round across
// the waves of the block.  Per element the VALU work
// is about six operations (widen, scale, max, rescale, round, pack/4).
//
// The FP8 variant (same smoothing, FP8 E4M3 grid as the page's remark on
// low-bit float formats allows) differs only in the grid maximum (448) and in
// the rounding: the hardware conversion to E4M3, round to nearest even.
//
// The RMS-norm fold (NORM) reuses this kernel; the LayerNorm fold, whose
// row statistics enter every element, is k_layernorm_quant_rows at the end.
#include "common.h"

namespace w8a8 {

namespace {

// 1.5 * 2^23: adding it to a float t with |t| < 2^22 rounds t to an integer
// (to nearest, ties to even, by the fp32 add itself) and leaves that integer
// in the low mantissa bits, two's complement in the low byte.
constexpr float kRoundMagic = 12582912.0f;

// v as seen from the lane that the DPP control CTRL names (within rows of 16
// lanes); every lane of the wave must be active.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float lane_value(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Reduction over the 64 lanes of a wave (all active), the same value in
// every lane: pairs of lanes (quad_perm 1,0,3,2), quads (2,3,0,1), the other
// quad of each 8 (row_half_mirror), the other 8 of each 16 (row_mirror),
// then the four 16-lane rows read out and combined in a fixed order.  Each
// step combines a value with its partner symmetrically, so the lanes agree.
template <class Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = op(v, dpp<0xb1>(v));
  v = op(v, dpp<0x4e>(v));
  v = op(v, dpp<0x141>(v));
  v = op(v, dpp<0x140>(v));
  return op(op(lane_value(v, 0), lane_value(v, 16)), op(lane_value(v, 32), lane_value(v, 48)));
}

__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}

// Low bytes of four magic-rounded floats, packed little-endian.
__device__ __forceinline__ unsigned pack_codes(float a, float b, float c, float d) {
  const unsigned ua = __float_as_uint(a), ub = __float_as_uint(b);
  const unsigned uc = __float_as_uint(c), ud = __float_as_uint(d);
  const unsigned p01 = __builtin_amdgcn_perm(ub, ua, 0x0c0c0400u);  // ua.b0, ub.b0
  const unsigned p23 = __builtin_amdgcn_perm(ud, uc, 0x0c0c0400u);  // uc.b0, ud.b0
  return __builtin_amdgcn_perm(p23, p01, 0x05040100u);
}

// Element e (0..7) of a 16-byte chunk of fp16/bf16 values, widened to fp32.
template <bool BF16>
__device__ __forceinline__ float elem(const v4u& c, int e) {
  const unsigned w = c[e / 2];
  if (BF16) return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  return widen16((unsigned short)((e & 1) ? (w >> 16) : (w & 0xffffu)), false);
}

// |v| above 448 (by at most the fp32 rounding of v * (448 / m)) rounds to 448
// on the E4M3 grid; clamp it explicitly so the conversion never sees an
// out-of-range input.  The sign, including that of zero, is kept.
__device__ __forceinline__ float clamp_e4m3(float v) {
  return fabsf(v) > 448.0f ? copysignf(448.0f, v) : v;
}

// Four FP8 (E4M3) codes of a, b, c, d packed little-endian.  The hardware
// conversion rounds to nearest even and keeps the sign of zero, like the
// format's definition (checked bit for bit against it).
__device__ __forceinline__ unsigned pack_e4m3(float a, float b, float c, float d) {
  a = clamp_e4m3(a);
  b = clamp_e4m3(b);
  c = clamp_e4m3(c);
  d = clamp_e4m3(d);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (unsigned)w;
}

__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float a, float b) { return a + b; });
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// acc + a^2 + b^2 for the 16-bit pair (a, b) packed in w (v_dot2_f32_*):
// the squares of 16-bit values are exact in fp32.
template <bool BF16>
__device__ __forceinline__ float add_squares(unsigned w, float acc) {
  if (BF16)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                           __builtin_bit_cast(bf16x2, w), acc, false);
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), __builtin_bit_cast(f16x2, w), acc,
                                false);
}

// FMT 0: symmetric INT8 codes (grid max 127); FMT 1: FP8 E4M3 codes (max 448).
// NORM: the row is the input of an RMS norm whose weight carries the
// smoothing (col_scale = the folded RN32(gamma_j * inv_s_j)); the row scale
// is RN32(m / 127) times 1 / sqrt(RN32(sum_j x_j^2 / cols) + eps).  The
// per-token quantizer does not change under a positive factor common to the
// row, so the norm's factor only enters the scale; the codes are those of
// x * g.
// One matrix of the launch: rows of cols8 16-byte chunks, its column scales,
// codes and row scales.
struct RowSet {
  const v4u* x;
  int64_t rows;
  const float4* col_scale;
  uint2* q;
  float* row_scale;
};

// Blocks [0, b_first) take the rows of set a, blocks from b_first on those of
// set b (both with cols8 chunks per row): two matrices with the same row
// length, such as a layer's weight and its activations, quantize in one launch.
// Block 0 also clears `zero` (nzero words), at its end where the row's
// registers are free: the counters of the product that follows in the same
// stream, so that no separate fill is needed.
template <int CPT, int R, bool BF16, int FMT, bool NORM>
__global__ __launch_bounds__(1024) void k_scale_quant_rows(RowSet a, RowSet b, unsigned b_first,
                                                           int cols8, float eps,
                                                           unsigned* __restrict__ zero, int nzero) {
  const bool in_b = blockIdx.x >= b_first;
  const v4u* __restrict__ x = in_b ? b.x : a.x;
  const int64_t rows = in_b ? b.rows : a.rows;
  const float4* __restrict__ col_scale = in_b ? b.col_scale : a.col_scale;
  uint2* __restrict__ q = in_b ? b.q : a.q;
  float* __restrict__ row_scale = in_b ? b.row_scale : a.row_scale;
  const int tid = threadIdx.x;
  const int G = blockDim.x;
  const int lane = tid % kWave, wave = tid / kWave, nwaves = G / kWave;
  const int64_t row0 = (int64_t)(in_b ? blockIdx.x - b_first : blockIdx.x) * R;

  // all of this block's input loads first
  v4u xv[R][CPT];
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

  // pass 1: the row max of |v|, v = x * c
  float m[R], ss[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float mr = 0.0f, sr = 0.0f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
#pragma unroll
      for (int e = 0; e < 8; ++e) mr = fmaxf(mr, fabsf(elem<BF16>(xv[r][i], e) * sc[i][e]));
      // the sum of squares straight from the packed pairs
      if (NORM)
#pragma unroll
        for (int d = 0; d < 4; ++d) sr = add_squares<BF16>(xv[r][i][d], sr);
    }
    m[r] = wave_max(mr);
    ss[r] = NORM ? wave_sum(sr) : 0.0f;
  }
  // In the RMS-norm form at four rows of two chunks (rows of 8200 to 12288
  // values), pass 2 forms v again from the 16-bit inputs (the same one
  // rounding): the empty asm hides their values, so the fp32 products of
  // pass 1 cannot be kept instead, and the packed inputs take half their
  // registers (66-68 in place of 83-104, which admits a second 11-wave block
  // per CU).  Elsewhere the instance fits its occupancy either way and the
  // extra pass-2 work only costs time (RMS-norm fold at 2048 x 4096: 9.07
  // against 8.75 us; plain quantizer at 2048 x 11008: 16.4 against 15.1 us),
  // so the compiler keeps the products.
  if constexpr (NORM && R > 1 && R * CPT >= 8) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < CPT; ++i) asm volatile("" : "+v"(xv[r][i]));
  }
  __shared__ float red[R][16];
  __shared__ float red2[R][16];
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      red[r][wave] = m[r];
      if (NORM) red2[r][wave] = ss[r];
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float mr = red[r][0];
    for (int w = 1; w < nwaves; ++w) mr = fmaxf(mr, red[r][w]);
    m[r] = mr;
    if (NORM) {
      float sr = red2[r][0];
      for (int w = 1; w < nwaves; ++w) sr += red2[r][w];
      ss[r] = sr;
    }
  }

  // pass 2: codes = round_half_even(v * (127 / m)); m == 0 gives r = 0 and
  // all-zero codes.  |v * r| <= 127 (1 + 2^-23) for every element of a row,
  // so the rounded code never leaves [-127, 127] and no clamp is needed.
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = row0 + r;
    if (row >= rows) break;
    const float mr = m[r];
    constexpr float kGridMax = FMT == 0 ? 127.0f : 448.0f;
    const float rcp = mr > 0.0f ? kGridMax / mr : 0.0f;
    if (tid == 0) {
      float d = mr > 0.0f ? mr / kGridMax : 0.0f;
      if (NORM && mr > 0.0f) {
        const float ms = ss[r] / (float)(cols8 * 8);
        d = d * (1.0f / sqrtf(ms + eps));
      }
      row_scale[row] = d;
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = i * G + tid;
      if (c >= cols8) continue;
      float t[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        t[e] = (elem<BF16>(xv[r][i], e) * sc[i][e]) * rcp;
        if (FMT == 0) t[e] = t[e] + kRoundMagic;
      }
      uint2 o;
      if (FMT == 0) {
        o.x = pack_codes(t[0], t[1], t[2], t[3]);
        o.y = pack_codes(t[4], t[5], t[6], t[7]);
      } else {
        o.x = pack_e4m3(t[0], t[1], t[2], t[3]);
        o.y = pack_e4m3(t[4], t[5], t[6], t[7]);
      }
      q[row * cols8 + c] = o;
    }
  }
  if (blockIdx.x == 0)
    for (int i = tid; i < nzero; i += G) zero[i] = 0u;
}

RowSet row_set(const void* x, int64_t rows, const float* cs, void* q, float* row_scale) {
  return RowSet{(const v4u*)x, rows, (const float4*)cs, (uint2*)q, row_scale};
}

struct Zero {
  unsigned* p;
  int n;
};

template <int CPT, int R, bool BF16, int FMT, bool NORM>
void launch_one(const RowSet& a, const RowSet& b, int cols8, int G, float eps, Zero z,
                hipStream_t st) {
  const unsigned blocks_a = (unsigned)((a.rows + R - 1) / R);
  unsigned blocks = blocks_a + (unsigned)((b.rows + R - 1) / R);
  if (blocks == 0) blocks = 1;  // no rows: one block still clears z
  hipLaunchKernelGGL((k_scale_quant_rows<CPT, R, BF16, FMT, NORM>), dim3(blocks), dim3(G), 0, st,
                     a, b, blocks_a, cols8, eps, z.p, z.n);
}

template <int CPT, int R>
hipError_t launch_cfg(const RowSet& a, const RowSet& b, bool bf16, int fmt, int cols8, int G,
                      bool norm, float eps, Zero z, hipStream_t st) {
  if (norm) {  // RMS norm fold (INT8 only)
    if (bf16) launch_one<CPT, R, true, 0, true>(a, b, cols8, G, eps, z, st);
    else launch_one<CPT, R, false, 0, true>(a, b, cols8, G, eps, z, st);
  } else if (fmt == 0) {
    if (bf16) launch_one<CPT, R, true, 0, false>(a, b, cols8, G, eps, z, st);
    else launch_one<CPT, R, false, 0, false>(a, b, cols8, G, eps, z, st);
  } else {
    if (bf16) launch_one<CPT, R, true, 1, false>(a, b, cols8, G, eps, z, st);
    else launch_one<CPT, R, false, 1, false>(a, b, cols8, G, eps, z, st);
  }
  return hipGetLastError();
}

hipError_t launch_sets(const RowSet& a, const RowSet& b, bool bf16, int64_t cols, bool norm,
                       float eps, int fmt, Zero z, hipStream_t st) {
  if (a.rows + b.rows == 0 && z.n == 0) return hipSuccess;
  const int cols8 = (int)(cols / 8);
  // Threads per row: two 16-byte chunks each (more for rows past 2048 chunks,
  // where the block size reaches 1024), a whole number of waves.  Rows per
  // block: two while a thread holds two chunks, one beyond, which keeps the
  // fp32 row slice a thread carries between the passes at 32 values or fewer
  // (more would cost occupancy).  The exception is rows of 8200 to 12288
  // values (blocks of 9 to 12 waves, two per CU): four rows per block there
  // measured 4-8% faster at 11008 columns, and slower at 4096 and 16384.
  int G = (cols8 + 1) / 2;
  G = ((G + kWave - 1) / kWave) * kWave;
  if (G < kWave) G = kWave;
  if (G > 1024) G = 1024;
  const int cpt = (cols8 + G - 1) / G;
  switch (cpt <= 1 ? 1 : cpt) {
    case 1: return launch_cfg<1, 4>(a, b, bf16, fmt, cols8, G, norm, eps, z, st);
    case 2:
      if (cols8 > 1024 && cols8 <= 1536)
        return launch_cfg<2, 4>(a, b, bf16, fmt, cols8, G, norm, eps, z, st);
      return launch_cfg<2, 2>(a, b, bf16, fmt, cols8, G, norm, eps, z, st);
    case 3: return launch_cfg<3, 1>(a, b, bf16, fmt, cols8, G, norm, eps, z, st);
    case 4: return launch_cfg<4, 1>(a, b, bf16, fmt, cols8, G, norm, eps, z, st);
    case 5: return launch_cfg<5, 1>(a, b, bf16, fmt, cols8, G, norm, eps, z, st);
    case 6: return launch_cfg<6, 1>(a, b, bf16, fmt, cols8, G, norm, eps, z, st);
    case 7: return launch_cfg<7, 1>(a, b, bf16, fmt, cols8, G, norm, eps, z, st);
    case 8: return launch_cfg<8, 1>(a, b, bf16, fmt, cols8, G, norm, eps, z, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_scale_quant_rows(const void* x, bool bf16, int64_t rows, int64_t cols,
                                   const float* col_scale, bool norm, float eps, void* q,
                                   float* row_scale, int fmt, hipStream_t st, unsigned* zero,
                                   int nzero) {
  const RowSet a = row_set(x, rows, col_scale, q, row_scale);
  return launch_sets(a, row_set(nullptr, 0, nullptr, nullptr, nullptr), bf16, cols, norm, eps, fmt,
                     Zero{zero, nzero}, st);
}

hipError_t launch_scale_quant_pair(const void* w, int64_t n, const float* s, void* qw, float* sw,
                                   const void* x, int64_t m, const float* inv_s, void* qx,
                                   float* sx, bool bf16, int64_t k, hipStream_t st) {
  return launch_sets(row_set(w, n, s, qw, sw), row_set(x, m, inv_s, qx, sx), bf16, k, false, 0.0f,
                     0, Zero{nullptr, 0}, st);
}

// LayerNorm fold (fp16 rows), one row per block.  The smoothing's inv_s is
// folded into the LayerNorm's affine pair, g = RN32(gamma * inv_s) and
// b = RN32(beta * inv_s), and the additive b keeps the row statistics in
// every element, so they decide codes; they are therefore computed without
// any dependence on a summation order.  Every finite fp16 value is an integer
// multiple of 2^-24, so with X = x * 2^24 (|X| < 2^41) the sums S1 = sum X and
// S2 = sum X^2 are exact integers.  Then, once per row:
//   mean = f32(f64(f64(S1) / (K 2^24)))
//   var  = f32(f64(f64(K S2 - S1^2) / (K^2 2^48)))     (population variance)
//   r    = RN32(1 / RN32(sqrt(RN32(var + eps)))), or 0 when var + eps == 0
// and per element v = RN32(RN32(RN32(RN32(x - mean) * r) * g) + b), one IEEE
// fp32 operation per step, followed by the per-row quantizer.
//
// The sums are taken in fp64 up to the wave level, where no addition rounds:
// a wave covers at most 4096 elements (64 lanes, 8 chunks of 8 per lane).
//   - sum x: every partial sum is a multiple of 2^-24 below 4096 * 65504 <
//     2^28, so it needs at most 52 significant bits.
//   - sum x^2: x^2 is exact in fp64 (11-bit significand squared) and t =
//     x^2 * 2^8 is a multiple of 2^-40 below 2^40.  t splits exactly into
//     its integer part (summed: below 2^52) and its fraction (summed: a
//     multiple of 2^-40 below 2^12), each within 52 bits.
// So the wave sums are the exact values, and each becomes an int64 in
// fixed units (S1 in 2^-24, the integer part in 2^-8 of x^2, the fraction in
// 2^-48) for the order-free integer sum across waves.  That keeps the VALU
// cost near nine fp64 operations per element where 64-bit integer squares
// took several times as many.
namespace {

// Correctly rounded (to nearest even) conversion of a nonnegative 128-bit
// integer to double: normalize the top 64 bits and fold every bit below them
// into the lowest one, a sticky bit under the rounding position.
__device__ __forceinline__ double u128_to_f64(unsigned __int128 v) {
  const unsigned long long hi = (unsigned long long)(v >> 64), lo = (unsigned long long)v;
  if (hi == 0) return (double)lo;
  const int lz = __builtin_clzll(hi);
  unsigned long long top = lz ? (hi << lz) | (lo >> (64 - lz)) : hi;
  const unsigned long long rest = lz ? (lo << lz) : lo;
  top |= (rest != 0) ? 1ull : 0ull;
  return __builtin_ldexp((double)top, 64 - lz);
}

// Per-wave sums of the LayerNorm statistics, as integers in fixed units.
struct LnSums {
  long long s1;  // sum x, units of 2^-24
  long long ta;  // sum of the integer parts of x^2 * 2^8, units of 2^-8 of x^2
  long long tb;  // sum of the fractions of x^2 * 2^8, units of 2^-48 of x^2
};

__device__ __forceinline__ LnSums ln_add(LnSums a, const LnSums& b) {
  a.s1 += b.s1;
  a.ta += b.ta;
  a.tb += b.tb;
  return a;
}

// WPE bounds the registers: 8 waves per SIMD (64 registers) so that two
// blocks of 1024 threads fit on a CU (one block per CU measured 15% slower),
// 6 (80 registers) for blocks of up to 512 threads at three or four chunks,
// 4 beyond four chunks.
template <int CPT, int WPE>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 1024),
                          amdgpu_waves_per_eu(WPE))) void
k_layernorm_quant_rows(const v4u* __restrict__ x,
                                                               int cols8,
                                                               const float4* __restrict__ gv,
                                                               const float4* __restrict__ bv,
                                                               float eps, uint2* __restrict__ q,
                                                               float* __restrict__ row_scale) {
  const int tid = threadIdx.x;
  const int G = blockDim.x;
  const int lane = tid % kWave, wave = tid / kWave, nwaves = G / kWave;
  const int64_t row = blockIdx.x;

  v4u xv[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = i * G + tid;
    xv[i] = c < cols8 ? __builtin_nontemporal_load(x + row * cols8 + c) : v4u{0u, 0u, 0u, 0u};
  }

  // pass 1: exact fp64 sums within the wave (chunks past the row hold zeros
  // and add nothing)
  double s1 = 0.0, ta = 0.0, tb = 0.0;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double xd = (double)elem<false>(xv[i], e);
      s1 += xd;
      const double t = (xd * xd) * 256.0;
      const double ti = __builtin_trunc(t);
      ta += ti;
      tb += t - ti;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    s1 += __shfl_xor(s1, off, kWave);
    ta += __shfl_xor(ta, off, kWave);
    tb += __shfl_xor(tb, off, kWave);
  }
  const LnSums acc = {(long long)(s1 * 16777216.0), (long long)ta,
                      (long long)(tb * 1099511627776.0)};
  __shared__ LnSums red[16];
  __shared__ float stat[2];
  __shared__ float redm[16];
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  if (tid == 0) {
    LnSums t = red[0];
    for (int w = 1; w < nwaves; ++w) t = ln_add(t, red[w]);
    const long long K = (long long)cols8 * 8;
    // sum X^2 = sum x^2 * 2^48 = ta * 2^40 + tb
    const __int128 s2 = ((__int128)t.ta << 40) + (__int128)t.tb;
    const __int128 v = (__int128)K * s2 - (__int128)t.s1 * (__int128)t.s1;  // >= 0
    const double kd = (double)K;
    const float mean = (float)((double)t.s1 / (kd * 16777216.0));
    const float var = (float)(u128_to_f64((unsigned __int128)v) / (kd * kd * 281474976710656.0));
    const float tv = var + eps;
    stat[0] = mean;
    stat[1] = tv > 0.0f ? 1.0f / sqrtf(tv) : 0.0f;
  }
  __syncthreads();
  const float mean = stat[0], r = stat[1];

  // pass 2: v in registers and the row max of |v|
  float v[CPT][8];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = i * G + tid;
    if (c < cols8) {
      const float4 g0 = gv[2 * c], g1 = gv[2 * c + 1], b0 = bv[2 * c], b1 = bv[2 * c + 1];
      const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float t = elem<false>(xv[i], e) - mean;
        t = t * r;
        t = t * gg[e];
        t = t + bb[e];
        v[i][e] = t;
        m = fmaxf(m, fabsf(t));
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] = 0.0f;
    }
  }
  m = wave_max(m);
  if (lane == 0) redm[wave] = m;
  __syncthreads();
  m = redm[0];
  for (int w = 1; w < nwaves; ++w) m = fmaxf(m, redm[w]);

  // the per-row quantizer, as in k_scale_quant_rows
  const float rcp = m > 0.0f ? 127.0f / m : 0.0f;
  if (tid == 0) row_scale[row] = m > 0.0f ? m / 127.0f : 0.0f;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = i * G + tid;
    if (c >= cols8) continue;
    float t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      t[e] = v[i][e] * rcp;
      t[e] = t[e] + kRoundMagic;
    }
    uint2 o;
    o.x = pack_codes(t[0], t[1], t[2], t[3]);
    o.y = pack_codes(t[4], t[5], t[6], t[7]);
    q[row * cols8 + c] = o;
  }
}

template <int CPT, int WPE = (CPT <= 4 ? 8 : 4)>
void launch_ln(const void* x, int64_t rows, int cols8, int G, const float* g, const float* b,
               float eps, void* q, float* row_scale, hipStream_t st) {
  hipLaunchKernelGGL((k_layernorm_quant_rows<CPT, WPE>), dim3((unsigned)rows), dim3(G), 0, st,
                     (const v4u*)x, cols8, (const float4*)g, (const float4*)b, eps, (uint2*)q,
                     row_scale);
}

}  // namespace

hipError_t launch_layernorm_quant_rows(const void* x, int64_t rows, int64_t cols, const float* g,
                                       const float* b, float eps, void* q, float* row_scale,
                                       hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int cols8 = (int)(cols / 8);
  // Chunks per thread: four for rows of up to 8192 values, three up to 16384,
  // then blocks of 1024 threads.  The per-row work (the fp64 wave sums and
  // their fixed-point conversion, two LDS rounds) is paid once per wave, so
  // fewer, fuller waves per row issue fewer VALU instructions per element.
  // Measured at 2048 rows against two chunks per thread: 13.3 against 15.0 us
  // at 5120 columns, 16.9 against 18.5 at 7168, 24.3 against 30.1 at 11008;
  // at 20480 columns three chunks measured slower (29.8 against 26.2).
  const int target = cols8 <= 1024 ? 4 : cols8 <= 2048 ? 3 : 2;
  int G = (cols8 + target - 1) / target;  // whole waves, at most 1024
  G = ((G + kWave - 1) / kWave) * kWave;
  if (G < kWave) G = kWave;
  if (G > 1024) G = 1024;
  switch ((cols8 + G - 1) / G) {
    case 1: launch_ln<1>(x, rows, cols8, G, g, b, eps, q, row_scale, st); break;
    case 2: launch_ln<2>(x, rows, cols8, G, g, b, eps, q, row_scale, st); break;
    case 3:
      if (G <= 512) launch_ln<3, 6>(x, rows, cols8, G, g, b, eps, q, row_scale, st);
      else launch_ln<3>(x, rows, cols8, G, g, b, eps, q, row_scale, st);
      break;
    case 4:
      if (G <= 512) launch_ln<4, 6>(x, rows, cols8, G, g, b, eps, q, row_scale, st);
      else launch_ln<4>(x, rows, cols8, G, g, b, eps, q, row_scale, st);
      break;
    case 5: launch_ln<5>(x, rows, cols8, G, g, b, eps, q, row_scale, st); break;
    case 6: launch_ln<6>(x, rows, cols8, G, g, b, eps, q, row_scale, st); break;
    case 7: launch_ln<7>(x, rows, cols8, G, g, b, eps, q, row_scale, st); break;
    case 8: launch_ln<8>(x, rows, cols8, G, g, b, eps, q, row_scale, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace w8a8
