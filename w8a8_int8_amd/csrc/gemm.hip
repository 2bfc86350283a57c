// INT8 x INT8 -> INT32 GEMM on CDNA4 matrix cores, with the dequant epilogue.
//
// Method: jisaku.com glossary page "SmoothQuant": section "SmoothQuantとは" and
// the GPTQ / AWQ comparison table (W8A8 multiplies the INT8 operands directly;
// the speed comes from the integer matrix units, not from bandwidth).  The
// per-token and per-output-channel scales factor out of the K sum, so the
// accumulator is dequantized once, in the epilogue:
//   C[t, k] = sum_j qa[t, j] qb[k, j]                     (exact int32)
//   Y[t, k] = out(fp32(fp32(C[t, k]) * sa[t]) * sb[k])    (IEEE fp32, RNE)
//
// Operands: qa = activation codes, M x K; qb = weight codes, N x K; both K
// contiguous ("TN").  Every MFMA is v_mfma_i32_32x32x32_i8 with the weight
// fragment as its first operand (32 output channels x 32 k) and the activation
// fragment as its second (32 k x 32 tokens), so that each lane's four
// consecutive accumulator registers hold four consecutive output channels of
// one token: the epilogue writes 4 fp16 / bf16 (8 B) or 4 int32 (16 B) per
// lane per register group.  Integer accumulation is exact and order free.
//
// Tiling: a 256-thread block (4 waves, one per SIMD) owns a BM x BN output
// tile (tokens x channels); the waves form a 2 x 2 grid, each with a
// (BM/2) x (BN/2) register tile of 32 x 32 MFMA blocks, accumulators in the
// accumulation registers.  The K loop steps 128 bytes at a time through two
// LDS stages: while the MFMAs consume stage s, the global loads for stage s+1
// are in flight in registers, then written to the other stage; one barrier per
// step.  In LDS each tile row is 128 B = 8 chunks of 16 B, and chunk c of row
// r is stored at chunk slot c ^ ((r >> 1) & 7): the 16 lanes of any quarter
// wave then touch 16 distinct 16-byte bank groups both when the fragment
// reads walk down 16 rows at one k and when the stores walk along rows.
//
// Global loads are buffer loads against a resource that ends at the last valid
// row of the tile, so rows past M or N read as zero (no clamping, no
// branches); a K that is not a multiple of 128 zeroes its tail chunks the same
// way.  Blocks are dispatched round-robin over the 8 XCDs; the tile index is
// remapped so that each XCD (with its own L2) works on a contiguous run of
// tiles, ordered token-tile fastest within groups of 8 token tiles, so the
// CUs of one XCD share both operand panels.
#include "common.h"

namespace w8a8 {

namespace {

constexpr int kBK = 128;         // bytes of K per LDS stage
constexpr int kThreads = 256;    // 4 waves
constexpr int kGroupM = 8;       // token tiles per ordering group
constexpr unsigned kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)
constexpr int kOob = 0x40000000;  // voffset that is out of range for every resource here

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const int8_t* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, (int)kRsrcWord3);
}

__device__ __forceinline__ v4i load16(rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

__device__ __forceinline__ int swz(int row, int chunk) {
  return (row << 7) + ((chunk ^ ((row >> 1) & 7)) << 4);
}

__device__ __forceinline__ unsigned short f32_to_bf16_rne(float f) {
  unsigned u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

__device__ __forceinline__ unsigned short f32_to_f16_rne(float f) {
  return __builtin_bit_cast(unsigned short, (_Float16)f);
}

// Map the linear block index to (token tile, channel tile).
__device__ __forceinline__ void tile_of(int bid, int m_tiles, int n_tiles, int& tm, int& tn) {
  const int total = m_tiles * n_tiles;
  const int q = total / 8, rem = total % 8;
  const int xcd = bid % 8, idx = bid / 8;
  const int t = xcd * q + min(xcd, rem) + idx;
  const int per_group = kGroupM * n_tiles;
  const int g = t / per_group;
  const int first_m = g * kGroupM;
  const int gsize = min(m_tiles - first_m, kGroupM);
  const int in_g = t - g * per_group;
  tm = first_m + in_g % gsize;
  tn = in_g / gsize;
}

// OUT: 0 = int32 C, 1 = fp16 Y, 2 = bf16 Y
template <int BM, int BN, int OUT>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(1, 1))) void
k_gemm_i8(const int8_t* __restrict__ qa, const int8_t* __restrict__ qb, int M, int N, int K,
          const float* __restrict__ sa, const float* __restrict__ sb, void* __restrict__ out,
          int m_tiles, int n_tiles) {
  constexpr int WM = BM / 2, WN = BN / 2;  // wave tile (tokens, channels)
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int LA = BM / 32, LB = BN / 32;  // 16-byte loads per thread per stage
  constexpr int STAGE = (BM + BN) * kBK;
  __shared__ __attribute__((aligned(16))) int8_t lds[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  int tm, tn;
  tile_of(blockIdx.x, m_tiles, n_tiles, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
  const rsrc_t ra = make_rsrc(qa + (int64_t)m0 * K, (unsigned)rows_a * (unsigned)K);
  const rsrc_t rb = make_rsrc(qb + (int64_t)n0 * K, (unsigned)rows_b * (unsigned)K);

  // this thread's load slots: rows i*32 + (tid >> 3), chunk c = tid & 7
  const int c = tid & 7;
  const int r_in = tid >> 3;
  const int st_off = swz(r_in, c);  // + i * 32 * 128 for slot i
  int voff_a[LA], voff_b[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) voff_a[i] = (i * 32 + r_in) * K + c * 16;
#pragma unroll
  for (int i = 0; i < LB; ++i) voff_b[i] = (i * 32 + r_in) * K + c * 16;

  // fragment read offsets (row part; the swizzle depends only on lane & 31)
  const int fr = lane & 31, fk = lane >> 5;
  const int fsw = (fr >> 1) & 7;

  v16i acc[FN][FM];
#pragma unroll
  for (int a = 0; a < FN; ++a)
#pragma unroll
    for (int b = 0; b < FM; ++b) acc[a][b] = v16i{};

  const int nk = (K + kBK - 1) / kBK;
  v4i ga[LA], gb[LB];

  auto gload = [&](int kt) {
    const int k0 = kt * kBK;
    const bool tail = (k0 + c * 16) >= K;
#pragma unroll
    for (int i = 0; i < LA; ++i) ga[i] = load16(ra, tail ? kOob : voff_a[i], k0);
#pragma unroll
    for (int i = 0; i < LB; ++i) gb[i] = load16(rb, tail ? kOob : voff_b[i], k0);
  };
  auto lstore = [&](int s) {
    int8_t* base = lds + s * STAGE;
#pragma unroll
    for (int i = 0; i < LA; ++i) *(v4i*)(base + i * 32 * kBK + st_off) = ga[i];
#pragma unroll
    for (int i = 0; i < LB; ++i) *(v4i*)(base + BM * kBK + i * 32 * kBK + st_off) = gb[i];
  };

  if (nk > 0) {
    gload(0);
    lstore(0);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int s = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const int8_t* sA = lds + s * STAGE;
    const int8_t* sB = sA + BM * kBK;
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      const int ch = ((2 * kk + fk) ^ fsw) << 4;
      v4i fb[FN], fa[FM];
#pragma unroll
      for (int a = 0; a < FN; ++a)
        fb[a] = *(const v4i*)(sB + ((wn * WN + a * 32 + fr) << 7) + ch);
#pragma unroll
      for (int b = 0; b < FM; ++b)
        fa[b] = *(const v4i*)(sA + ((wm * WM + b * 32 + fr) << 7) + ch);
#pragma unroll
      for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int b = 0; b < FM; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[a], fa[b], acc[a][b], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(s ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds, for register group g, channels n .. n+3 of token m
  const int hi = lane >> 5;
#pragma unroll
  for (int b = 0; b < FM; ++b) {
    const int m = m0 + wm * WM + b * 32 + (lane & 31);
    if (m >= M) continue;
    float am = 0.0f;
    if (OUT != 0) am = sa[m];
#pragma unroll
    for (int a = 0; a < FN; ++a) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * WN + a * 32 + g * 8 + hi * 4;
        if (n >= N) continue;
        const v16i& C = acc[a][b];
        if (OUT == 0) {
          v4i o = {C[4 * g + 0], C[4 * g + 1], C[4 * g + 2], C[4 * g + 3]};
          *(v4i*)((int32_t*)out + (int64_t)m * N + n) = o;
        } else {
          const float4 bn = *(const float4*)(sb + n);
          const float w[4] = {bn.x, bn.y, bn.z, bn.w};
          unsigned short h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float y = (float)C[4 * g + e];
            y = y * am;
            y = y * w[e];
            h[e] = OUT == 1 ? f32_to_f16_rne(y) : f32_to_bf16_rne(y);
          }
          uint2 o;
          o.x = (unsigned)h[0] | ((unsigned)h[1] << 16);
          o.y = (unsigned)h[2] | ((unsigned)h[3] << 16);
          *(uint2*)((unsigned short*)out + (int64_t)m * N + n) = o;
        }
      }
    }
  }
}

template <int BM, int BN>
hipError_t launch_tile(const int8_t* qa, const int8_t* qb, int64_t M, int64_t N, int64_t K,
                       const float* sa, const float* sb, void* out, int mode, hipStream_t st) {
  const int mt = (int)((M + BM - 1) / BM), nt = (int)((N + BN - 1) / BN);
  const dim3 grid((unsigned)(mt * nt)), block(kThreads);
  switch (mode) {
    case 0:
      hipLaunchKernelGGL((k_gemm_i8<BM, BN, 0>), grid, block, 0, st, qa, qb, (int)M, (int)N,
                         (int)K, sa, sb, out, mt, nt);
      break;
    case 1:
      hipLaunchKernelGGL((k_gemm_i8<BM, BN, 1>), grid, block, 0, st, qa, qb, (int)M, (int)N,
                         (int)K, sa, sb, out, mt, nt);
      break;
    default:
      hipLaunchKernelGGL((k_gemm_i8<BM, BN, 2>), grid, block, 0, st, qa, qb, (int)M, (int)N,
                         (int)K, sa, sb, out, mt, nt);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const int8_t* qa, const int8_t* qb, int64_t M, int64_t N, int64_t K,
                       const float* sa, const float* sb, void* out, int out_mode,
                       hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  // Pick the tile whose last wave of blocks over 256 CUs is fullest, with a
  // small preference for the larger tile (more MACs per byte of LDS traffic).
  struct Cand { int bm, bn; double eff; };
  const Cand cands[] = {{256, 256, 1.0}, {256, 128, 0.92}, {128, 128, 0.8}};
  int best = 0;
  double best_score = -1.0;
  for (int i = 0; i < 3; ++i) {
    const int64_t tiles = ((M + cands[i].bm - 1) / cands[i].bm) * ((N + cands[i].bn - 1) / cands[i].bn);
    const int64_t waves = (tiles + 255) / 256;
    const double fill = (double)tiles / (double)(waves * 256);
    // useful fraction of the padded tile rows
    const double mfill = (double)M / (double)(((M + cands[i].bm - 1) / cands[i].bm) * cands[i].bm);
    const double score = fill * mfill * cands[i].eff;
    if (score > best_score + 1e-9) { best_score = score; best = i; }
  }
  switch (best) {
    case 0: return launch_tile<256, 256>(qa, qb, M, N, K, sa, sb, out, out_mode, st);
    case 1: return launch_tile<256, 128>(qa, qb, M, N, K, sa, sb, out, out_mode, st);
    default: return launch_tile<128, 128>(qa, qb, M, N, K, sa, sb, out, out_mode, st);
  }
}

}  // namespace w8a8
