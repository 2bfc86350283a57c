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
// contiguous.  Every MFMA is v_mfma_i32_32x32x32_i8 with the weight fragment
// as its first operand (32 output channels x 32 k) and the activation
// fragment as its second (32 k x 32 tokens), so that each lane's four
// consecutive accumulator registers hold four consecutive output channels of
// one token.  Integer accumulation is exact and order free.  The epilogue
// dequantizes in registers and restages each wave's results through LDS so
// that every global store writes whole rows of 16 bytes per lane.
//
// Block: WGM x WGN waves (8 for the 256-row tiles, 4 for 128 x 128) own a
// BM x BN output tile (tokens x channels); wave (wm, wn) holds a
// (BM / WGM) x (BN / WGN) register tile of 32 x 32 MFMA blocks.  Tiles:
// 256 x 256, 256 x 192, 256 x 128 and 128 x 128; launch_gemm picks the one
// whose last wave of blocks over the 256 CUs is fullest, preferring fewer
// operand bytes per MFMA (the return path of the operand loads is the
// limiting resource).
//
// K pipeline: K advances BK = 128 bytes per stage (one full cache line per
// operand row) through NST LDS slots (2 to 4, as many as 160 KB of LDS holds
// for the tile).  Operand rows go from global memory straight into LDS with
// buffer loads in LDS mode (16 B per lane, each wave instruction fills 1 KiB
// of LDS), NST - 1 or NST - 2 stages in flight while one is computed, and a
// wave never holds global data in registers.  Which waves issue a stage's
// loads, and when, is set by the slot count (see the pipeline in the kernel):
// a SIMD stalls its matrix pipe while both of its waves have loads waiting to
// issue, so with two slots one wave per SIMD issues them all.  Stages past the
// end are issued with out-of-range offsets (no memory traffic) so the
// per-stage load count, and with it every vmcnt wait, is constant.
//
// Per stage a wave runs BK / 32 k steps (BK / 64 for FP8, whose
// MFMA takes 64 bytes of K) of (BM / WGM / 32) x (BN / WGN / 32) MFMAs.  The
// fragment reads are software pipelined: the next k step's fragments are read
// while the current step's MFMAs run, and the next stage's first fragments
// are read (after the stage barrier) while the last step's MFMAs run.  One
// barrier per stage; it is a plain s_barrier (no memory fence), with the
// needed waits explicit: each wave waits for its own LDS-mode loads of the
// next stage (vmcnt) and for its own LDS reads of the slot that is about to
// be refilled (lgkmcnt).
//
// LDS layout: a tile row is BK bytes = CPR chunks of 16 B; RPW = 16 / CPR
// rows share one 256-byte bank window.  Chunk c of row r sits at chunk slot
// c ^ ((r / RPW) % CPR) of that row, so the lanes of a quarter wave reading
// one k chunk down consecutive rows hit distinct 16-byte bank groups.  The
// loads realize the swizzle by choosing, per lane, which global chunk lands in
// its slot.
//
// Edges: the buffer resource of each operand tile ends at its last valid row,
// so rows past M or N load as zero; chunks past K use an out-of-range offset
// and load as zero too.  Blocks are dispatched round-robin over the 8 XCDs;
// tile indices are remapped so each XCD (own L2) gets a contiguous run of
// tiles, ordered token-tile fastest in groups of 8 token tiles.
//
// The same pipeline serves the dense fp16 / bf16 product (the comparison
// baseline) and the FP8 E4M3 variant; few-token shapes go to k_gemm_skinny
// and, in the runtime forward, to the split-K k_gemm_splitk (below).
#include <algorithm>

#include "common.h"

namespace w8a8 {

namespace {

constexpr int kGroupM = 8;       // token tiles per ordering group
constexpr unsigned kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)
constexpr int kOob = 0x40000000;  // voffset that is out of range for every resource here

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// OUT selects operands, accumulation and epilogue of the tiled kernel:
//   0: int8 operands, int32 accumulators stored as they are
//   1: int8 operands, int32 accumulators dequantized to fp16
//   2: int8 operands, int32 accumulators dequantized to bf16
//   3: fp16 operands, fp32 accumulators rounded to fp16 (the dense baseline)
//   4: bf16 operands, fp32 accumulators rounded to bf16 (the dense baseline)
//   5: FP8 E4M3 operands, fp32 accumulators dequantized to fp16
//   6: FP8 E4M3 operands, fp32 accumulators dequantized to bf16
// A fragment is FR 16-byte chunks per lane: the 32 x 32 MFMAs for int8, fp16
// and bf16 take 32 bytes of K per row (FR = 1), the FP8 one 64 bytes (FR = 2);
// the byte-addressed LDS pipeline is the same for all of them.
typedef int v8i __attribute__((ext_vector_type(8)));
template <int OUT>
struct MmaKind {
  static constexpr int FR = 1;
  typedef v16i acc_t;
  __device__ static __forceinline__ acc_t mma(const v4i* a, const v4i* b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a[0], b[0], c, 0, 0, 0);
  }
};
template <>
struct MmaKind<3> {
  static constexpr int FR = 1;
  typedef v16f acc_t;
  __device__ static __forceinline__ acc_t mma(const v4i* a, const v4i* b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a[0]),
                                                  __builtin_bit_cast(v8h, b[0]), c, 0, 0, 0);
  }
};
template <>
struct MmaKind<4> {
  static constexpr int FR = 1;
  typedef v16f acc_t;
  __device__ static __forceinline__ acc_t mma(const v4i* a, const v4i* b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a[0]),
                                                   __builtin_bit_cast(v8bf, b[0]), c, 0, 0, 0);
  }
};
struct MmaE4m3 {
  static constexpr int FR = 2;
  typedef v16f acc_t;
  // format selectors 0 / 0: both operands FP8 E4M3, no block scales
  __device__ static __forceinline__ acc_t mma(const v4i* a, const v4i* b, acc_t c) {
    const v8i a8 = __builtin_shufflevector(a[0], a[1], 0, 1, 2, 3, 4, 5, 6, 7);
    const v8i b8 = __builtin_shufflevector(b[0], b[1], 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 0, 0, 0, 0, 0, 0);
  }
};
template <>
struct MmaKind<5> : MmaE4m3 {};
template <>
struct MmaKind<6> : MmaE4m3 {};

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ rsrc_t make_rsrc(const int8_t* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, (int)kRsrcWord3);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
}

// Hardware barrier without a memory fence.  The asm memory clobber keeps the
// compiler from moving LDS or global accesses across it, and the scheduling
// barriers keep every other instruction (MFMAs included) on its side, so each
// half-iteration is its own scheduling region.
__device__ __forceinline__ void block_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
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

// Scheduling hint for the compiler: interleave each MFMA with up to DPM LDS
// reads and a share of the global (LDS-mode) loads, so that no wave stalls on
// a memory queue while its matrix pipe idles.  I counts MFMAs; memory
// instructions are front-loaded so their latency overlaps the remaining
// MFMAs.  The three- and four-slot tiles issue all of a k step's fragment
// reads with its first MFMA (measured 2% faster on the 256 x 128 tile; on
// the two-slot tiles, where the loads come in a burst after the barrier, one
// read per MFMA is as fast or faster).
template <int I, int NMFMA, int NDS, int NVM, int DPM = 1>
__device__ __forceinline__ void interleave() {
  constexpr int VPM = (NVM + NMFMA - 1) / NMFMA;  // VMEMs per MFMA
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
  if constexpr (I * DPM < NDS)
    __builtin_amdgcn_sched_group_barrier(0x100, NDS - I * DPM < DPM ? NDS - I * DPM : DPM, 0);
  if constexpr (I * VPM < NVM)
    __builtin_amdgcn_sched_group_barrier(0x010, NVM - I * VPM < VPM ? NVM - I * VPM : VPM, 0);
  if constexpr (I + 1 < NMFMA) interleave<I + 1, NMFMA, NDS, NVM, DPM>();
}

// The tiled kernels' LDS, sized for the largest tile's stages (every tiled
// kernel runs one block per CU).  It is one file-scope array rather than a
// pointer handed to the tile code: with a pointer the compiler can no longer
// tell the LDS-mode loads of later stages from the fragment reads of the
// current one and waits for every outstanding load before the first reads
// (measured 12% slower on the 256 x 192 tile).
constexpr int kTileLds = 3 * (256 + 128) * 128;
__shared__ __attribute__((aligned(1024))) int8_t lds[kTileLds];

// One output tile (token tile tm, channel tile tn) of the tiled GEMM.  OUT as
// in MmaKind.  The block has WGM x WGN waves; K (in bytes per row) advances
// BK bytes per stage through NST LDS slots.  N is the number of channels this
// call covers (qb, sb and out start at its first one) and ldc the row stride
// of out in elements.
template <int BM, int BN, int BK, int NST, int WGM, int WGN, int OUT>
__device__ __forceinline__ void gemm_tile(const int8_t* __restrict__ qa,
                                          const int8_t* __restrict__ qb, int M, int N, int K,
                                          const float* __restrict__ sa,
                                          const float* __restrict__ sb, void* __restrict__ out,
                                          int ldc, int tm, int tn) {
  constexpr int NW = WGM * WGN;                 // waves per block
  constexpr int WM = BM / WGM, WN = BN / WGN;   // wave tile (tokens, channels)
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int CPR = BK / 16;                  // 16-byte chunks per LDS row
  constexpr int RPW = 16 / CPR;                 // rows per 256-byte bank window
  constexpr int RPI = 1024 / BK;                // rows filled by one LDS-mode wave load
  constexpr int FR = MmaKind<OUT>::FR;          // 16-byte chunks per fragment
  constexpr int KK = BK / (32 * FR);            // MFMA k steps per stage
  constexpr int LA = BM / RPI / NW;             // LDS-mode loads per wave per stage, activations
  constexpr int LB = BN / RPI / NW;             // ... weights
  constexpr int L = LA + LB;
  constexpr int SLOT = (BM + BN) * BK;          // bytes per LDS stage
  static_assert(LA >= 1 && LB >= 1 && LA * RPI * NW == BM && LB * RPI * NW == BN &&
                FM >= 1 && FN >= 1 && KK % 2 == 0, "unsupported tile");
  static_assert(NST >= 2 && (NST - 1) * 2 * L < 64, "unsupported pipeline depth");  // vmcnt range
  static_assert(NST * SLOT <= kTileLds, "LDS size");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  const int m0 = tm * BM, n0 = tn * BN;
  const rsrc_t ra = make_rsrc(qa + (int64_t)m0 * K, (unsigned)min(BM, M - m0) * (unsigned)K);
  const rsrc_t rb = make_rsrc(qb + (int64_t)n0 * K, (unsigned)min(BN, N - n0) * (unsigned)K);

  // LDS-mode load i of this wave fills LDS rows (i * NW + wave) * RPI + lane / CPR,
  // chunk slot lane % CPR, with the global chunk slot ^ ((row / RPW) % CPR).
  const int lrow = lane / CPR, lslot = lane % CPR;
  int voff_a[LA], voff_b[LB], kc_a[LA], kc_b[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int row = (i * NW + wave) * RPI + lrow;
    kc_a[i] = (lslot ^ ((row / RPW) % CPR)) << 4;
    voff_a[i] = row * K + kc_a[i];
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int row = (i * NW + wave) * RPI + lrow;
    kc_b[i] = (lslot ^ ((row / RPW) % CPR)) << 4;
    voff_b[i] = row * K + kc_b[i];
  }

  const int nk = (K + BK - 1) / BK;

  // LDS-mode loads of stage `st`, numbered j = h * L + i: for h = 0 this
  // wave's own loads (i < LA activations, then weights), for h = 1 those of
  // wave + NW / 2, issued on its behalf (see the pipeline below).  Rows of
  // wave + NW / 2 lie NW / 2 * RPI rows further down with the same chunk
  // swizzle, so they differ only in the scalar offset.  Loads j0 <= j < j1
  // are issued.  A stage past the end (st >= nk) is issued with out-of-range
  // offsets: it moves no data, keeps every wave's per-stage load count
  // constant (so fixed vmcnt values serve every iteration) and only touches
  // the slot that the stage would have used, which no live stage occupies.
  auto dma = [&](int st, int j0, int j1) {
    const int k0 = st * BK;
    int8_t* slot = lds + (st % NST) * SLOT;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int so = k0 + h * (NW / 2) * RPI * K;
      const int w = wave + h * (NW / 2);
#pragma unroll
      for (int i = 0; i < LA; ++i) {
        if (h * L + i < j0 || h * L + i >= j1) continue;
        const int vo = (k0 + kc_a[i] >= K) ? kOob : voff_a[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (lds_void_t*)(slot + (i * NW + w) * 1024), 16, vo, so, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < LB; ++i) {
        if (h * L + LA + i < j0 || h * L + LA + i >= j1) continue;
        const int vo = (k0 + kc_b[i] >= K) ? kOob : voff_b[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (lds_void_t*)(slot + BM * BK + (i * NW + w) * 1024), 16, vo, so, 0, 0);
      }
    }
  };

  // fragment reads: lane reads row (base + (lane & 31)), k chunk 2 * kk + (lane >> 5);
  // bases are multiples of 32 rows, so the swizzle depends on lane & 31 only
  const int fr = lane & 31, fk = lane >> 5;
  const int fsw = (fr / RPW) % CPR;
  const int off_a = (wm * WM + fr) * BK;
  const int off_b = BM * BK + (wn * WN + fr) * BK;

  typedef typename MmaKind<OUT>::acc_t acc_t;
  acc_t acc[FN][FM];
#pragma unroll
  for (int a = 0; a < FN; ++a)
#pragma unroll
    for (int b = 0; b < FM; ++b) acc[a][b] = acc_t{};

  // fragment f of a lane is chunks FR * (2 * kk + fk) + f of its row (f < FR)
  v4i fb0[FN * FR], fa0[FM * FR], fb1[FN * FR], fa1[FM * FR];
  auto read_frags = [&](int st, int kk, v4i* fb, v4i* fa) {
    const int8_t* slot = lds + (st % NST) * SLOT;
#pragma unroll
    for (int f = 0; f < FR; ++f) {
      const int ch = ((FR * (2 * kk + fk) + f) ^ fsw) << 4;
#pragma unroll
      for (int a = 0; a < FN; ++a) fb[a * FR + f] = *(const v4i*)(slot + off_b + a * 32 * BK + ch);
#pragma unroll
      for (int b = 0; b < FM; ++b) fa[b * FR + f] = *(const v4i*)(slot + off_a + b * 32 * BK + ch);
    }
  };
  auto mfmas = [&](const v4i* fb, const v4i* fa) {
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
      for (int b = 0; b < FM; ++b)
        acc[a][b] = MmaKind<OUT>::mma(fb + a * FR, fa + b * FR, acc[a][b]);
  };

  // Pipeline (stage s lives in slot s % NST).  Iteration kt computes stage kt
  // as KK steps of 32-deep k (64-deep for FP8); the fragments of step kk+1 are
  // read while the MFMAs of step kk run.  Before the last step the stage
  // barrier is taken: each wave first waits for its own loads of stage kt+1
  // and for its own reads of slot kt, so after the barrier stage kt+1 is
  // visible to every wave and slot kt is free.
  //
  // Where the loads go matters because a SIMD whose two waves both have
  // loads waiting to issue leaves its matrix pipe idle (measured: the MFMA
  // rate with a stage of loads in flight is that of MFMAs alone only when one
  // of the two waves per SIMD issues all of them).  So:
  //  - NST >= 3: the loads of stage kt+NST-1 go into the slot freed at the
  //    previous barrier, spread over the first KK-1 steps of iteration kt,
  //    PER per step, each wave its own; NST-2 stages stay in flight.
  //  - NST == 2 with 8 waves: the loads of stage kt+2 go into slot kt right
  //    after the barrier, all issued by waves 0..3 (one per SIMD), each its
  //    own and those of wave + 4, while waves 4..7 only compute.
  //  - NST == 2 with 4 waves: each wave issues its own after the barrier.
  constexpr bool kSpread = NST >= 3;
  constexpr bool kHalf = !kSpread && NW == 8;
  constexpr int LW = kHalf ? 2 * L : L;              // loads per stage of a loading wave
  constexpr int PER = (LW + KK - 2) / (KK - 1);      // loads per step when spread
  static_assert(KK >= 2, "unsupported stage depth");
  static_assert(!kHalf || ((NW / 2) * RPI / RPW) % CPR == 0, "half-wave load swizzle");
  const bool loader = !kHalf || wave < NW / 2;
  auto step_ptrs = [&](int kk, v4i*& cb, v4i*& ca, v4i*& nb, v4i*& na) {
    cb = (kk & 1) ? fb1 : fb0;
    ca = (kk & 1) ? fa1 : fa0;
    nb = (kk & 1) ? fb0 : fb1;
    na = (kk & 1) ? fa0 : fa1;
  };
  if (nk > 0) {
    // prologue: the stages in flight before iteration 0
    constexpr int PRE = kSpread ? NST - 1 : NST;
    if (loader) {
#pragma unroll
      for (int st = 0; st < PRE; ++st) dma(st, 0, LW);
    }
    wait_vmcnt<(PRE - 1) * LW>();  // stage 0 landed
    block_barrier();
    read_frags(0, 0, fb0, fa0);
    for (int kt = 0; kt < nk - 1; ++kt) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        v4i *cb, *ca, *nb, *na;
        step_ptrs(kk, cb, ca, nb, na);
        if (kk + 1 < KK) {
          read_frags(kt, kk + 1, nb, na);
          if constexpr (kSpread) {
            dma(kt + NST - 1, kk * PER, min((kk + 1) * PER, LW));
            mfmas(cb, ca);
            interleave<0, FN * FM, FR * (FN + FM), PER, FR * (FN + FM)>();
          } else {
            mfmas(cb, ca);
            interleave<0, FN * FM, FR * (FN + FM), 0>();
          }
        } else {
          wait_vmcnt<(NST - 2) * LW>();  // this wave's loads of stage kt+1 landed
          wait_lgkmcnt0();               // this wave's reads of slot kt are done
          block_barrier();               // every wave: stage kt+1 landed, slot kt free
          if (!kSpread && loader) {
            dma(kt + NST, 0, LW);
            read_frags(kt + 1, 0, nb, na);
            mfmas(cb, ca);
            interleave<0, FN * FM, FR * (FN + FM), LW>();
          } else {
            read_frags(kt + 1, 0, nb, na);
            mfmas(cb, ca);
            interleave<0, FN * FM, FR * (FN + FM), 0>();
          }
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      v4i *cb, *ca, *nb, *na;
      step_ptrs(kk, cb, ca, nb, na);
      if (kk + 1 < KK) read_frags(nk - 1, kk + 1, nb, na);
      mfmas(cb, ca);
    }
    wait_vmcnt<0>();  // no LDS-mode load may outlive the block's LDS
  }

  // Epilogue.  A lane holds, for register group g of fragment (a, b), output
  // channels n .. n+3 of token m, with m = b * 32 + (lane & 31) and
  // n = a * 32 + g * 8 + (lane >> 5) * 4 inside the wave tile.  Stored like
  // that, a wave store would cover 32 rows with 16 bytes each, and the store
  // path, which pays per request, would run at a quarter of its byte rate.
  // So the results go through LDS, one 32-token slab of the wave tile at a
  // time: each wave writes its slab into a private staging area and reads it
  // back row-major, 16 contiguous bytes per lane, for full-line global stores.
  // The staging row pitch is an odd number of 16-byte chunks, so the 32 rows
  // of a slab write fall on distinct bank groups.
  //
  // The dequant scales are loaded before any store: the memory counter that
  // their loads are waited on also counts stores, so a scale load issued after
  // a store would make its use wait for that store to complete.  Indices are
  // clamped so the loads stay in bounds; stores are guarded (N % 8 == 0, so a
  // 16-byte chunk of a row is either inside N or wholly outside).
  constexpr int ES = OUT == 0 ? 4 : 2;  // output element bytes
  constexpr int CPO = WN * ES / 16;     // 16-byte output chunks per wave-tile row
  constexpr int PITCH = WN * ES + 16;   // staging row pitch in bytes
  static_assert((PITCH / 16) % 2 == 1 && NW * 32 * PITCH <= NST * SLOT && (32 * CPO) % 64 == 0,
                "epilogue staging");
  const int hi = lane >> 5;
  constexpr bool kDequant = OUT == 1 || OUT == 2 || OUT == 5 || OUT == 6;
  float am[FM];
  float4 bn[FN][4];
  if constexpr (kDequant) {
#pragma unroll
    for (int b = 0; b < FM; ++b) am[b] = sa[min(m0 + wm * WM + b * 32 + (lane & 31), M - 1)];
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        bn[a][g] = *(const float4*)(sb + min(n0 + wn * WN + a * 32 + g * 8 + hi * 4, N - 4));
  }
  // every wave is past its last fragment read and its last LDS-mode load
  wait_lgkmcnt0();
  block_barrier();
  int8_t* stage = lds + wave * 32 * PITCH;
#pragma unroll
  for (int b = 0; b < FM; ++b) {
#pragma unroll
    for (int a = 0; a < FN; ++a) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const acc_t& C = acc[a][b];
        int8_t* dst = stage + (lane & 31) * PITCH + (a * 32 + g * 8 + hi * 4) * ES;
        if constexpr (OUT == 0) {
          *(v4i*)dst = v4i{(int)C[4 * g + 0], (int)C[4 * g + 1], (int)C[4 * g + 2], (int)C[4 * g + 3]};
        } else {
          unsigned short h[4];
          if constexpr (OUT == 3 || OUT == 4) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              h[e] = OUT == 3 ? f32_to_f16_rne((float)C[4 * g + e]) : f32_to_bf16_rne((float)C[4 * g + e]);
          } else {
            const float w[4] = {bn[a][g].x, bn[a][g].y, bn[a][g].z, bn[a][g].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float y = (float)C[4 * g + e];
              y = y * am[b];
              y = y * w[e];
              h[e] = (OUT == 1 || OUT == 5) ? f32_to_f16_rne(y) : f32_to_bf16_rne(y);
            }
          }
          *(uint2*)dst = uint2{(unsigned)h[0] | ((unsigned)h[1] << 16),
                               (unsigned)h[2] | ((unsigned)h[3] << 16)};
        }
      }
    }
    // read the slab back row-major (LDS operations of one wave complete in
    // order, so the reads see the writes above and precede the next slab's)
    constexpr int NR = 32 * CPO / 64;
    v4i v[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int f = i * 64 + lane;
      v[i] = *(const v4i*)(stage + (f / CPO) * PITCH + (f % CPO) * 16);
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int f = i * 64 + lane;
      const int m = m0 + wm * WM + b * 32 + f / CPO;
      const int n = n0 + wn * WN + (f % CPO) * (16 / ES);
      if (m < M && n < N) *(v4i*)((int8_t*)out + ((int64_t)m * ldc + n) * ES) = v[i];
    }
  }
}

template <int BM, int BN, int BK, int NST, int WGM, int WGN, int OUT>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WGM * WGN, 64 * WGM * WGN),
                          amdgpu_waves_per_eu(WGM * WGN / 4, WGM * WGN / 4))) void
k_gemm_i8(const int8_t* __restrict__ qa, const int8_t* __restrict__ qb, int M, int N, int K,
          const float* __restrict__ sa, const float* __restrict__ sb, void* __restrict__ out,
          int m_tiles, int n_tiles) {
  int tm, tn;
  tile_of(blockIdx.x, m_tiles, n_tiles, tm, tn);
  gemm_tile<BM, BN, BK, NST, WGM, WGN, OUT>(qa, qb, M, N, K, sa, sb, out, N, tm, tn);
}

// Two tile shapes in one grid, for a channel count whose tiles of the larger
// shape leave the last wave of blocks part-empty: the first n1 channels run
// as whole waves of BN1-channel tiles (blocks 0 .. m_tiles * nt1 - 1, a
// multiple of 256 and so of the 8 XCDs, which keeps the tile order per XCD),
// and the rest as BN2-channel tiles in the blocks after them, which the
// dispatcher starts as CUs free up.  Both shapes use 8 waves, 256-token tiles
// and 128-byte stages.
template <int BN1, int NST1, int WGM1, int WGN1, int BN2, int NST2, int WGM2, int WGN2, int OUT>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2))) void
k_gemm_i8_two(const int8_t* __restrict__ qa, const int8_t* __restrict__ qb, int M, int N, int K,
              const float* __restrict__ sa, const float* __restrict__ sb, void* __restrict__ out,
              int m_tiles, int nt1, int n1, int nt2) {
  static_assert(WGM1 * WGN1 == 8 && WGM2 * WGN2 == 8, "8-wave tiles");
  constexpr int ES = OUT == 0 ? 4 : 2;  // output element bytes
  const int t1 = m_tiles * nt1;
  int tm, tn;
  if ((int)blockIdx.x < t1) {
    tile_of(blockIdx.x, m_tiles, nt1, tm, tn);
    gemm_tile<256, BN1, 128, NST1, WGM1, WGN1, OUT>(qa, qb, M, n1, K, sa, sb, out, N, tm, tn);
  } else {
    tile_of(blockIdx.x - t1, m_tiles, nt2, tm, tn);
    gemm_tile<256, BN2, 128, NST2, WGM2, WGN2, OUT>(qa, qb + (int64_t)n1 * K, M, N - n1, K, sa,
                                                    sb + n1, (int8_t*)out + (int64_t)n1 * ES, N,
                                                    tm, tn);
  }
}

// Skinny GEMM for few tokens (decode-like M <= 32): the product is weight
// streaming, so the tiling follows the weight.  A block owns 16 output
// channels over all of K and all M tokens; its NW waves split K (below: by
// interleaved 64-deep k steps, or by contiguous ranges when K is long).  Each
// step is one v_mfma_i32_16x16x64_i8 per 16 tokens with the weight fragment
// as the first operand (16 channels x 64 k) and the activation fragment as the second
// (64 k x 16 tokens).  Operands load straight into registers with buffer
// loads, U steps in flight per wave; token rows past M and channel rows past N
// are outside their buffer resources and read as zero without touching
// memory.  The waves' partial int32 sums are added exactly through LDS, and
// one wave applies the same dequant epilogue as the tiled kernel (each lane
// holds 4 consecutive channels of one token).
template <int MT, int NW, int OUT>
__global__ __launch_bounds__(64 * NW) void k_gemm_skinny(
    const int8_t* __restrict__ qa, const int8_t* __restrict__ qb, int M, int N, int K,
    const float* __restrict__ sa, const float* __restrict__ sb, void* __restrict__ out) {
  constexpr int U = 8;  // k steps in flight per wave
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 16;
  const rsrc_t rw = make_rsrc(qb + (int64_t)n0 * K, (unsigned)min(16, N - n0) * (unsigned)K);
  const rsrc_t rx = make_rsrc(qa, (unsigned)M * (unsigned)K);
  const int r16 = lane & 15, kq = lane >> 4;  // fragment row, 16-byte k chunk
  const int voff_w = r16 * K + kq * 16;
  int voff_x[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) voff_x[t] = (t * 16 + r16) * K + kq * 16;

  v4i acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = v4i{0, 0, 0, 0};
  // Which 64-deep k steps a wave takes: with at least two batches per wave
  // (K >= 8192), a contiguous range of K per wave; otherwise steps
  // interleaved across the waves.  Measured on 16384 -> 4096 at 1-16 tokens,
  // the contiguous ranges are 6-16% faster; on 4096 -> 16384 and
  // 4096 -> 12288 (one batch per wave) the interleaved order is 0-10% faster.
  const int nsteps = (K + 63) / 64;
  const bool contig = nsteps >= 2 * NW * U;
  const int per = (nsteps + NW - 1) / NW;
  const int first = contig ? wave * per : wave;
  const int last = contig ? min(nsteps, first + per) : nsteps;
  const int du = contig ? 1 : NW;  // distance between a wave's consecutive steps
  for (int s0 = first; s0 < last; s0 += du * U) {
    v4i w[U], x[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int st = s0 + u * du;
      const int k0 = st * 64;
      const bool out_k = st >= last || k0 + kq * 16 >= K;
      w[u] = __builtin_amdgcn_raw_buffer_load_b128(rw, out_k ? kOob : voff_w, k0, 0);
#pragma unroll
      for (int t = 0; t < MT; ++t)
        x[u][t] = __builtin_amdgcn_raw_buffer_load_b128(rx, out_k ? kOob : voff_x[t], k0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < MT; ++t)
        acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[u], x[u][t], acc[t], 0, 0, 0);
  }

  // exact sum of the waves' partial accumulators
  __shared__ v4i red[NW][MT][64];
#pragma unroll
  for (int t = 0; t < MT; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    v4i c = red[0][t][lane];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) c += red[w2][t][lane];
    // lane holds channels n .. n+3 of token m
    const int m = t * 16 + (lane & 15);
    const int n = n0 + 4 * (lane >> 4);
    if (m >= M || n >= N) continue;
    if (OUT == 0) {
      *(v4i*)((int32_t*)out + (int64_t)m * N + n) = c;
    } else {
      const float am = sa[m];
      const float4 bn = *(const float4*)(sb + n);
      const float wv[4] = {bn.x, bn.y, bn.z, bn.w};
      unsigned short h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float y = (float)c[e];
        y = y * am;
        y = y * wv[e];
        h[e] = OUT == 1 ? f32_to_f16_rne(y) : f32_to_bf16_rne(y);
      }
      uint2 o;
      o.x = (unsigned)h[0] | ((unsigned)h[1] << 16);
      o.y = (unsigned)h[2] | ((unsigned)h[3] << 16);
      *(uint2*)((unsigned short*)out + (int64_t)m * N + n) = o;
    }
  }
}

template <int MT>
hipError_t launch_skinny(const int8_t* qa, const int8_t* qb, int64_t M, int64_t N, int64_t K,
                         const float* sa, const float* sb, void* out, int mode, hipStream_t st) {
  constexpr int NW = 8;
  const dim3 grid((unsigned)((N + 15) / 16)), block(64 * NW);
  switch (mode) {
    case 0:
      hipLaunchKernelGGL((k_gemm_skinny<MT, NW, 0>), grid, block, 0, st, qa, qb, (int)M, (int)N,
                         (int)K, sa, sb, out);
      break;
    case 1:
      hipLaunchKernelGGL((k_gemm_skinny<MT, NW, 1>), grid, block, 0, st, qa, qb, (int)M, (int)N,
                         (int)K, sa, sb, out);
      break;
    default:
      hipLaunchKernelGGL((k_gemm_skinny<MT, NW, 2>), grid, block, 0, st, qa, qb, (int)M, (int)N,
                         (int)K, sa, sb, out);
      break;
  }
  return hipGetLastError();
}

// Split-K few-token GEMM (the runtime forward's path for 17 <= M <= 32, where
// the skinny kernel's per-16-channel re-reading of the activations costs more
// than splitting K; measured slower than the skinny kernel below 17).  A block
// owns 16 * CT output channels and one of S contiguous ranges of 64-deep k
// steps; its NW waves take the steps of that range in turn.  Per step a wave
// loads CT weight fragments and MT activation fragments straight into
// registers and issues CT * MT v_mfma_i32_16x16x64_i8, so each activation
// fragment serves CT weight fragments (the skinny kernel re-reads the whole
// activation once per 16 channels).  The waves' int32 partials add exactly
// through LDS.  With S == 1 the block applies the dequant epilogue itself;
// otherwise it stores its int32 partial slice (rows < M) and
// k_splitk_reduce adds the S slices exactly and dequantizes.
template <int MT, int CT, int U, int OUT>
__global__ __launch_bounds__(512) void k_gemm_splitk(const int8_t* __restrict__ qa,
                                                     const int8_t* __restrict__ qb, int M, int N,
                                                     int K, int steps_per_split,
                                                     const float* __restrict__ sa,
                                                     const float* __restrict__ sb,
                                                     void* __restrict__ out) {
  constexpr int NW = 8;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 16 * CT;
  const int split = blockIdx.y;
  const int nsteps = (K + 63) / 64;
  const int st0 = split * steps_per_split;
  const int st1 = min(nsteps, st0 + steps_per_split);
  const rsrc_t rw = make_rsrc(qb + (int64_t)n0 * K, (unsigned)min(16 * CT, N - n0) * (unsigned)K);
  const rsrc_t rx = make_rsrc(qa, (unsigned)M * (unsigned)K);
  const int r16 = lane & 15, kq = lane >> 4;  // fragment row, 16-byte k chunk
  int voff_w[CT], voff_x[MT];
#pragma unroll
  for (int c = 0; c < CT; ++c) voff_w[c] = (c * 16 + r16) * K + kq * 16;
#pragma unroll
  for (int t = 0; t < MT; ++t) voff_x[t] = (t * 16 + r16) * K + kq * 16;

  v4i acc[CT][MT];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[c][t] = v4i{0, 0, 0, 0};
  for (int s0 = st0 + wave; s0 < st1; s0 += NW * U) {
    v4i w[U][CT], x[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int st = s0 + u * NW;
      const int k0 = st * 64;
      const bool out_k = st >= st1 || k0 + kq * 16 >= K;
#pragma unroll
      for (int c = 0; c < CT; ++c)
        w[u][c] = __builtin_amdgcn_raw_buffer_load_b128(rw, out_k ? kOob : voff_w[c], k0, 0);
#pragma unroll
      for (int t = 0; t < MT; ++t)
        x[u][t] = __builtin_amdgcn_raw_buffer_load_b128(rx, out_k ? kOob : voff_x[t], k0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[c][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[u][c], x[u][t], acc[c][t], 0, 0, 0);
  }

  // exact sum of the waves' partials; fragment f is finished by wave f % NW
  __shared__ v4i red[NW][CT * MT][64];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int t = 0; t < MT; ++t) red[wave][c * MT + t][lane] = acc[c][t];
  __syncthreads();
  for (int f = wave; f < CT * MT; f += NW) {
    v4i cs = red[0][f][lane];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) cs += red[w2][f][lane];
    // lane holds channels n .. n+3 of token m
    const int m = (f % MT) * 16 + (lane & 15);
    const int n = n0 + (f / MT) * 16 + 4 * (lane >> 4);
    if (m >= M || n >= N) continue;
    if (OUT == 0) {
      *(v4i*)((int32_t*)out + ((int64_t)split * M + m) * N + n) = cs;
    } else {
      const float am = sa[m];
      const float4 bn = *(const float4*)(sb + n);
      const float wv[4] = {bn.x, bn.y, bn.z, bn.w};
      unsigned short h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float y = (float)cs[e];
        y = y * am;
        y = y * wv[e];
        h[e] = OUT == 1 ? f32_to_f16_rne(y) : f32_to_bf16_rne(y);
      }
      uint2 o;
      o.x = (unsigned)h[0] | ((unsigned)h[1] << 16);
      o.y = (unsigned)h[2] | ((unsigned)h[3] << 16);
      *(uint2*)((unsigned short*)out + (int64_t)m * N + n) = o;
    }
  }
}

// Exact int32 sum of the S partial slices (S x M x N), then the dequant
// epilogue; one thread per 4 consecutive channels of one token.
template <int OUT>
__global__ __launch_bounds__(256) void k_splitk_reduce(const int32_t* __restrict__ part, int S,
                                                       int M, int N, const float* __restrict__ sa,
                                                       const float* __restrict__ sb,
                                                       void* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (m, n / 4)
  const int n4 = N / 4;
  if (i >= (int64_t)M * n4) return;
  const int m = (int)(i / n4), n = (int)(i % n4) * 4;
  v4i c = *(const v4i*)(part + (int64_t)m * N + n);
  for (int s = 1; s < S; ++s) c += *(const v4i*)(part + ((int64_t)s * M + m) * N + n);
  const float am = sa[m];
  const float4 bn = *(const float4*)(sb + n);
  const float wv[4] = {bn.x, bn.y, bn.z, bn.w};
  unsigned short h[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float v = (float)c[e];
    v = v * am;
    v = v * wv[e];
    h[e] = OUT == 1 ? f32_to_f16_rne(v) : f32_to_bf16_rne(v);
  }
  uint2 o;
  o.x = (unsigned)h[0] | ((unsigned)h[1] << 16);
  o.y = (unsigned)h[2] | ((unsigned)h[3] << 16);
  *(uint2*)((unsigned short*)y + (int64_t)m * N + n) = o;
}

template <int MT, int OUT>
void launch_splitk_kernel(const int8_t* qa, const int8_t* qb, int M, int N, int K, int s, int spp,
                          const float* sa, const float* sb, void* out, hipStream_t st) {
  constexpr int CT = kSplitkCT, U = 3;
  const dim3 grid((unsigned)((N + 16 * CT - 1) / (16 * CT)), (unsigned)s), block(512);
  hipLaunchKernelGGL((k_gemm_splitk<MT, CT, U, OUT>), grid, block, 0, st, qa, qb, M, N, K, spp, sa,
                     sb, out);
}

template <int BM, int BN, int BK, int NST, int WGM, int WGN>
hipError_t launch_tile(const int8_t* qa, const int8_t* qb, int64_t M, int64_t N, int64_t K,
                       const float* sa, const float* sb, void* out, int mode, hipStream_t st) {
  const int mt = (int)((M + BM - 1) / BM), nt = (int)((N + BN - 1) / BN);
  const dim3 grid((unsigned)(mt * nt)), block(64 * WGM * WGN);
  switch (mode) {
    case 0:
      hipLaunchKernelGGL((k_gemm_i8<BM, BN, BK, NST, WGM, WGN, 0>), grid, block, 0, st, qa, qb, (int)M,
                         (int)N, (int)K, sa, sb, out, mt, nt);
      break;
    case 1:
      hipLaunchKernelGGL((k_gemm_i8<BM, BN, BK, NST, WGM, WGN, 1>), grid, block, 0, st, qa, qb, (int)M,
                         (int)N, (int)K, sa, sb, out, mt, nt);
      break;
    case 2:
      hipLaunchKernelGGL((k_gemm_i8<BM, BN, BK, NST, WGM, WGN, 2>), grid, block, 0, st, qa, qb, (int)M,
                         (int)N, (int)K, sa, sb, out, mt, nt);
      break;
    case 3:
      hipLaunchKernelGGL((k_gemm_i8<BM, BN, BK, NST, WGM, WGN, 3>), grid, block, 0, st, qa, qb, (int)M,
                         (int)N, (int)K, sa, sb, out, mt, nt);
      break;
    case 4:
      hipLaunchKernelGGL((k_gemm_i8<BM, BN, BK, NST, WGM, WGN, 4>), grid, block, 0, st, qa, qb, (int)M,
                         (int)N, (int)K, sa, sb, out, mt, nt);
      break;
    case 5:
      hipLaunchKernelGGL((k_gemm_i8<BM, BN, BK, NST, WGM, WGN, 5>), grid, block, 0, st, qa, qb, (int)M,
                         (int)N, (int)K, sa, sb, out, mt, nt);
      break;
    default:
      hipLaunchKernelGGL((k_gemm_i8<BM, BN, BK, NST, WGM, WGN, 6>), grid, block, 0, st, qa, qb, (int)M,
                         (int)N, (int)K, sa, sb, out, mt, nt);
      break;
  }
  return hipGetLastError();
}

// The two-shape grid: whole waves of 256 x 256 tiles over the first
// nt1 * 256 channels, 256 x 192 tiles over the rest.
hipError_t launch_two(const int8_t* qa, const int8_t* qb, int64_t M, int64_t N, int64_t K,
                      const float* sa, const float* sb, void* out, int mode, hipStream_t st,
                      int mt, int nt1) {
  const int n1 = nt1 * 256;
  const int nt2 = (int)((N - n1 + 191) / 192);
  const dim3 grid((unsigned)(mt * (nt1 + nt2))), block(512);
#define W8A8_TWO(O)                                                                               \
  hipLaunchKernelGGL((k_gemm_i8_two<256, 2, 2, 4, 192, 2, 4, 2, O>), grid, block, 0, st, qa, qb, \
                     (int)M, (int)N, (int)K, sa, sb, out, mt, nt1, n1, nt2)
  switch (mode) {
    case 0: W8A8_TWO(0); break;
    case 1: W8A8_TWO(1); break;
    case 2: W8A8_TWO(2); break;
    case 3: W8A8_TWO(3); break;
    case 4: W8A8_TWO(4); break;
    case 5: W8A8_TWO(5); break;
    default: W8A8_TWO(6); break;
  }
#undef W8A8_TWO
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const int8_t* qa, const int8_t* qb, int64_t M, int64_t N, int64_t K,
                       const float* sa, const float* sb, void* out, int out_mode,
                       hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  // fp16 / bf16 operands: K counts elements; the tiled kernel works in bytes.
  // The skinny few-token kernel serves the INT8 modes only.
  const bool tiled_only = out_mode >= 3;
  if (out_mode == 3 || out_mode == 4) K *= 2;
  // Few tokens: weight streaming.  12 to 32 tokens over at least 192 blocks
  // of 64 channels: the split-K
  // kernel with one K range per block.  Each of its activation fragments
  // serves four weight fragments, where the skinny kernel re-reads the
  // activations once per 16 channels (at 16 tokens that doubles its operand
  // stream); below 12 tokens, or with fewer blocks, the skinny kernel is as
  // fast or faster.
  if (!tiled_only && M >= 12 && M <= 32 && N >= 192 * 16 * kSplitkCT) {
    const int nst = (int)((K + 63) / 64);
    if (M <= 16) {
      if (out_mode == 0) launch_splitk_kernel<1, 0>(qa, qb, (int)M, (int)N, (int)K, 1, nst, sa, sb, out, st);
      else if (out_mode == 1) launch_splitk_kernel<1, 1>(qa, qb, (int)M, (int)N, (int)K, 1, nst, sa, sb, out, st);
      else launch_splitk_kernel<1, 2>(qa, qb, (int)M, (int)N, (int)K, 1, nst, sa, sb, out, st);
    } else {
      if (out_mode == 0) launch_splitk_kernel<2, 0>(qa, qb, (int)M, (int)N, (int)K, 1, nst, sa, sb, out, st);
      else if (out_mode == 1) launch_splitk_kernel<2, 1>(qa, qb, (int)M, (int)N, (int)K, 1, nst, sa, sb, out, st);
      else launch_splitk_kernel<2, 2>(qa, qb, (int)M, (int)N, (int)K, 1, nst, sa, sb, out, st);
    }
    return hipGetLastError();
  }
  // Otherwise the skinny kernel; between 17 and 32 tokens it reads two
  // activation fragments per step, and the tiled kernel is as fast once N
  // alone gives it 128 or more blocks.
  if (!tiled_only && M <= 16) return launch_skinny<1>(qa, qb, M, N, K, sa, sb, out, out_mode, st);
  if (!tiled_only && M <= 32 && N < 16384)
    return launch_skinny<2>(qa, qb, M, N, K, sa, sb, out, out_mode, st);
  // Pick the tile whose last wave of blocks over 256 CUs is fullest, with a
  // small preference for the larger tile (more MACs per byte of LDS traffic).
  struct Cand { int bm, bn; double eff; };
  // eff: operand bytes per MFMA, which the load-return path into LDS limits,
  // fall with the tile's BM * BN / (BM + BN)
  const Cand cands[] = {{256, 256, 1.0}, {256, 128, 0.92}, {128, 128, 0.8}, {256, 192, 0.96}};
  int best = 0;
  double best_score = -1.0;
  for (int i = 0; i < 4; ++i) {
    const int64_t tiles = ((M + cands[i].bm - 1) / cands[i].bm) * ((N + cands[i].bn - 1) / cands[i].bn);
    const int64_t waves = (tiles + 255) / 256;
    const double fill = (double)tiles / (double)(waves * 256);
    // useful fraction of the padded tile rows
    const double mfill = (double)M / (double)(((M + cands[i].bm - 1) / cands[i].bm) * cands[i].bm);
    const double score = fill * mfill * cands[i].eff;
    if (score > best_score + 1e-9) { best_score = score; best = i; }
  }
  // Two tile shapes in one grid when the 256 x 256 tiles leave the last wave
  // part-empty: whole waves of them, then 256 x 192 tiles over the remaining
  // channels.  The estimate counts waves of blocks times the cycles per stage
  // measured for each tile at the same clock (2339 for 256 x 256, 1853 for
  // 256 x 192, 1404 for 256 x 128); the split is taken when it is 3% or more
  // below the single shape's.  Measured: gate_up 4096 -> 22016 at 2048 tokens
  // 155 -> 152 us, and the OPT-30B 7168-channel layers 2% faster.
  if (cands[best].bm == 256) {
    const int64_t mt = (M + 255) / 256;
    const int64_t cyc[4] = {2339, 1404, 0, 1853};
    const int64_t tiles = mt * ((N + cands[best].bn - 1) / cands[best].bn);
    const int64_t single = (tiles + 255) / 256 * cyc[best];
    const int64_t w = mt * ((N + 255) / 256) / 256;
    if (w >= 1 && (w * 256) % mt == 0 && w * 256 / mt * 256 < N) {
      const int64_t nt1 = w * 256 / mt;
      const int64_t nt2 = (N - nt1 * 256 + 191) / 192;
      const int64_t two = w * cyc[0] + (mt * nt2 + 255) / 256 * cyc[3];
      if (two * 100 <= single * 97)
        return launch_two(qa, qb, M, N, K, sa, sb, out, out_mode, st, (int)mt, (int)nt1);
    }
  }
  // template arguments after the tile: stage bytes BK, LDS slots NST, waves WGM x WGN
  switch (best) {
    case 0: return launch_tile<256, 256, 128, 2, 2, 4>(qa, qb, M, N, K, sa, sb, out, out_mode, st);
    case 1: return launch_tile<256, 128, 128, 3, 4, 2>(qa, qb, M, N, K, sa, sb, out, out_mode, st);
    case 3: return launch_tile<256, 192, 128, 2, 4, 2>(qa, qb, M, N, K, sa, sb, out, out_mode, st);
    default: return launch_tile<128, 128, 128, 4, 2, 2>(qa, qb, M, N, K, sa, sb, out, out_mode, st);
  }
}


SplitkPlan splitk_plan(int64_t M, int64_t N, int64_t K) {
  SplitkPlan p{1, 0};
  if (M < 17 || M > 32 || N < 1 || K < 1) return p;
  const int64_t tiles = (N + 16 * kSplitkCT - 1) / (16 * kSplitkCT);
  const int64_t nsteps = (K + 63) / 64;
  // about one block per CU, and at least 32 k steps (2 KiB of each weight row)
  // per split; with 192 or more channel tiles one K range per block is faster
  // than splitting (measured on a 4096 -> 12288 layer at 17-32 tokens)
  int64_t s = tiles >= 192 ? 1 : (256 + tiles - 1) / tiles;
  s = std::min<int64_t>(s, std::max<int64_t>(1, nsteps / 32));
  s = std::min<int64_t>(s, 16);
  p.splits = (int)s;
  p.steps_per_split = (int)((nsteps + s - 1) / s);
  return p;
}

hipError_t launch_gemm_splitk(const int8_t* qa, const int8_t* qb, int64_t M, int64_t N, int64_t K,
                              const float* sa, const float* sb, void* y, bool bf16,
                              int32_t* partials, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  const SplitkPlan p = splitk_plan(M, N, K);
  if (p.steps_per_split == 0) return hipErrorInvalidValue;
  const int m = (int)M, n = (int)N, k = (int)K;
  if (p.splits == 1) {
    if (bf16) launch_splitk_kernel<2, 2>(qa, qb, m, n, k, 1, p.steps_per_split, sa, sb, y, st);
    else launch_splitk_kernel<2, 1>(qa, qb, m, n, k, 1, p.steps_per_split, sa, sb, y, st);
    return hipGetLastError();
  }
  launch_splitk_kernel<2, 0>(qa, qb, m, n, k, p.splits, p.steps_per_split, sa, sb, partials, st);
  const int64_t threads = M * (N / 4);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (bf16)
    hipLaunchKernelGGL(k_splitk_reduce<2>, grid, block, 0, st, partials, p.splits, m, n, sa, sb, y);
  else
    hipLaunchKernelGGL(k_splitk_reduce<1>, grid, block, 0, st, partials, p.splits, m, n, sa, sb, y);
  return hipGetLastError();
}


}  // namespace w8a8
