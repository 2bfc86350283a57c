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
// contiguous.  Every INT8 MFMA is v_mfma_i32_16x16x64_i8 with the weight
// fragment as its first operand (16 output channels x 64 k) and the
// activation fragment as its second (64 k x 16 tokens), so that each lane's
// four accumulator registers hold four consecutive output channels of one
// token.  Integer accumulation is exact and order free.  The epilogue
// dequantizes in registers and restages each wave's results through LDS so
// that every global store writes whole rows of 16 bytes per lane.
//
// Block: WGM x WGN waves (8 for the 256-row tiles, 4 for 128 x 128) own a
// BM x BN output tile (tokens x channels); wave (wm, wn) holds a
// (BM / WGM) x (BN / WGN) register tile of MFMA blocks (16 x 16 for INT8,
// 32 x 32 for the 16-bit and FP8 forms, see MmaKind).  Tiles:
// 256 x 256, 256 x 192, 256 x 128 and 128 x 128; launch_gemm picks the one
// whose last wave of blocks over the 256 CUs is fullest, preferring fewer
// operand bytes per MFMA (the return path of the operand loads is the
// limiting resource).
//
// K pipeline: K advances BK = 128 bytes per stage (one full cache line per
// operand row) through NST LDS slots (2 to 4, as many as 160 KB of LDS holds
// for the tile; the single-shape 256 x 256 tile keeps a third slot for its
// weights).  Operand rows go from global memory straight into LDS with
// buffer loads in LDS mode (16 B per lane, each wave instruction fills 1 KiB
// of LDS), NST - 1 or NST - 2 stages in flight while one is computed, and a
// wave never holds global data in registers.  Which waves issue a stage's
// loads, and when, is set by the slot count (see the pipeline in the kernel):
// a SIMD stalls its matrix pipe while both of its waves have loads waiting to
// issue, so with two slots one wave per SIMD issues them all.  Stages past the
// end are issued with out-of-range offsets (no memory traffic) so the
// per-stage load count, and with it every vmcnt wait, is constant.
//
// Per stage a wave runs BK / KSTEP k steps (KSTEP = 64 bytes for INT8 and
// FP8, 32 for fp16 / bf16) of (BM / WGM / MB) x (BN / WGN / MB) MFMAs.  The
// fragment reads are software pipelined: the next k step's fragments are read
// while the current step's MFMAs run (the larger operand in place, column by
// column; before a stage barrier the last column's fragment early, into
// registers of its own), and the next stage's first fragments are read (after
// the stage barrier) while the last step's MFMAs run.  One
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
// and every row offset is part of the range-checked vector offset, so rows
// past M or N load as zero without a memory access; chunks past K use an
// out-of-range offset and load as zero too.  Blocks are dispatched
// round-robin over the 8 XCDs; tile indices are remapped so each XCD (own L2)
// gets a contiguous run of tiles, ordered token-tile fastest in groups of 8
// token tiles.
//
// The same pipeline serves the dense fp16 / bf16 product (the comparison
// baseline) and the FP8 E4M3 variant; few-token shapes go to k_gemv_rows (one
// or two tokens) and k_gemm_fewtok (3 to 32, up to 128 on narrower layers;
// in the runtime forward its
// split-K form on narrow layers with long rows, below).
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace w8a8 {

namespace {

constexpr int kGroupM = 8;       // token tiles per ordering group
constexpr unsigned kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)
constexpr int kOob = 0x40000000;  // voffset that is out of range for every resource here
constexpr int kGemvRows = 4;      // output channels per block of the row-streaming kernel
constexpr int kGemvMaxM = 2;      // token counts that take the row-streaming kernel
constexpr int kEarlyCols = 1;     // in-place fragments read early before a stage barrier
constexpr bool kDeepB = true;     // single-shape 256 x 256 tile: a third weight slot

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
// Geometry of an MFMA: it multiplies an MB x KSTEP block of the weight by a
// KSTEP x MB block of the activations (MB = 32 or 16 rows each).  A lane's
// fragment of a block is FR 16-byte chunks of row lane % MB, k chunks
// FR * (lane / MB) .. + FR - 1 of the k step, so KSTEP = 16 * FR * 64 / MB
// bytes.  A lane's accumulators hold, for group g < NACC / 4, the four
// consecutive output channels g * (256 / MB) + (lane / MB) * 4 .. + 3 of
// token lane % MB.  The byte-addressed LDS pipeline is the same for all.
//   int8:       16 x 16 x 64 (MB 16, FR 1).  Back-to-back INT8 MFMAs from
//               registers run at 3.8-3.9 POPS with random operands in this
//               shape (the shader clock holds about 1.95 GHz) against 3.3-3.4
//               POPS in the 32 x 32 x 32 shape (about 1.65 GHz); a 16 x 16
//               block also gives a wave four times the independent
//               accumulators, which the matrix pipe needs to issue back to
//               back.  In this kernel it is 2-7% faster on the 256 x 256 and
//               256 x 192 tiles and equal on 256 x 128.
//   fp16, bf16: 32 x 32 x 16 (MB 32, FR 1)
//   FP8 E4M3:   32 x 32 x 64 (MB 32, FR 2)
typedef int v8i __attribute__((ext_vector_type(8)));
template <int OUT>
struct MmaKind {
  static constexpr int MB = 16, FR = 1;
  typedef v4i acc_t;
  __device__ static __forceinline__ acc_t mma(const v4i* a, const v4i* b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a[0], b[0], c, 0, 0, 0);
  }
};
template <>
struct MmaKind<3> {
  static constexpr int MB = 32, FR = 1;
  typedef v16f acc_t;
  __device__ static __forceinline__ acc_t mma(const v4i* a, const v4i* b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a[0]),
                                                  __builtin_bit_cast(v8h, b[0]), c, 0, 0, 0);
  }
};
template <>
struct MmaKind<4> {
  static constexpr int MB = 32, FR = 1;
  typedef v16f acc_t;
  __device__ static __forceinline__ acc_t mma(const v4i* a, const v4i* b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a[0]),
                                                   __builtin_bit_cast(v8bf, b[0]), c, 0, 0, 0);
  }
};
struct MmaE4m3 {
  static constexpr int MB = 32, FR = 2;
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

// The hardware conversion (v_cvt_pk_bf16_f32 on this target, two values per
// instruction) rounds to nearest even and keeps fp32 subnormals, as the
// kernels' fp32 denormal mode does.
__device__ __forceinline__ unsigned short f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(unsigned short, (__bf16)f);
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

// Scheduling hint for the compiler, for one k step of the tiled kernel (see
// kstep there): the step's first MFMA, then the NQ double-buffered fragment
// reads of the next step; then column P of NP finishes its NQ MFMAs and reads
// its in-place fragment (FR chunks) for the next step, with a share of the
// NVM global (LDS-mode) loads, so that no wave stalls on a memory queue
// while its matrix pipe idles.
// EARLY: the step before a stage barrier, where the next step's fragment of
// the last column is read with the first MFMA too (into a register set of its
// own) rather than after that column's MFMAs.
template <int P, int NP, int NQ, int FR, int NVM, bool EARLY = false>
__device__ __forceinline__ void interleave_cols() {
  constexpr int VPC = (NVM + NP - 1) / NP;  // VMEMs per column
  constexpr int EC = EARLY ? kEarlyCols : 0;
  if constexpr (P == 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, FR * NQ + EC * FR, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, NQ - 1, 0);
  } else {
    __builtin_amdgcn_sched_group_barrier(0x008, NQ, 0);
  }
  if constexpr (P < NP - EC) __builtin_amdgcn_sched_group_barrier(0x100, FR, 0);
  if constexpr (P * VPC < NVM)
    __builtin_amdgcn_sched_group_barrier(0x010, NVM - P * VPC < VPC ? NVM - P * VPC : VPC, 0);
  if constexpr (P + 1 < NP) interleave_cols<P + 1, NP, NQ, FR, NVM, EARLY>();
}


// The tiled kernels' LDS, sized for the largest tile's stages (every tiled
// kernel but the 128 x 32 one runs one block per CU).  It is one file-scope array rather than a
// pointer handed to the tile code: with a pointer the compiler can no longer
// tell the LDS-mode loads of later stages from the fragment reads of the
// current one and waits for every outstanding load before the first reads
// (measured 12% slower on the 256 x 192 tile).
constexpr int kTileLds = 2 * 256 * 128 + 3 * 256 * 128;  // 160 KiB, the whole LDS
__shared__ __attribute__((aligned(1024))) int8_t lds[kTileLds];
// The narrow 128 x 32 tile's own, smaller LDS, so that two of its blocks fit
// a CU (with its registers held to two waves per SIMD).  Selected at compile
// time from one of two file-scope arrays, so the compiler still sees which
// array every access uses.
constexpr int kSmallLds = 80 * 1024;
__shared__ __attribute__((aligned(1024))) int8_t lds_small[kSmallLds];
template <bool SMALL>
__device__ __forceinline__ int8_t* tile_lds() {
  if constexpr (SMALL) return lds_small;
  else return lds;
}

// One output tile (token tile tm, channel tile tn) of the tiled GEMM.  OUT as
// in MmaKind.  The block has WGM x WGN waves; K (in bytes per row) advances
// BK bytes per stage through NST LDS slots.  N is the number of channels this
// call covers (qb, sb and out start at its first one) and ldc the row stride
// of out in elements.
template <int BM, int BN, int BK, int NST, int WGM, int WGN, int OUT, bool DEEP = false>
__device__ __forceinline__ void gemm_tile(const int8_t* __restrict__ qa,
                                          const int8_t* __restrict__ qb, int M, int N, int K,
                                          const float* __restrict__ sa,
                                          const float* __restrict__ sb, void* __restrict__ out,
                                          int ldc, int tm, int tn) {
  constexpr int NW = WGM * WGN;                 // waves per block
  constexpr int WM = BM / WGM, WN = BN / WGN;   // wave tile (tokens, channels)
  constexpr int MB = MmaKind<OUT>::MB;          // rows of an MFMA block
  constexpr int LPR = 64 / MB;                  // lane groups (k chunks) per fragment row
  constexpr int FM = WM / MB, FN = WN / MB;
  constexpr int CPR = BK / 16;                  // 16-byte chunks per LDS row
  constexpr int RPW = 16 / CPR;                 // rows per 256-byte bank window
  constexpr int RPI = 1024 / BK;                // rows filled by one LDS-mode wave load
  constexpr int FR = MmaKind<OUT>::FR;          // 16-byte chunks per fragment
  constexpr int KK = BK / (16 * FR * LPR);      // MFMA k steps per stage
  constexpr int LA = BM / RPI / NW;             // LDS-mode loads per wave per stage, activations
  constexpr int LB = BN / RPI / NW;             // ... weights
  constexpr int L = LA + LB;
  constexpr int SLOT = (BM + BN) * BK;          // bytes per LDS stage
  // Two-slot tiles with 8 waves may keep three weight slots: the weight
  // stage then goes out two stages ahead instead of one.
  constexpr bool kHalfT = NST == 2 && WGM * WGN == 8;
  constexpr int NSA = NST;
  constexpr int NSB =
      (DEEP && kHalfT && BN == 256 && (NST * BM + (NST + 1) * BN) * BK <= kTileLds) ? NST + 1 : NST;
  // With as many weight as activation slots, stage s holds its activation
  // and weight rows side by side in one (BM + BN) x BK slot; otherwise the
  // activation slots come first, then the weight slots.
  constexpr bool kSym = NSA == NSB;
  static_assert(LA >= 1 && LB >= 1 && LA * RPI * NW == BM && LB * RPI * NW == BN &&
                FM >= 1 && FN >= 1 && FM * MB == WM && FN * MB == WN && KK % 2 == 0 &&
                (MB / RPW) % CPR == 0, "unsupported tile");
  static_assert(NST >= 2 && (NST - 1) * 2 * L < 64, "unsupported pipeline depth");  // vmcnt range
  static_assert(NSA * BM * BK + NSB * BN * BK <= (BN == 32 ? kSmallLds : kTileLds), "LDS size");

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
  // swizzle.  That row offset goes into the vector offset, the one the
  // hardware compares with the resource's size (the scalar offset, which
  // carries k0, is not range checked), so a row past the tile's last valid
  // one reads zero and touches no memory.  Loads j0 <= j < j1 are issued.
  // A stage past the end (st >= nk) is issued with out-of-range offsets: it
  // moves no data, keeps every wave's per-stage load count constant (so
  // fixed vmcnt values serve every iteration) and only touches the slot that
  // the stage would have used, which no live stage occupies.
  auto slot_a = [&](int st) -> int8_t* {
    int8_t* const base = tile_lds<BN == 32>();
    return kSym ? base + (st % NST) * SLOT : base + (st % NSA) * BM * BK;
  };
  auto slot_b = [&](int st) -> int8_t* {
    int8_t* const base = tile_lds<BN == 32>();
    return kSym ? base + (st % NST) * SLOT + BM * BK : base + NSA * BM * BK + (st % NSB) * BN * BK;
  };
  auto dma = [&](int st, int j0, int j1) {
    const int k0 = st * BK;
    int8_t* sa_ = slot_a(st);
    int8_t* sb_ = slot_b(st);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ro = h * (NW / 2) * RPI * K;
      const int w = wave + h * (NW / 2);
#pragma unroll
      for (int i = 0; i < LA; ++i) {
        if (h * L + i < j0 || h * L + i >= j1) continue;
        const int vo = (k0 + kc_a[i] >= K) ? kOob : voff_a[i] + ro;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (lds_void_t*)(sa_ + (i * NW + w) * 1024), 16, vo, k0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < LB; ++i) {
        if (h * L + LA + i < j0 || h * L + LA + i >= j1) continue;
        const int vo = (k0 + kc_b[i] >= K) ? kOob : voff_b[i] + ro;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (lds_void_t*)(sb_ + (i * NW + w) * 1024), 16, vo, k0, 0, 0);
      }
    }
  };
  // The two-slot tiles' loads (issued by waves 0 .. NW/2 - 1 for themselves
  // and for wave + NW/2): all activation loads of stage sta, then all weight
  // loads of stage stb (a negative stage: none).
  auto dma2 = [&](int sta, int stb) {
#pragma unroll
    for (int op = 0; op < 2; ++op) {
      const int st = op == 0 ? sta : stb;
      if (st < 0) continue;
      const int k0 = st * BK;
      int8_t* slot = op == 0 ? slot_a(st) : slot_b(st);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ro = h * (NW / 2) * RPI * K;
        const int w = wave + h * (NW / 2);
        if (op == 0) {
#pragma unroll
          for (int i = 0; i < LA; ++i) {
            const int vo = (k0 + kc_a[i] >= K) ? kOob : voff_a[i] + ro;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (lds_void_t*)(slot + (i * NW + w) * 1024), 16, vo, k0, 0, 0);
          }
        } else {
#pragma unroll
          for (int i = 0; i < LB; ++i) {
            const int vo = (k0 + kc_b[i] >= K) ? kOob : voff_b[i] + ro;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (lds_void_t*)(slot + (i * NW + w) * 1024), 16, vo, k0, 0, 0);
          }
        }
      }
    }
  };

  // fragment reads: lane reads row (base + lane % MB), k chunks
  // FR * (LPR * kk + lane / MB) + f; bases are multiples of MB rows, a whole
  // number of swizzle periods, so the swizzle depends on lane % MB only
  const int fr = lane % MB, fk = lane / MB;
  const int fsw = (fr / RPW) % CPR;
  const int off_a = (wm * WM + fr) * BK;
  const int off_b = (wn * WN + fr) * BK;

  typedef typename MmaKind<OUT>::acc_t acc_t;
  acc_t acc[FN][FM];
#pragma unroll
  for (int a = 0; a < FN; ++a)
#pragma unroll
    for (int b = 0; b < FM; ++b) acc[a][b] = acc_t{};

  // Fragments.  Fragment f of a lane is chunk FR * (LPR * kk + fk) + f of its
  // row (f < FR).  Of the two operands, the one with more fragments per wave
  // (P, NP of them) is read in place: fragment p of the next k step goes into
  // the registers of fragment p as soon as the MFMAs of column p have been
  // issued.  The other (Q, NQ <= NP) is double-buffered, and all of its
  // fragments of the next step are read with the step's first MFMA, since
  // the next step's first column needs every one of them (measured 3-5%
  // faster on the 256 x 128 tile than reading fragment q after column q).
  // So a wave holds NP + 2 NQ fragments instead of 2 (NP + NQ).
  constexpr bool kAin = FM >= FN;  // the activation fragments are read in place
  constexpr int NP = kAin ? FM : FN, NQ = kAin ? FN : FM;
  constexpr int EC = kEarlyCols < NP ? kEarlyCols : NP;
  v4i fp[NP * FR], fq0[NQ * FR], fq1[NQ * FR], fx[EC * FR];
  auto read_frag = [&](int st, int kk, bool act, int i, v4i* dst) {
    const int8_t* slot = act ? slot_a(st) : slot_b(st);
    const int base = act ? off_a + i * MB * BK : off_b + i * MB * BK;
#pragma unroll
    for (int f = 0; f < FR; ++f)
      dst[f] = *(const v4i*)(slot + base + (((FR * (LPR * kk + fk) + f) ^ fsw) << 4));
  };
  auto read_all = [&](int st, int kk, v4i* fq) {
#pragma unroll
    for (int p = 0; p < NP; ++p) read_frag(st, kk, kAin, p, fp + p * FR);
#pragma unroll
    for (int q = 0; q < NQ; ++q) read_frag(st, kk, !kAin, q, fq + q * FR);
  };

  // One k step: the reads of the Q fragments of step rkk of stage rst go
  // out with the first MFMA; then column p issues its NQ MFMAs and (when
  // `rd`) reads its P fragment of step rkk in place.  In the step before a
  // stage barrier (early) the last column's next fragment is read at the
  // start as well, into fx, so that the reads a wave must wait for at the
  // barrier were issued a column of MFMAs earlier; the step after the barrier
  // (use_fx) takes that column's operand from fx.
  auto kstep = [&](const v4i* cq, v4i* nq, bool rd, int rst, int rkk, auto early_tag,
                   auto use_fx_tag) {
    constexpr bool kEarly = decltype(early_tag)::value;
    constexpr bool kUseFx = decltype(use_fx_tag)::value;
    if (rd) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) read_frag(rst, rkk, !kAin, q, nq + q * FR);
      if constexpr (kEarly) {
#pragma unroll
        for (int e = 0; e < EC; ++e) read_frag(rst, rkk, kAin, NP - EC + e, fx + e * FR);
      }
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const v4i* cp = (kUseFx && p >= NP - EC) ? fx + (p - (NP - EC)) * FR : fp + p * FR;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if constexpr (kAin)
          acc[q][p] = MmaKind<OUT>::mma(cq + q * FR, cp, acc[q][p]);
        else
          acc[p][q] = MmaKind<OUT>::mma(cp, cq + q * FR, acc[p][q]);
      }
      if (rd && !(kEarly && p >= NP - EC)) read_frag(rst, rkk, kAin, p, fp + p * FR);
    }
  };
  const std::false_type kNo{};
  const std::true_type kYes{};

  // Pipeline (stage s lives in slot s % NST).  Iteration kt computes stage kt
  // as KK k steps (64 bytes deep for INT8 and FP8, 32 for fp16 / bf16); the
  // fragments of step kk+1 are read while the MFMAs of step kk run.  Before the last step the stage
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
  //    own and those of wave + 4, while waves 4..7 only compute.  The
  //    256 x 256 tile of the single-shape kernel keeps a third weight slot
  //    (the whole 160 KiB of LDS): its weight loads go out two stages ahead
  //    (measured 4-11% faster on the OPT-30B and Llama-2-70B layers, equal
  //    on the others; slower inside the two-shape grid and on 256 x 192).
  //  - NST == 2 with 4 waves: each wave issues its own after the barrier.
  constexpr bool kSpread = NST >= 3;
  constexpr bool kHalf = !kSpread && NW == 8;
  constexpr int LW = kHalf ? 2 * L : L;              // loads per stage of a loading wave
  constexpr int PER = (LW + KK - 2) / (KK - 1);      // loads per step when spread
  static_assert(KK >= 2, "unsupported stage depth");
  static_assert(!kHalf || ((NW / 2) * RPI / RPW) % CPR == 0, "half-wave load swizzle");
  // The K loop, in one copy for waves that issue loads and one for waves that
  // only compute: with a run-time branch on the role inside the loop, the
  // accumulators would meet at every join, where the register allocator
  // copies them.
  // Two-slot tiles with a third weight slot (NSB = 3): the prologue issues
  // activations 0, weights 0, weights 1, activations 1, weights 2, and the
  // barrier of iteration kt activations kt+2 and weights kt+3, so at each
  // barrier only the weights of the next-but-one stage may still be in flight.
  constexpr int LAW = 2 * LA, LBW = 2 * LB;  // a loading wave's loads per stage and operand
  static_assert(kSpread || kHalf, "pipeline");
  constexpr int kWaitBarrier = kSpread ? (NST - 2) * LW : (NSB == 3 ? LBW : 0);
  constexpr int kWaitFirst = kSpread ? (NST - 2) * LW : (NSB == 3 ? 2 * LBW + LAW : LW);
  auto kloop = [&](auto loads_tag) {
    constexpr bool kLoads = decltype(loads_tag)::value;
    // prologue: the stages in flight before iteration 0
    if constexpr (kLoads) {
      if constexpr (kSpread) {
#pragma unroll
        for (int st = 0; st < NST - 1; ++st) dma(st, 0, LW);
      } else if constexpr (NSB == 3) {
        dma2(0, 0);
        dma2(-1, 1);
        dma2(1, 2);
      } else {
        dma(0, 0, LW);
        dma(1, 0, LW);
      }
    }
    wait_vmcnt<kWaitFirst>();  // stage 0 landed
    block_barrier();
    read_all(0, 0, fq0);
    for (int kt = 0; kt < nk - 1; ++kt) {
      // the steps before the barrier step: all but the last one plain
      auto pre = [&](auto kk_tag) {
        constexpr int kk = decltype(kk_tag)::value;
        v4i* cq = (kk & 1) ? fq1 : fq0;
        v4i* nq = (kk & 1) ? fq0 : fq1;
        constexpr bool kE = kk == KK - 2;
        if constexpr (kSpread) {
          dma(kt + NST - 1, kk * PER, min((kk + 1) * PER, LW));
          kstep(cq, nq, true, kt, kk + 1, std::integral_constant<bool, kE>{}, kNo);
          interleave_cols<0, NP, NQ, FR, PER, kE>();
        } else {
          kstep(cq, nq, true, kt, kk + 1, std::integral_constant<bool, kE>{}, kNo);
          interleave_cols<0, NP, NQ, FR, 0, kE>();
        }
      };
      pre(std::integral_constant<int, 0>{});
      if constexpr (KK > 2) pre(std::integral_constant<int, 1>{});
      if constexpr (KK > 3) pre(std::integral_constant<int, 2>{});
      static_assert(KK <= 4, "k steps per stage");
      {
        constexpr int kk = KK - 1;
        v4i* cq = (kk & 1) ? fq1 : fq0;
        v4i* nq = (kk & 1) ? fq0 : fq1;
        // the previous step's MFMAs stay ahead of the waits
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<kWaitBarrier>();  // this wave's loads of stage kt+1 landed
        wait_lgkmcnt0();             // this wave's reads of slot kt are done
        block_barrier();             // every wave: stage kt+1 landed, slot kt free
        if constexpr (!kSpread && kLoads) {
          if constexpr (NSB == 3)
            dma2(kt + 2, kt + 3);
          else
            dma(kt + 2, 0, LW);
          kstep(cq, nq, true, kt + 1, 0, kNo, kYes);
          interleave_cols<0, NP, NQ, FR, LW>();
        } else {
          kstep(cq, nq, true, kt + 1, 0, kNo, kYes);
          interleave_cols<0, NP, NQ, FR, 0>();
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      v4i* cq = (kk & 1) ? fq1 : fq0;
      v4i* nq = (kk & 1) ? fq0 : fq1;
      kstep(cq, nq, kk + 1 < KK, nk - 1, kk + 1, kNo, kNo);
    }
    wait_vmcnt<0>();  // no LDS-mode load may outlive the block's LDS
  };
  if (nk > 0) {
    if constexpr (kHalf) {
      if (wave < NW / 2)
        kloop(std::true_type{});
      else
        kloop(std::false_type{});
    } else {
      kloop(std::true_type{});
    }
  }

  // Epilogue.  A lane holds, for register group g of fragment (a, b), output
  // channels n .. n+3 of token m, with m = b * MB + lane % MB and
  // n = a * MB + g * 4 * LPR + (lane / MB) * 4 inside the wave tile.  Stored
  // like that, a wave store would cover MB rows with 64 / MB * 16 bytes each,
  // and the store path, which pays per request, would run below its byte
  // rate.  So the results go through LDS, one MB-token slab of the wave tile
  // at a time: each wave writes its slab into a private staging area and
  // reads it back row-major, 16 contiguous bytes per lane, for full-line
  // global stores.  The staging row pitch is an odd number of 16-byte chunks,
  // so the rows of a slab write fall on distinct bank groups.
  //
  // The dequant scales are loaded before any store: the memory counter that
  // their loads are waited on also counts stores, so a scale load issued after
  // a store would make its use wait for that store to complete.  Indices are
  // clamped so the loads stay in bounds; stores are guarded (N % 8 == 0, so a
  // 16-byte chunk of a row is either inside N or wholly outside).
  constexpr int NG = sizeof(acc_t) / 16;  // groups of 4 accumulators per lane
  constexpr int ES = OUT == 0 ? 4 : 2;    // output element bytes
  constexpr int CPO = WN * ES / 16;       // 16-byte output chunks per wave-tile row
  constexpr int PITCH = WN * ES + 16;     // staging row pitch in bytes
  static_assert((PITCH / 16) % 2 == 1 && NW * MB * PITCH <= NST * SLOT && (MB * CPO) % 64 == 0 &&
                NG * 4 * LPR == MB, "epilogue staging");
  const int hi = lane / MB;
  constexpr bool kDequant = OUT == 1 || OUT == 2 || OUT == 5 || OUT == 6;
  float am[FM];
  float4 bn[FN][NG];
  if constexpr (kDequant) {
#pragma unroll
    for (int b = 0; b < FM; ++b) am[b] = sa[min(m0 + wm * WM + b * MB + fr, M - 1)];
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
      for (int g = 0; g < NG; ++g)
        bn[a][g] = *(const float4*)(sb + min(n0 + wn * WN + a * MB + g * 4 * LPR + hi * 4, N - 4));
  }
  // every wave is past its last fragment read and its last LDS-mode load
  wait_lgkmcnt0();
  block_barrier();
  int8_t* stage = tile_lds<BN == 32>() + wave * MB * PITCH;
#pragma unroll
  for (int b = 0; b < FM; ++b) {
#pragma unroll
    for (int a = 0; a < FN; ++a) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const acc_t& C = acc[a][b];
        int8_t* dst = stage + fr * PITCH + (a * MB + g * 4 * LPR + hi * 4) * ES;
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
    constexpr int NR = MB * CPO / 64;
    v4i v[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int f = i * 64 + lane;
      v[i] = *(const v4i*)(stage + (f / CPO) * PITCH + (f % CPO) * 16);
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int f = i * 64 + lane;
      const int m = m0 + wm * WM + b * MB + f / CPO;
      const int n = n0 + wn * WN + (f % CPO) * (16 / ES);
      if (m < M && n < N) *(v4i*)((int8_t*)out + ((int64_t)m * ldc + n) * ES) = v[i];
    }
  }
}

template <int BM, int BN, int BK, int NST, int WGM, int WGN, int OUT>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WGM * WGN, 64 * WGM * WGN),
                          amdgpu_waves_per_eu(BN == 32 ? 2 : WGM * WGN / 4,
                                              BN == 32 ? 2 : WGM * WGN / 4))) void
k_gemm_i8(const int8_t* __restrict__ qa, const int8_t* __restrict__ qb, int M, int N, int K,
          const float* __restrict__ sa, const float* __restrict__ sb, void* __restrict__ out,
          int m_tiles, int n_tiles) {
  int tm, tn;
  tile_of(blockIdx.x, m_tiles, n_tiles, tm, tn);
  gemm_tile<BM, BN, BK, NST, WGM, WGN, OUT, kDeepB>(qa, qb, M, N, K, sa, sb, out, N, tm, tn);
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

// Few-token GEMM (3 to 128 tokens): the product is weight streaming, and the
// weight streams fastest in whole cache lines per load instruction, which
// the matrix-core operand layout (16 rows x 64 bytes per instruction) does
// not give.  So each wave loads its weight rows in 256-byte pieces, four
// 1 KiB instructions per 16 rows (lane l: row 4 i + l / 16, bytes 16 (l % 16)
// of the piece, non-temporal), writes them to an LDS area of its own and
// reads them back as the four 64-deep MFMA fragments of the piece (lane:
// row l % 16, chunk 4 s + l / 16; chunk c of row r sits at slot c ^ r, so
// both the writes and the reads are free of bank conflicts).  No barrier is
// involved: a wave's LDS operations complete in order.
//
// A block owns 16 CG output channels over all of K; its NW waves take
// contiguous ranges of the pieces.  Each wave holds CG weight groups, which
// share the activation fragments (MT token slots of 16, read from L2; rows
// past M are outside their buffer resource and read as zero).  Chunks past K
// in a row's last piece are issued with out-of-range offsets.  The waves' int32
// partial sums add exactly through LDS and the dequant epilogue follows, as
// in the tiled kernel (a lane holds channels n .. n+3 of one token).
// The dequant epilogue of one lane's four channels n .. n+3 of token m (or
// their int32 sums for OUT == 0), with the token's scale am and the
// channels' scales bn.
template <int OUT>
__device__ __forceinline__ void fewtok_store(const v4i& cs, int m, int n, int N, float am,
                                             float4 bn, void* __restrict__ out) {
  if (OUT == 0) {
    *(v4i*)((int32_t*)out + (int64_t)m * N + n) = cs;
  } else {
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

// SPLIT: the block covers the pieces [np y / S, np (y + 1) / S) of split
// y = blockIdx.y of S = gridDim.y, and the S blocks of one channel group meet
// in memory.  Each stores its exact int32 partial slice (part[y][m][n]) with
// the device-scope cache policy (sc1: the form the compiler gives
// agent-scope atomic stores and loads on this target, coherent across the
// XCDs' L2s), waits until the stores have completed, and counts itself on
// the group's counter (zero on entry, a device-scope atomic).  The block that
// brings the count to S adds the other slices, read with the same policy, to
// its own sum held in registers and applies the epilogue.  No block waits
// for another.
template <int MT, int NW, int CG, int OUT, bool SPLIT>
__global__ __launch_bounds__(64 * NW) void k_gemm_fewtok(
    const int8_t* __restrict__ qa, const int8_t* __restrict__ qb, int M, int N, int K,
    const float* __restrict__ sa, const float* __restrict__ sb, void* __restrict__ out,
    int32_t* __restrict__ part, unsigned* __restrict__ counters) {
  constexpr int kNt = 2;     // cache policy: non-temporal
  constexpr int kDev = 16;   // cache policy: device scope (sc1)
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 16 * CG;
  const rsrc_t rw = make_rsrc(qb + (int64_t)n0 * K, (unsigned)min(16 * CG, N - n0) * (unsigned)K);
  const rsrc_t rx = make_rsrc(qa, (unsigned)M * (unsigned)K);
  // a wave's 16 rows x 16 chunks per group during the K loop; the waves'
  // partial sums afterwards, in the same LDS
  constexpr int kWl = NW * CG * 256, kRed = NW * CG * MT * 64;
  __shared__ v4i lbuf[kWl > kRed ? kWl : kRed];
  v4i(*wl)[CG][256] = (v4i(*)[CG][256])lbuf;
  v4i(*red)[CG * MT][64] = (v4i(*)[CG * MT][64])lbuf;
  const int np = (K + 255) / 256;  // 256-byte pieces per row
  const int S = SPLIT ? (int)gridDim.y : 1, sp = SPLIT ? (int)blockIdx.y : 0;
  const int q0 = (int)((int64_t)np * sp / S), q1 = (int)((int64_t)np * (sp + 1) / S);
  const int per = (q1 - q0 + NW - 1) / NW;
  const int p0 = q0 + wave * per, p1 = min(q1, p0 + per);
  const int lr = lane >> 4, lc = lane & 15;   // load: row within 4, 16-byte chunk
  const int r16 = lane & 15, kq = lane >> 4;  // fragment: row, chunk within the k step

  v4i acc[CG][MT];
#pragma unroll
  for (int c = 0; c < CG; ++c)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[c][t] = v4i{0, 0, 0, 0};
  // One piece: loads, transpose through the wave's LDS area, MFMAs.  Only a
  // row's last piece can pass K (K % 256 != 0); it takes the checked form,
  // whose chunks past K load zero, and the others skip the checks (5-16%
  // faster at 33 to 64 tokens).
  auto piece = [&](int p, auto checked) {
    constexpr bool kChecked = decltype(checked)::value;
    const int kb = p * 256;
    v4i w[CG][4];
#pragma unroll
    for (int c = 0; c < CG; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = c * 16 + 4 * i + lr;
        const int col = kb + 16 * lc;
        const int off = !kChecked || col < K ? row * K + col : kOob;
        w[c][i] = __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, kNt);
      }
    v4i x[4][MT];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int col = kb + 64 * s + 16 * kq;
        const int off = !kChecked || col < K ? (t * 16 + r16) * K + col : kOob;
        x[s][t] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
      }
#pragma unroll
    for (int c = 0; c < CG; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * i + lr;
        wl[wave][c][row * 16 + (lc ^ row)] = w[c][i];
      }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int c = 0; c < CG; ++c) {
        const v4i a = wl[wave][c][r16 * 16 + ((4 * s + kq) ^ r16)];
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[c][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, x[s][t], acc[c][t], 0, 0, 0);
      }
  };
  const int p_full = min(p1, K / 256);  // pieces wholly inside K
  for (int p = p0; p < p_full; ++p) piece(p, std::false_type{});
  for (int p = max(p0, p_full); p < p1; ++p) piece(p, std::true_type{});

  // exact sum of the waves' partials; fragment f is finished by wave f % NW
  __syncthreads();  // every wave is done with its pieces in LDS
#pragma unroll
  for (int c = 0; c < CG; ++c)
#pragma unroll
    for (int t = 0; t < MT; ++t) red[wave][c * MT + t][lane] = acc[c][t];
  __syncthreads();
  constexpr int FW = (CG * MT + NW - 1) / NW;  // fragments finished per wave
  v4i own[FW];
  float am[FW];
  float4 bn[FW];
  // the slices: S x M x N int32 (the launcher keeps this under 2^31 bytes)
  const rsrc_t rp = make_rsrc((const int8_t*)part, SPLIT ? (unsigned)S * (unsigned)M * (unsigned)N * 4u : 0u);
#pragma unroll
  for (int j = 0; j < FW; ++j) {
    const int f = wave + j * NW;
    if (f >= CG * MT) break;
    v4i cs = red[0][f][lane];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) cs += red[w2][f][lane];
    own[j] = cs;
    // lane holds channels n .. n+3 of token m
    const int m = (f % MT) * 16 + (lane & 15);
    const int n = n0 + (f / MT) * 16 + 4 * (lane >> 4);
    if (m >= M || n >= N) continue;
    // the scales now, so that the last block of a split does not wait for them
    if (OUT != 0) {
      am[j] = sa[m];
      bn[j] = *(const float4*)(sb + n);
    }
    if (!SPLIT)
      fewtok_store<OUT>(cs, m, n, N, am[j], bn[j], out);
    else
      __builtin_amdgcn_raw_buffer_store_b128(cs, rp, (unsigned)(((sp * M + m) * N + n) * 4), 0, kDev);
  }
  if constexpr (SPLIT) {
    __shared__ unsigned last;
    // this thread's slice stores have completed before the block is counted
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) last = atomicAdd(counters + blockIdx.x, 1u) == (unsigned)S - 1 ? 1u : 0u;
    __syncthreads();
    if (!last) return;
#pragma unroll
    for (int j = 0; j < FW; ++j) {
      const int f = wave + j * NW;
      if (f >= CG * MT) break;
      const int m = (f % MT) * 16 + (lane & 15);
      const int n = n0 + (f / MT) * 16 + 4 * (lane >> 4);
      if (m >= M || n >= N) continue;
      v4i c = own[j];
      for (int s2 = 0; s2 < S; ++s2) {
        if (s2 == sp) continue;
        c += __builtin_amdgcn_raw_buffer_load_b128(rp, (unsigned)(((s2 * M + m) * N + n) * 4), 0, kDev);
      }
      fewtok_store<OUT>(c, m, n, N, am[j], bn[j], out);
    }
  }
}

template <int MT, int NW, int CG, bool SPLIT>
void launch_fewtok_cfg(const int8_t* qa, const int8_t* qb, int M, int N, int K, const float* sa,
                       const float* sb, void* out, int mode, int splits, int32_t* part,
                       unsigned* counters, hipStream_t st) {
  const dim3 grid((unsigned)((N + 16 * CG - 1) / (16 * CG)), (unsigned)splits), block(64 * NW);
  if (mode == 0)
    hipLaunchKernelGGL((k_gemm_fewtok<MT, NW, CG, 0, SPLIT>), grid, block, 0, st, qa, qb, M, N, K, sa, sb,
                       out, part, counters);
  else if (mode == 1)
    hipLaunchKernelGGL((k_gemm_fewtok<MT, NW, CG, 1, SPLIT>), grid, block, 0, st, qa, qb, M, N, K, sa, sb,
                       out, part, counters);
  else
    hipLaunchKernelGGL((k_gemm_fewtok<MT, NW, CG, 2, SPLIT>), grid, block, 0, st, qa, qb, M, N, K, sa, sb,
                       out, part, counters);
}

// Shape choice, measured on the OPT-6.7B decode layers at 1-32 tokens: with
// 12288 or more channels each wave takes several channel groups, which
// share the activation fragments (up to 16 tokens two groups and four waves
// splitting K; from 17 tokens, where the activations are two fragments per
// step, four groups and eight waves); with fewer channels one group per wave
// and eight waves per block, so that enough waves stream.  From 33 tokens
// (measured at 48-128 tokens on 4096 to 22016 channels) four waves per block
// were fastest at every width, with one, two or four groups.
template <int MT>
hipError_t launch_fewtok(const int8_t* qa, const int8_t* qb, int64_t M, int64_t N, int64_t K,
                         const float* sa, const float* sb, void* out, int mode, hipStream_t st) {
  const int m = (int)M, n = (int)N, k = (int)K;
  if constexpr (MT >= 4) {
    // 33 to 128 tokens: four waves per block, and as many channel groups as
    // keep the grid near 256 blocks
    if (N <= 4096)
      launch_fewtok_cfg<MT, 4, 1, false>(qa, qb, m, n, k, sa, sb, out, mode, 1, nullptr, nullptr, st);
    else if (N <= 8192)
      launch_fewtok_cfg<MT, 4, 2, false>(qa, qb, m, n, k, sa, sb, out, mode, 1, nullptr, nullptr, st);
    else
      launch_fewtok_cfg<MT, 4, 4, false>(qa, qb, m, n, k, sa, sb, out, mode, 1, nullptr, nullptr, st);
  } else if (N < 12288) {
    launch_fewtok_cfg<MT, 8, 1, false>(qa, qb, m, n, k, sa, sb, out, mode, 1, nullptr, nullptr, st);
  } else if constexpr (MT == 2) {
    launch_fewtok_cfg<MT, 8, 4, false>(qa, qb, m, n, k, sa, sb, out, mode, 1, nullptr, nullptr, st);
  } else {
    launch_fewtok_cfg<MT, 4, 2, false>(qa, qb, m, n, k, sa, sb, out, mode, 1, nullptr, nullptr, st);
  }
  return hipGetLastError();
}

// Weight-row streaming for one or two tokens.  Here the product is a few
// dot products per weight row, and what bounds it is how fast the weight
// streams from HBM; the matrix-core layout (16 rows x 64 bytes per load
// instruction) streams it slower than whole rows do.  A 256-thread block owns
// R consecutive output channels; thread t holds the 16-byte chunks t, t + 256,
// ... of each of its rows, so every block-wide load instruction reads 4 KiB
// of one row contiguously, with the non-temporal hint (the weight is read
// once).  JB chunks per row are in flight at a time (R * JB loads per
// thread), with the activation chunks of the same k range for the MT token
// slots (rows past M read as zero through their buffer resource).  Products
// accumulate exactly in int32 with v_dot4 (four int8 products per
// instruction); each wave reduces its MT * R partial sums by a butterfly
// (halving the live values at each exchange), the four waves' sums add
// through LDS, and the same dequant epilogue as the tiled kernel follows.
template <int MT, int R, int JB, int OUT>
__global__ __launch_bounds__(256) void k_gemv_rows(const int8_t* __restrict__ qa,
                                                   const int8_t* __restrict__ qb, int M, int N,
                                                   int K, const float* __restrict__ sa,
                                                   const float* __restrict__ sb,
                                                   void* __restrict__ out) {
  constexpr int V = MT * R;  // partial sums per thread, a power of two
  static_assert((V & (V - 1)) == 0 && V <= 64, "butterfly over a power of two");
  constexpr int kNt = 2;  // cache policy: non-temporal
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * R;
  const int nr = min(R, N - n0);
  const rsrc_t rw = make_rsrc(qb + (int64_t)n0 * K, (unsigned)nr * (unsigned)K);
  const rsrc_t rx = make_rsrc(qa, (unsigned)M * (unsigned)K);
  const int kc = K / 16;  // 16-byte chunks per row
  int acc[MT][R];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[t][r] = 0;
  for (int c0 = tid; c0 < kc; c0 += 256 * JB) {
    v4i w[R][JB], x[MT][JB];
#pragma unroll
    for (int j = 0; j < JB; ++j) {
      const int c = c0 + 256 * j;
      const bool in = c < kc;
#pragma unroll
      for (int r = 0; r < R; ++r)
        w[r][j] = __builtin_amdgcn_raw_buffer_load_b128(rw, in ? r * K + 16 * c : kOob, 0, kNt);
#pragma unroll
      for (int t = 0; t < MT; ++t)
        x[t][j] = __builtin_amdgcn_raw_buffer_load_b128(rx, in ? t * K + 16 * c : kOob, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < R; ++r) {
          int a = acc[t][r];
          a = __builtin_amdgcn_sdot4(w[r][j].x, x[t][j].x, a, false);
          a = __builtin_amdgcn_sdot4(w[r][j].y, x[t][j].y, a, false);
          a = __builtin_amdgcn_sdot4(w[r][j].z, x[t][j].z, a, false);
          a = __builtin_amdgcn_sdot4(w[r][j].w, x[t][j].w, a, false);
          acc[t][r] = a;
        }
  }
  // Butterfly: at the exchange over lane distance d, a lane keeps the upper
  // half of its live values when bit d of its lane index is set, sends the
  // other half to its partner and adds what the partner sends back.  After
  // log2(V) exchanges one value is live, the sum over those lanes of value
  // idx; the remaining exchanges add it over the low lane bits.
  int v[V];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int r = 0; r < R; ++r) v[t * R + r] = acc[t][r];
  int idx = 0;
#pragma unroll
  for (int s = 0; (V >> s) > 1; ++s) {
    const int d = 32 >> s, h = V >> (s + 1);
    const bool up = (lane & d) != 0;
#pragma unroll
    for (int i = 0; i < h; ++i) {
      const int send = up ? v[i] : v[i + h];
      const int keep = up ? v[i + h] : v[i];
      v[i] = keep + __shfl_xor(send, d, 64);
    }
    if (up) idx += h;
  }
  constexpr int kLow = 64 / V;  // lanes that share one value index
#pragma unroll
  for (int d = kLow / 2; d >= 1; d >>= 1) v[0] += __shfl_xor(v[0], d, 64);
  __shared__ int red[4][V];
  if ((lane & (kLow - 1)) == 0) red[wave][idx] = v[0];
  __syncthreads();
  if (tid >= V) return;
  const int t = tid / R, r = tid % R;
  const int m = t, n = n0 + r;
  if (m >= M || r >= nr) return;
  const int c = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
  if (OUT == 0) {
    ((int32_t*)out)[(int64_t)m * N + n] = c;
  } else {
    float y = (float)c;
    y = y * sa[m];
    y = y * sb[n];
    // Keep the fp32 product as a value of its own: a lone product followed
    // by a narrowing conversion may otherwise be compiled into one
    // mixed-precision FMA that rounds the exact product to 16 bits once,
    // where the epilogue rounds it to fp32 first.
    asm volatile("" : "+v"(y));
    ((unsigned short*)out)[(int64_t)m * N + n] = OUT == 1 ? f32_to_f16_rne(y) : f32_to_bf16_rne(y);
  }
}

template <int MT, int JB>
void launch_gemv_jb(const int8_t* qa, const int8_t* qb, int M, int N, int K, const float* sa,
                    const float* sb, void* out, int mode, hipStream_t st) {
  constexpr int R = kGemvRows;
  const dim3 grid((unsigned)((N + R - 1) / R)), block(256);
  if (mode == 0)
    hipLaunchKernelGGL((k_gemv_rows<MT, R, JB, 0>), grid, block, 0, st, qa, qb, M, N, K, sa, sb, out);
  else if (mode == 1)
    hipLaunchKernelGGL((k_gemv_rows<MT, R, JB, 1>), grid, block, 0, st, qa, qb, M, N, K, sa, sb, out);
  else
    hipLaunchKernelGGL((k_gemv_rows<MT, R, JB, 2>), grid, block, 0, st, qa, qb, M, N, K, sa, sb, out);
}

// JB: as many 4 KiB row segments in flight as a row has, up to four.
template <int MT>
hipError_t launch_gemv(const int8_t* qa, const int8_t* qb, int64_t M, int64_t N, int64_t K,
                       const float* sa, const float* sb, void* out, int mode, hipStream_t st) {
  const int64_t segs = (K / 16 + 255) / 256;
  if (segs <= 1)
    launch_gemv_jb<MT, 1>(qa, qb, (int)M, (int)N, (int)K, sa, sb, out, mode, st);
  else if (segs == 2)
    launch_gemv_jb<MT, 2>(qa, qb, (int)M, (int)N, (int)K, sa, sb, out, mode, st);
  else
    launch_gemv_jb<MT, 4>(qa, qb, (int)M, (int)N, (int)K, sa, sb, out, mode, st);
  return hipGetLastError();
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
  // The few-token kernels serve the INT8 modes only.
  const bool tiled_only = out_mode >= 3;
  if (out_mode == 3 || out_mode == 4) K *= 2;
  // Few tokens: weight streaming.  One or two tokens: whole weight rows
  // (measured 9-19% faster than a matrix-core form on the OPT-6.7B decode
  // layers; at four tokens two to three times slower).  3 to 32 tokens: the
  // weight pieces transposed through LDS (on the same layers 12-35% faster
  // than streaming matrix-core fragments straight from memory, and 8-22%
  // faster at 32 tokens than 64-channel blocks over one K range).
  if (!tiled_only && M <= kGemvMaxM) {
    if (M == 1) return launch_gemv<1>(qa, qb, M, N, K, sa, sb, out, out_mode, st);
    return launch_gemv<2>(qa, qb, M, N, K, sa, sb, out, out_mode, st);
  }
  if (!tiled_only && M <= 16) return launch_fewtok<1>(qa, qb, M, N, K, sa, sb, out, out_mode, st);
  if (!tiled_only && M <= 32) return launch_fewtok<2>(qa, qb, M, N, K, sa, sb, out, out_mode, st);
  // 33 to 128 tokens on layers of up to 12288 channels (up to 64 tokens) or
  // 8192 (up to 128): the same kernel with four or eight token fragments.
  // The tiled kernel gets only 32 to 64 blocks there (one or two token tiles);
  // measured 1.2-2.2 times faster at 48 to 128 tokens on 4096 x 4096,
  // 11008 -> 4096 and 8192 x 8192, and 1.3-1.5 times at 48 and 64 tokens on
  // 4096 -> 11008 / 12288.  From 22016 channels, and from 12288 above 64
  // tokens, the tiled kernel is faster.
  if (!tiled_only && M <= 64 && N <= 12288)
    return launch_fewtok<4>(qa, qb, M, N, K, sa, sb, out, out_mode, st);
  if (!tiled_only && M <= 128 && N <= 8192)
    return launch_fewtok<8>(qa, qb, M, N, K, sa, sb, out, out_mode, st);
  // 129 to 512 tokens on up to 4096 channels (INT8): 128 x 32 tiles, four
  // waves, four stages in flight in an LDS array of their own (80 KiB), two
  // blocks per CU, so that up to 512 blocks run at once where the other
  // tiles give 32 to 128.  Measured on 4096 x 4096 24 -> 11.3-12.5 us at
  // 129-256 tokens and 24-25 -> 18-21 us at 320-512; on 11008 -> 4096
  // 57 -> 27.5-31.3 us and 57-59 -> 50-56 us.
  if (out_mode <= 2 && M <= 512 && N <= 4096)
    return launch_tile<128, 32, 128, 4, 4, 1>(qa, qb, M, N, K, sa, sb, out, out_mode, st);
  // Pick the tile whose last wave of blocks over 256 CUs is fullest, weighted
  // by the tile's output rate per CU relative to 256 x 256 (eff).  INT8
  // (16 x 16 x 64 MFMAs), measured per wave of blocks at K = 4096 on
  // Llama-2-7B-shaped codes: 256 x 256 about 50 us, 256 x 192 44 us,
  // 256 x 128 37 us, so eff 1, 0.85 and 0.68.  The 16-bit and FP8 forms
  // (32 x 32 MFMAs) follow the operand bytes per MFMA, which fall with
  // BM * BN / (BM + BN).
  struct Cand { int bm, bn; double eff; };
  const bool i8 = out_mode <= 2;
  const Cand cands[] = {{256, 256, 1.0},
                        {256, 128, i8 ? 0.68 : 0.92},
                        {128, 128, i8 ? 0.6 : 0.8},
                        {256, 192, i8 ? 0.85 : 0.96}};
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
  // channels.  The estimate counts waves of blocks times the time of a wave
  // of each tile (in cycles per stage, 2339 for 256 x 256; INT8: 2063 for
  // 256 x 192 and 1715 for 256 x 128, from the wave times above; 16-bit and
  // FP8: 1853 and 1404, per-block timelines); the split is taken when it is 3%
  // or more below the single shape's.  Measured: gate_up 4096 -> 22016 at
  // 2048 tokens 155 -> 152 us, and the OPT-30B 7168-channel layers 2% faster.
  if (cands[best].bm == 256) {
    const int64_t mt = (M + 255) / 256;
    const int64_t cyc[4] = {2339, i8 ? 1715 : 1404, 0, i8 ? 2063 : 1853};
    const int64_t tiles = mt * ((N + cands[best].bn - 1) / cands[best].bn);
    // The single-shape 256 x 256 tile streams its weights two stages ahead;
    // on long rows that makes it about 11% faster than inside the two-shape
    // grid (OPT-30B fc2, K = 28672: 651 -> 616 us), while at K = 4096 and
    // 7168 the two-shape grid stays ahead (measured).
    const int64_t c_single = (best == 0 && K >= 16384) ? 2100 : cyc[best];
    const int64_t single = (tiles + 255) / 256 * c_single;
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
  SplitkPlan p{0, 0};
  if (M < 3 || M > 32 || N < 1 || N >= 12288 || K < 1) return p;
  // Below 12288 channels the unsplit few-token kernel gives each block one
  // 16-channel group, and every block reads the whole activation rows; under
  // 2048 channels it also gets fewer than 128 blocks.  The split form gives a
  // block four groups and 1/S of K, and pays a hand-over of partial sums
  // through memory, which long rows amortize.  Measured on the few-token
  // kernels alone and in the runtime forward:
  //   17-32 tokens, rows of 32 or more 256-byte pieces: 7-17% faster on
  //     16384 -> 4096, 11008 -> 4096 and 8192 -> 8192, up to 45% on
  //     16384 -> 1024; at 16 pieces (4096 -> 1024, 1536, 4096) slower;
  //   3-16 tokens, under 2048 channels with rows of 64 or more pieces:
  //     9-67% faster (16384 -> 1024, 65536 -> 264); at 32 pieces and on
  //     wider layers level or slower.
  // About one block per CU, at least 8 pieces per split (one per wave), at
  // most 16 splits.
  const int64_t np = (K + 255) / 256;
  if (M >= 17 ? np < 32 : (N >= 2048 || np < 64)) return p;
  const int64_t groups = (N + 16 * kSplitkCG - 1) / (16 * kSplitkCG);
  int64_t s = (256 + groups - 1) / groups;
  s = std::min<int64_t>(s, np / 8);
  s = std::min<int64_t>(s, 16);
  if (s < 2) return p;
  p.splits = (int)s;
  p.groups = (int)groups;
  return p;
}

hipError_t launch_gemm_splitk(const int8_t* qa, const int8_t* qb, int64_t M, int64_t N, int64_t K,
                              const float* sa, const float* sb, void* y, bool bf16,
                              int32_t* partials, unsigned* counters, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  const SplitkPlan p = splitk_plan(M, N, K);
  if (p.splits == 0) return hipErrorInvalidValue;
  const int m = (int)M, n = (int)N, k = (int)K, mode = bf16 ? 2 : 1;
  if (M <= 16)
    launch_fewtok_cfg<1, 8, kSplitkCG, true>(qa, qb, m, n, k, sa, sb, y, mode, p.splits, partials,
                                             counters, st);
  else
    launch_fewtok_cfg<2, 8, kSplitkCG, true>(qa, qb, m, n, k, sa, sb, y, mode, p.splits, partials,
                                             counters, st);
  return hipGetLastError();
}


}  // namespace w8a8
