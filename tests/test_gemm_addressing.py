"""Operand addressing of the GEMM kernels, checked on the CPU.

The kernels read their operands with raw buffer loads: the hardware compares
a load's vector offset (plus its immediate offset) with the buffer
resource's size and returns zero without touching memory when it is past
the end; the scalar offset is added to the address but not compared.  This
file models the offsets each kernel issues, lane by lane, and checks that
every load the hardware would not mask reads 16 bytes inside a valid row of
the operand: rows past M or N and chunks past K must be masked.  The model
restates the kernels' index arithmetic (w8a8_int8_amd/csrc/gemm.hip), so a
change there needs the same change here; the GPU parity tests cannot see an
out-of-bounds read whose data only feeds discarded outputs.
"""
from __future__ import annotations

import numpy as np
import pytest

K_OOB = 0x40000000


def tiled_loads(BM, BN, NST, WGM, WGN, M, N, K, tm, tn, row_offset_in_scalar=False):
    """(operand, row_base, vector offset, scalar offset, num_records) of every
    LDS-mode load one block of the tiled kernel issues (128-byte stages).
    row_offset_in_scalar models the mistaken form in which the loads issued
    for waves NW/2 .. NW-1 carry their row offset in the scalar offset."""
    BK = 128
    NW = WGM * WGN
    CPR, RPI = BK // 16, 1024 // BK
    RPW = 16 // CPR
    LA, LB = BM // RPI // NW, BN // RPI // NW
    spread = NST >= 3
    half = (not spread) and NW == 8
    nk = (K + BK - 1) // BK
    # every stage the pipeline issues: 0 .. nk - 1 plus the zero-filled ones past the end
    last = nk - 1 + (NST - 1 if spread else NST)
    out = []
    lane = np.arange(64)
    lrow, lslot = lane // CPR, lane % CPR
    for opnd, base, rows_tile, LX in (("a", tm * BM, BM, LA), ("b", tn * BN, BN, LB)):
        size = M if opnd == "a" else N
        recs = min(rows_tile, size - base) * K
        for wave in range(NW // 2 if half else NW):
            for h in range(2 if half else 1):
                for i in range(LX):
                    row = (i * NW + wave) * RPI + lrow
                    kc = (lslot ^ ((row // RPW) % CPR)) << 4
                    voff = row * K + kc
                    ro = h * (NW // 2) * RPI * K
                    for st in range(last + 1):
                        k0 = st * BK
                        if row_offset_in_scalar:
                            out.append((opnd, base, np.where(k0 + kc >= K, K_OOB, voff), k0 + ro, recs))
                        else:
                            out.append((opnd, base, np.where(k0 + kc >= K, K_OOB, voff + ro), k0, recs))
    return out


def assert_in_bounds(loads, M, N, K):
    for opnd, base, vo, so, recs in loads:
        size = M if opnd == "a" else N
        live = vo < recs  # what the hardware does not mask
        off = vo[live].astype(np.int64) + so
        row = base + off // K
        col = off % K
        assert (row < size).all() and (row >= 0).all(), (opnd, base)
        assert (col + 16 <= K).all() and (col % 16 == 0).all(), (opnd, base)


TILES = [  # BM, BN, NST, WGM, WGN: every tile the launcher can pick
    (256, 256, 2, 2, 4),
    (256, 192, 2, 4, 2),
    (256, 128, 3, 4, 2),
    (128, 128, 4, 2, 2),
    (128, 32, 4, 4, 1),
]


@pytest.mark.parametrize("tile", TILES, ids=lambda t: f"{t[0]}x{t[1]}")
@pytest.mark.parametrize("M,N,K", [(2000, 8192, 256), (37, 136, 1040), (300, 520, 272),
                                   (2048, 4104, 144), (2, 8, 16), (259, 200, 400)])
def test_tiled_kernel_loads_stay_in_bounds(tile, M, N, K):
    BM, BN, NST, WGM, WGN = tile
    mt, nt = -(-M // BM), -(-N // BN)
    # the last tile in each direction is where the rows run out
    for tm in sorted({0, mt - 1}):
        for tn in sorted({0, nt - 1}):
            assert_in_bounds(tiled_loads(BM, BN, NST, WGM, WGN, M, N, K, tm, tn), M, N, K)


def test_the_scalar_offset_is_not_a_row_offset():
    """The case that motivated this file: a 256 x 256 tile whose last token
    tile ends inside a 64-row group (M = 2000).  Loads issued for waves 4-7
    carry their 32-row offset in the vector offset.  The model with that
    offset moved into the (unchecked) scalar offset must fail, reading rows
    past M."""
    M, N, K = 2000, 8192, 256
    assert_in_bounds(tiled_loads(256, 256, 2, 2, 4, M, N, K, M // 256, 0), M, N, K)
    with pytest.raises(AssertionError):
        assert_in_bounds(tiled_loads(256, 256, 2, 2, 4, M, N, K, M // 256, 0,
                                     row_offset_in_scalar=True), M, N, K)


def fewtok_loads(M, N, K, n0, MT, NW, CG, S=1, sp=0):
    """Loads of one block of the 3-32 token kernel: 16 CG weight rows in
    256-byte pieces (wave w takes a contiguous range of the block's pieces:
    all of them, or those of split sp of S), and the activation fragments of
    the same k range for MT token slots."""
    lane = np.arange(64)
    lr, lc = lane // 16, lane % 16
    r16, kq = lane % 16, lane // 16
    npc = -(-K // 256)
    q0, q1 = npc * sp // S, npc * (sp + 1) // S
    per = -(-(q1 - q0) // NW)
    recs_w = min(16 * CG, N - n0) * K
    recs_x = M * K
    out = []
    for w in range(NW):
        for p in range(q0 + w * per, min(q1, q0 + (w + 1) * per)):
            kb = 256 * p
            for c in range(CG):
                for i in range(4):
                    row = 16 * c + 4 * i + lr
                    col = kb + 16 * lc
                    out.append(("b", n0, np.where(col < K, row * K + col, K_OOB), 0, recs_w))
            for s in range(4):
                for t in range(MT):
                    col = kb + 64 * s + 16 * kq
                    out.append(("a", 0, np.where(col < K, (16 * t + r16) * K + col, K_OOB), 0, recs_x))
    return out


def fewtok_config(M, N):
    """(MT, NW, CG) of the few-token kernel (launch_gemm / launch_fewtok)."""
    MT = 1 if M <= 16 else 2 if M <= 32 else 4 if M <= 64 else 8
    if MT >= 4:
        return MT, 4, 1 if N <= 4096 else 2 if N <= 8192 else 4
    return (MT,) + ((8, 1) if N < 12288 else (8, 4) if MT == 2 else (4, 2))


@pytest.mark.parametrize("M,N,K", [(3, 16392, 4096), (13, 136, 1040), (31, 4104, 16384), (17, 8, 16),
                                   (32, 12288, 4112), (5, 24, 65536), (20, 12296, 272),
                                   (33, 4104, 4112), (64, 8200, 272), (37, 12288, 65536),
                                   (65, 8192, 4112), (128, 4096, 16), (100, 24, 8208)])
def test_few_token_kernel_loads_stay_in_bounds(M, N, K):
    MT, NW, CG = fewtok_config(M, N)
    for n0 in sorted({0, (N - 1) // (16 * CG) * (16 * CG)}):
        assert_in_bounds(fewtok_loads(M, N, K, n0, MT, NW, CG), M, N, K)


def splitk_plan(M, N, K):
    """(splits, groups) of the runtime forward's split-K form, or None."""
    if M < 3 or M > 32 or N < 1 or N >= 12288 or K < 1:
        return None
    groups = -(-N // 64)
    npc = -(-K // 256)
    if (npc < 32) if M >= 17 else (N >= 2048 or npc < 64):
        return None
    s = min(-(-256 // groups), npc // 8, 16)
    return (s, groups) if s >= 2 else None


def splitk_slice_offsets(M, N, S, sp, n0, MT, CG=4):
    """Byte offsets of the partial-slice stores of block (n0, sp) and of the
    loads the last block of the group makes from the other slices: one
    16-byte access per lane and fragment, rows m < M and channels n < N."""
    lane = np.arange(64)
    out = []
    for f in range(CG * MT):
        m = (f % MT) * 16 + lane % 16
        n = n0 + (f // MT) * 16 + 4 * (lane // 16)
        live = (m < M) & (n < N)
        for s2 in range(S):
            out.append((((s2 * M + m) * N + n) * 4)[live])
    return out


@pytest.mark.parametrize("M,N,K", [(32, 4096, 16384), (24, 1024, 16384), (5, 1024, 16384),
                                   (31, 2056, 8208), (16, 264, 65536), (20, 8192, 8192),
                                   (17, 2040, 8192), (3, 2040, 16400)])
def test_split_k_loads_and_slices_stay_in_bounds(M, N, K):
    S, groups = splitk_plan(M, N, K)
    MT = -(-M // 16)
    assert S * M * N * 4 < 2 ** 31  # the slices' buffer resource has a 32-bit size
    for n0 in sorted({0, (groups - 1) * 64}):
        for sp in range(S):
            assert_in_bounds(fewtok_loads(M, N, K, n0, MT, 8, 4, S, sp), M, N, K)
            for off in splitk_slice_offsets(M, N, S, sp, n0, MT):
                assert (off >= 0).all() and (off + 16 <= S * M * N * 4).all()
                assert (off % 16 == 0).all()
    # the splits' piece ranges cover every piece once
    npc = -(-K // 256)
    cover = sorted(p for sp in range(S) for p in range(npc * sp // S, npc * (sp + 1) // S))
    assert cover == list(range(npc))


def test_split_k_plan_shapes():
    """Which shapes split (the rule the launcher and the workspace size share)."""
    assert splitk_plan(32, 4096, 16384) == (4, 64)
    assert splitk_plan(32, 8192, 8192) == (2, 128)
    assert splitk_plan(17, 1024, 16384) == (8, 16)
    assert splitk_plan(16, 1024, 16384) == (8, 16)
    assert splitk_plan(16, 2048, 16384) is None
    assert splitk_plan(16, 1024, 8192) is None
    assert splitk_plan(2, 1024, 16384) is None
    assert splitk_plan(32, 1024, 4096) is None
    assert splitk_plan(32, 4096, 4096) is None
    assert splitk_plan(32, 12288, 16384) is None
    assert splitk_plan(32, 520, 1040) is None  # 5 pieces per row


def gemv_loads(M, N, K, n0, MT, R=4):
    """Loads of one block of the row-streaming kernel (one or two tokens):
    thread t reads 16-byte chunk c = t + 256 j of each of the block's R weight
    rows and of the MT token slots' activation rows, JB chunks per pass."""
    kc = K // 16
    segs = -(-kc // 256)
    JB = 1 if segs <= 1 else 2 if segs == 2 else 4
    tid = np.arange(256)
    nr = min(R, N - n0)
    out = []
    c0 = tid.copy()
    while True:
        live = c0 < kc  # threads still in the pass loop
        if not live.any():
            break
        for j in range(JB):
            c = c0 + 256 * j
            inb = c < kc
            for r in range(R):
                vo = np.where(inb, r * K + 16 * c, K_OOB)[live]
                out.append(("b", n0, vo, 0, nr * K))
            for t in range(MT):
                vo = np.where(inb, t * K + 16 * c, K_OOB)[live]
                out.append(("a", 0, vo, 0, M * K))
        c0 = c0 + 256 * JB
    return out


@pytest.mark.parametrize("M,N,K", [(1, 16384, 4096), (2, 4096, 16384), (1, 8, 16), (2, 24, 4112),
                                   (1, 8192, 11008), (2, 16, 131072)])
def test_row_streaming_kernel_loads_stay_in_bounds(M, N, K):
    for n0 in sorted({0, (N - 1) // 4 * 4}):
        assert_in_bounds(gemv_loads(M, N, K, n0, M), M, N, K)
