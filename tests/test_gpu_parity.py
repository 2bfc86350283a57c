"""GPU parity: the HIP path against the CPU oracle, element by element.

Every input comes from the seeded generator in w8a8_int8_amd.synth; the
oracle gets the same bits on the host.  Integer results (codes, accumulators)
and the fp32 scales must be bit-identical; fp16/bf16 outputs must be
bit-identical too (both sides follow the same fp32 operation order) and are
additionally checked against the bar max|dY| <= 1e-3 max|Y| + 1 ulp.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import w8a8_int8_amd as w8
from tests.exact import rn32_decimal, decimal_pow_ratio, ulp32
from w8a8_int8_amd import _lib, synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TINY = synth.WORKLOADS["tiny_512"]


def np_bits(t: torch.Tensor):
    return synth.to_numpy_bits(t)


def dt_name(t: torch.Tensor) -> str:
    return {torch.float16: "f16", torch.bfloat16: "bf16"}[t.dtype]


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def rand_act(rows, cols, dtype, seed, outliers=3):
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn((rows, cols), generator=g)
    if cols and outliers:
        idx = torch.randperm(cols, generator=g)[:outliers]
        x[:, idx] *= 80.0
    return x.to(dtype).to(DEV)


def y_values(y_np: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return y_np.astype(np.float64)
    return oracle.widen(y_np, "bf16").astype(np.float64)


def assert_y_close(y_gpu: np.ndarray, y_or: np.ndarray, dtype: str):
    a, b = y_values(y_gpu, dtype), y_values(y_or, dtype)
    if dtype == "f16":
        ulp = np.spacing(np.abs(b).astype(np.float16)).astype(np.float64)
    else:
        e = np.floor(np.log2(np.maximum(np.abs(b), 2.0 ** -126)))
        ulp = 2.0 ** (e - 7)
    tol = 1e-3 * np.abs(b).max(initial=0.0) + ulp
    assert (np.abs(a - b) <= tol).all()
    # both sides take the same fp32 steps: expect identical bits
    assert np.array_equal(y_gpu.view(np.uint16), y_or.view(np.uint16))


def assert_s_parity(s_gpu, inv_gpu, amax_x, amax_w, alpha):
    s_or, inv_or = oracle.smooth_factors(amax_x, amax_w, alpha)
    diff = np.nonzero(s_gpu.view(np.uint32) != s_or.view(np.uint32))[0]
    for j in diff:
        # only acceptable where the fp64 value sits on an fp32 rounding midpoint
        # to within the fp64 evaluation error of pow (device vs host libm)
        _, dist = rn32_decimal(decimal_pow_ratio(float(amax_x[j]), float(amax_w[j]), alpha))
        assert dist < 2.0 ** -45, (j, s_gpu[j], s_or[j])
        assert abs(float(s_gpu[j]) - float(s_or[j])) <= ulp32(s_or[j])
    ok = np.setdiff1d(np.arange(len(s_or)), diff)
    assert np.array_equal(inv_gpu[ok].view(np.uint32), inv_or[ok].view(np.uint32))
    return len(diff)


# ------------------------------------------------------------ step 1: amax


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("rows,cols", [(1, 8), (37, 136), (300, 1032), (2048, 4096),
                                       (1000, 11008), (129, 28672), (3001, 4104),
                                       (22016, 4096)])
def test_channel_amax(dtype, rows, cols):
    x = rand_act(rows, cols, dtype, seed=rows * 7 + cols)
    got = host(w8.channel_amax(x))
    want = oracle.channel_amax(np_bits(x), dt_name(x))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_channel_amax_running_batches():
    xs = [rand_act(r, 520 * 8, torch.float16, seed=r) for r in (2048, 5, 777)]
    amax = None
    want = None
    for x in xs:
        amax = w8.channel_amax(x, amax)
        want = oracle.channel_amax(np_bits(x), "f16", amax=want)
    assert np.array_equal(host(amax).view(np.uint32), want.view(np.uint32))


def test_channel_amax_large_calibration_slice():
    """One call over 131072 calibration tokens of a 4096-channel layer (1 GiB)."""
    wl = synth.WORKLOADS["llama2_7b_prefill"]
    x = synth.calibration(wl, 0, 131072, chunk=99, device=DEV)
    got = host(w8.channel_amax(x))
    want = oracle.channel_amax(np_bits(x), "f16")
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_channel_amax_zero_rows_keeps_running_value():
    amax = torch.full((64,), 3.0, device=DEV)
    x = torch.empty((0, 64), dtype=torch.float16, device=DEV)
    w8.channel_amax(x, amax)
    assert (amax == 3.0).all()


# -------------------------------------------------------- step 2: factors


@pytest.mark.parametrize("alpha", [0.0, 0.3, 0.5, 0.8, 1.0])
def test_smooth_factors(alpha):
    rng = np.random.default_rng(int(alpha * 10))
    K = 28672
    ax = np.exp(rng.uniform(-8, 8, K)).astype(np.float32)
    aw = np.exp(rng.uniform(-8, 3, K)).astype(np.float32)
    ax[:5] = 0
    aw[3:9] = 0
    s, inv = w8.smooth_factors(torch.from_numpy(ax).to(DEV), torch.from_numpy(aw).to(DEV), alpha)
    n = assert_s_parity(host(s), host(inv), ax, aw, alpha)
    assert n == 0


# ------------------------------------------------- steps 2b/3: scale + quant


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("rows,cols", [(1, 16), (3, 48), (64, 512), (1025, 4096),
                                       (2050, 7168), (4100, 11008), (1027, 9008), (33, 28672),
                                       (5, 65536), (7, 0)])
def test_scale_quant_rows(dtype, rows, cols):
    x = rand_act(rows, cols, dtype, seed=rows + 3 * cols)
    if rows > 2:
        x[1] = 0  # a zero row: codes 0, scale 0
    g = torch.Generator(device="cpu").manual_seed(cols)
    c = torch.exp(torch.rand(cols, generator=g) * 8 - 4).to(DEV)
    q, d = w8.scale_quant_rows(x, c)
    q_or, d_or = oracle.scale_quant_rows(np_bits(x), dt_name(x), host(c))
    assert np.array_equal(host(q), q_or)
    assert np.array_equal(host(d).view(np.uint32), d_or.view(np.uint32))
    assert not (host(q) == -128).any()


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("N,M,K", [(8, 1, 16), (136, 37, 80), (4096, 2048, 4096), (1027, 3, 9008),
                                   (5, 4100, 11008), (0, 9, 512), (9, 0, 512), (3, 2, 65536),
                                   (0, 0, 64)])
def test_scale_quant_pair(dtype, N, M, K):
    """Weight (col_scale s) and activations (col_scale inv_s) in one launch:
    each matrix's codes and scales equal the oracle's, bit for bit."""
    w = rand_act(N, K, dtype, seed=N + 5 * K)
    x = rand_act(M, K, dtype, seed=M + 7 * K + 1)
    if N > 2:
        w[1] = 0
    if M > 2:
        x[2] = 0
    g = torch.Generator(device="cpu").manual_seed(K + 11)
    s = torch.exp(torch.rand(K, generator=g) * 8 - 4).to(DEV)
    inv_s = torch.exp(torch.rand(K, generator=g) * 8 - 4).to(DEV)
    qw, sw, qx, sx = w8.scale_quant_pair(w, s, x, inv_s)
    for q, d, a, c in ((qw, sw, w, s), (qx, sx, x, inv_s)):
        q_or, d_or = oracle.scale_quant_rows(np_bits(a), dt_name(a), host(c))
        assert np.array_equal(host(q), q_or)
        assert np.array_equal(host(d).view(np.uint32), d_or.view(np.uint32))


# ---------------------------------------------------------------- step 4


def rand_codes(rows, cols, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randint(-127, 128, (rows, cols), generator=g, dtype=torch.int8).to(DEV)


# shapes cover the five tile configurations (128x32, 128x128, 256x128, 256x192, 256x256),
# the few-token kernels (row streaming: M <= 2, one to four 4 KiB row segments in flight
# and ragged K; weight pieces through LDS: 3 to 128 tokens, one to four channel groups per
# block), ragged M, N and K tails, K = 0 and empty outputs
GEMM_SHAPES = [(1, 8, 16), (37, 136, 80), (300, 520, 1040), (64, 512, 512),
               (48, 4096, 4096), (100, 8192, 272), (64, 12288, 272), (65, 4104, 1040),
               (129, 4096, 1040), (256, 4104, 4112), (200, 32, 16),
               (2048, 4096, 256), (4000, 8184, 272), (4096, 8192, 144), (513, 264, 4112),
               (5, 16, 0), (0, 8, 32), (8, 0, 32),
               (1, 4096, 16384), (3, 8, 64), (16, 520, 1040), (17, 136, 80), (32, 264, 4112),
               (33, 136, 80), (32, 16384, 272), (3000, 6000, 272), (2048, 12288, 144),
               (12, 12288, 1040), (16, 16392, 272), (13, 24576, 4112),
               (1, 8, 0), (2, 24, 4112), (2, 8, 8192), (1, 8192, 11008),
               (1, 16, 131072), (2, 40, 12304), (3, 24, 4112), (20, 12296, 4112), (31, 12352, 80)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_i32(M, N, K):
    qa, qb = rand_codes(M, K, M + K), rand_codes(N, K, N + 2 * K + 1)
    c = host(w8.gemm_i32(qa, qb))
    assert np.array_equal(c, oracle.gemm_i32(host(qa), host(qb)))


@pytest.mark.parametrize("M,K", [(33, 28672), (300, 131072), (8, 131072), (1, 131072), (2, 131072)])
def test_gemm_i32_extremes(M, K):
    """All +127 against all -127 up to the largest K the int32 accumulator
    allows (W8A8_MAX_K): -16129 K = -2114060288 at K = 131072, inside int32."""
    qa = torch.full((M, K), 127, dtype=torch.int8, device=DEV)
    qb = torch.full((16, K), -127, dtype=torch.int8, device=DEV)
    c = host(w8.gemm_i32(qa, qb))
    assert (c == -16129 * K).all()
    qb[3] = 127  # and the largest positive sum
    c = host(w8.gemm_i32(qa, qb))
    assert (c[:, 3] == 16129 * K).all() and (c[:, 4] == -16129 * K).all()


@pytest.mark.parametrize("out", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("M,N,K", [(37, 136, 80), (300, 520, 1040), (2048, 4096, 256),
                                   (4000, 8184, 272), (5, 16, 0), (1, 4104, 4112), (32, 264, 1040),
                                   (3000, 6000, 272), (96, 8200, 528), (160, 4096, 1040)])
def test_gemm_dequant(out, M, N, K):
    qa, qb = rand_codes(M, K, M + K), rand_codes(N, K, N + 2 * K + 1)
    g = torch.Generator(device="cpu").manual_seed(M * N)
    sa = (torch.rand(M, generator=g) * 0.05 + 1e-3).to(DEV)
    sb = (torch.rand(N, generator=g) * 2e-4 + 1e-5).to(DEV)
    y = w8.gemm_dequant(qa, sa, qb, sb, out)
    name = "f16" if out == torch.float16 else "bf16"
    y_or = oracle.dequant(oracle.gemm_i32(host(qa), host(qb)), host(sa), host(sb), name)
    assert_y_close(np_bits(y), y_or, name)


@pytest.mark.parametrize("out", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("M,N,K", [(1, 136, 256), (2, 264, 512), (8, 520, 256), (24, 1032, 1040),
                                   (300, 520, 272)])
def test_gemm_dequant_extreme_scales(out, M, N, K):
    """Channel scales spread over the output format's whole exponent range
    (fp32 subnormals 2^-149 up to 2^127 for bf16, 2^-40 .. 2^30 for fp16) and
    token scales near 1, so that the fp32 products and the 16-bit outputs
    reach subnormals, ties and values past the format's range (which round
    to infinity) in every row: every epilogue (row streaming, few-token,
    tiled) rounds as the oracle does, bit for bit."""
    qa, qb = rand_codes(M, K, 5 * M + K), rand_codes(N, K, 7 * N + K)
    g = torch.Generator(device="cpu").manual_seed(M + N + K)
    lo, hi = (-149.0, 127.0) if out == torch.bfloat16 else (-40.0, 30.0)
    sb = torch.exp2(torch.linspace(lo, hi, N) + 0.5 * torch.rand(N, generator=g)).clamp(
        max=2.0 ** 127).to(DEV)
    sa = torch.exp2(torch.randint(-8, 9, (M,), generator=g).float()
                    + torch.rand(M, generator=g)).to(DEV)
    y = w8.gemm_dequant(qa, sa, qb, sb, out)
    name = "f16" if out == torch.float16 else "bf16"
    with np.errstate(over="ignore"):
        y_or = oracle.dequant(oracle.gemm_i32(host(qa), host(qb)), host(sa), host(sb), name)
    got = np_bits(y).view(np.uint16)
    want = y_or.view(np.uint16)
    assert np.array_equal(got, want)
    # the case mix the test is for
    exp_bits = (want >> (10 if name == "f16" else 7)) & (0x1F if name == "f16" else 0xFF)
    mant = want & (0x3FF if name == "f16" else 0x7F)
    top = 0x1F if name == "f16" else 0xFF
    assert ((exp_bits == 0) & (mant != 0)).any()  # subnormal outputs
    assert (exp_bits == top).any()  # infinities


def _tile_of_shape(M, N):
    """The tiled kernel's tile choice for an M x N output (restated from the
    launcher: 128 x 32 tiles for 129-512 tokens on up to 4096 channels;
    otherwise the fullest last wave of blocks over 256 CUs, times the useful
    fraction of padded token rows, times a per-tile preference)."""
    if 128 < M <= 512 and N <= 4096:
        return (128, 32)
    best, best_score = None, -1.0
    for bm, bn, eff in ((256, 256, 1.0), (256, 128, 0.92), (128, 128, 0.8), (256, 192, 0.96)):
        tiles = -(-M // bm) * -(-N // bn)
        fill = tiles / (-(-tiles // 256) * 256)
        score = fill * (M / (-(-M // bm) * bm)) * eff
        if score > best_score + 1e-9:
            best, best_score = (bm, bn), score
    # two shapes in one grid: whole waves of 256 x 256 tiles, then 256 x 192
    if best[0] == 256:
        cyc = {256: 2339, 192: 1853, 128: 1404}
        mt = -(-M // 256)
        single = -(-(mt * -(-N // best[1])) // 256) * cyc[best[1]]
        w = mt * -(-N // 256) // 256
        if w >= 1 and (w * 256) % mt == 0 and w * 256 // mt * 256 < N:
            nt2 = -(-(N - w * 256 // mt * 256) // 192)
            if (w * cyc[256] + -(-(mt * nt2) // 256) * cyc[192]) * 100 <= single * 97:
                return "two"
    return best


@pytest.mark.parametrize("M,N,K,tile", [(2000, 24560, 272, (256, 256)), (2000, 12280, 272, (256, 192)),
                                        (2000, 4088, 1040, (256, 128)), (600, 1000, 1040, (128, 128)),
                                        (2000, 22000, 272, "two"), (4000, 7160, 1040, "two"),
                                        (200, 4000, 1040, (128, 32)), (130, 1000, 272, (128, 32)),
                                        (500, 4096, 528, (128, 32))])
def test_gemm_tiles_ragged(M, N, K, tile):
    """Each tile of the tiled kernel, and the grid of two tile shapes (whole
    waves of 256 x 256 tiles, then 256 x 192 tiles over the last channels),
    with a partial last tile in M and in N and a K that ends inside a
    128-byte stage.  With the 256-row tiles, waves 0-3 load the rows of waves
    4-7 as well, so the rows checked include both halves of the first tile and
    the ragged last tile rows.  C is checked in full (Freivalds) and exactly
    on those rows; Y on the same rows."""
    assert _tile_of_shape(M, N) == tile
    qa, qb = rand_codes(M, K, M + 3 * K), rand_codes(N, K, N + K + 7)
    c = host(w8.gemm_i32(qa, qb))
    qa_h, qb_h = host(qa), host(qb)
    assert_freivalds(c, qa_h, qb_h, seed=M + N)
    rows = np.array(sorted(set(range(0, 64)) | set(range(M - 40, M)) | set(_sample_rows(M, 16).tolist())))
    c_or = oracle.gemm_i32(qa_h[rows], qb_h)
    assert np.array_equal(c[rows], c_or)
    g = torch.Generator(device="cpu").manual_seed(M + K)
    sa = (torch.rand(M, generator=g) * 0.05 + 1e-3).to(DEV)
    sb = (torch.rand(N, generator=g) * 2e-4 + 1e-5).to(DEV)
    for out, name in ((torch.float16, "f16"), (torch.bfloat16, "bf16")):
        y = np_bits(w8.gemm_dequant(qa, sa, qb, sb, out))
        y_or = oracle.dequant(c_or, host(sa)[rows], host(sb), name)
        assert_y_close(y[rows], y_or, name)


# ------------------------------------------------------ end to end, tiny


def test_tiny_linear_end_to_end():
    wl = TINY
    xc = synth.calibration(wl, 0, wl.cal_tokens, device=DEV)
    w = synth.weights(wl, 0, device=DEV)
    x = synth.activations(wl, 0, wl.M[0], device=DEV)
    amax_x = w8.channel_amax(xc)
    p = w8.prepare_weight(w, amax_x, 0.5)
    y = w8.linear(x, p["inv_s"], p["qw"], p["sw"])
    # separate entry points give the same result as the fused linear call
    qx, sx = w8.scale_quant_rows(x, p["inv_s"])
    y2 = w8.gemm_dequant(qx, sx, p["qw"], p["sw"], torch.float16)
    assert torch.equal(y, y2)

    ax_or = oracle.channel_amax(np_bits(xc), "f16")
    assert np.array_equal(host(amax_x), ax_or)
    po = oracle.prepare_weight(np_bits(w), "f16", ax_or, 0.5)
    assert np.array_equal(host(p["amax_w"]), po["amax_w"])
    assert assert_s_parity(host(p["s"]), host(p["inv_s"]), ax_or, po["amax_w"], 0.5) == 0
    assert np.array_equal(host(p["qw"]), po["qw"])
    assert np.array_equal(host(p["sw"]).view(np.uint32), po["sw"].view(np.uint32))
    lo = oracle.linear(np_bits(x), "f16", po["inv_s"], po["qw"], po["sw"])
    assert np.array_equal(host(qx), lo["qx"])
    assert np.array_equal(host(sx).view(np.uint32), lo["sx"].view(np.uint32))
    assert np.array_equal(host(w8.gemm_i32(qx, p["qw"])), lo["c"])
    assert_y_close(np_bits(y), lo["y"], "f16")


def test_zero_activation_rows_give_zero_outputs():
    wl = TINY
    w = synth.weights(wl, 0, device=DEV)
    x = synth.activations(wl, 0, 40, device=DEV)
    x[7] = 0
    p = w8.prepare_weight(w, torch.ones(512, device=DEV), 0.5)
    y = w8.linear(x, p["inv_s"], p["qw"], p["sw"])
    assert (y[7] == 0).all() and (y[6] != 0).any()


def test_gpu_alignment_errors_with_real_buffers():
    x = torch.zeros((4, 40), dtype=torch.float16, device=DEV)
    amax = torch.zeros(32, device=DEV)
    lib = _lib.load()
    st = torch.cuda.current_stream().cuda_stream
    # a view that starts 2 bytes into the buffer is rejected before any launch
    assert lib.w8a8_channel_amax(x.data_ptr() + 2, 0, 4, 32, amax.data_ptr(), st) == 3
    buf = torch.zeros(4 * 32 + 8, dtype=torch.float16, device=DEV)
    xm = buf[1:1 + 4 * 32].view(4, 32)  # contiguous, 2 bytes past a 16-byte boundary
    with pytest.raises(_lib.W8A8Error):
        w8.scale_quant_rows(xm, torch.ones(32, device=DEV))


# ---------------------------------------- the five workloads at full size


def assert_freivalds(c, qx, qw, seed, vectors=4):
    """The whole M x N accumulator matrix against the oracle's codes without
    forming their product: for random integer vectors r in [-256, 256]^N,
    C r == qX (qW^T r) exactly.  Every partial sum is an integer below 2^53
    (|qW^T r| <= 127 * 256 * N, |qX (qW^T r)| and |C r| <= 127^2 * 256 * K * N
    < 2^53 at every workload size), so fp64 products are exact.  A wrong C
    passes one vector with probability at most 1/513."""
    rng = np.random.default_rng(seed)
    N = qw.shape[0]
    for _ in range(vectors):
        r = rng.integers(-256, 257, N).astype(np.float64)
        v = np.zeros(qw.shape[1], dtype=np.float64)
        for n0 in range(0, N, 4096):  # qW^T r, in row blocks to bound host memory
            v += r[n0:n0 + 4096] @ qw[n0:n0 + 4096].astype(np.float64)
        lhs = np.zeros(c.shape[0], dtype=np.float64)
        rhs = np.zeros(c.shape[0], dtype=np.float64)
        for m0 in range(0, c.shape[0], 512):
            lhs[m0:m0 + 512] = c[m0:m0 + 512].astype(np.float64) @ r
            rhs[m0:m0 + 512] = qx[m0:m0 + 512].astype(np.float64) @ v
        assert np.array_equal(lhs, rhs)


def _sample_rows(M, n=48, seed=0):
    rng = np.random.default_rng(seed)
    rows = set([0, M - 1]) | set(rng.integers(0, M, n).tolist())
    return np.array(sorted(rows))


def _workload_cases():
    cases = []
    for name, wl in synth.WORKLOADS.items():
        for li in range(len(wl.layers)):
            for alpha in wl.alphas:
                cases.append(pytest.param(name, li, alpha, id=f"{name}-{wl.layers[li].name}-a{alpha}"))
    return cases


@pytest.mark.slow
@pytest.mark.parametrize("name,li,alpha", _workload_cases())
def test_workload_layer(name, li, alpha):
    """Full-size layer through the calls the benchmark times, against the oracle:
    amax, s, inv_s, qW, sw, qX and sx in full (from the separate calls and from
    the one-launch pair); C of sampled token rows against
    the oracle's product, all of C by the Freivalds check, then every element
    of the runtime forward's Y against the oracle's dequant of that C."""
    wl = synth.WORKLOADS[name]
    L = wl.layers[li]
    dname = wl.dtype
    cal_rows = min(wl.cal_batch, wl.cal_tokens)
    xc = synth.calibration(wl, li, cal_rows, device=DEV)
    w = synth.weights(wl, li, device=DEV)
    Mmax = max(wl.M)
    x_all = synth.activations(wl, li, Mmax, device=DEV)

    amax_x = w8.channel_amax(xc)
    p = w8.prepare_weight(w, amax_x, alpha)
    # the benchmark step's form of the two quantizations: one launch
    M0 = wl.M[0]
    pair = w8.scale_quant_pair(w, p["s"], x_all[:M0].contiguous(), p["inv_s"])
    torch.cuda.synchronize()

    ax_or = oracle.channel_amax(np_bits(xc), dname)
    assert np.array_equal(host(amax_x).view(np.uint32), ax_or.view(np.uint32))
    w_np = np_bits(w)
    del w
    aw_or = oracle.channel_amax(w_np, dname)
    assert np.array_equal(host(p["amax_w"]).view(np.uint32), aw_or.view(np.uint32))
    s_or, inv_or = oracle.smooth_factors(ax_or, aw_or, alpha)
    assert assert_s_parity(host(p["s"]), host(p["inv_s"]), ax_or, aw_or, alpha) == 0
    qw_or, sw_or = oracle.scale_quant_rows(w_np, dname, s_or)
    del w_np
    assert np.array_equal(host(p["qw"]), qw_or)
    assert np.array_equal(host(p["sw"]).view(np.uint32), sw_or.view(np.uint32))
    assert np.array_equal(host(pair[0]), qw_or)
    assert np.array_equal(host(pair[1]).view(np.uint32), sw_or.view(np.uint32))

    ys = {}
    for M in wl.M:
        x = x_all[:M].contiguous()
        ws = torch.empty(w8.linear_workspace_bytes(M, L.N, L.K), dtype=torch.uint8, device=DEV)
        y = w8.linear(x, p["inv_s"], p["qw"], p["sw"], workspace=ws)
        qx = ws[:M * L.K].view(torch.int8).view(M, L.K)
        off = (M * L.K + 255) // 256 * 256
        sx = ws[off:off + 4 * M].view(torch.float32)
        qx_or, sx_or = oracle.scale_quant_rows(np_bits(x), dname, inv_or)
        assert np.array_equal(host(qx), qx_or)
        assert np.array_equal(host(sx).view(np.uint32), sx_or.view(np.uint32))
        if M == M0:
            assert np.array_equal(host(pair[2]), qx_or)
            assert np.array_equal(host(pair[3]).view(np.uint32), sx_or.view(np.uint32))
        rows = _sample_rows(M, seed=M + li)
        c_or = oracle.gemm_i32(qx_or[rows], qw_or)
        y_or = oracle.dequant(c_or, sx_or[rows], sw_or, dname)
        y_np = np_bits(y)
        assert_y_close(y_np[rows], y_or, dname)
        c = host(w8.gemm_i32(qx, p["qw"]))
        assert np.array_equal(c[rows], c_or)
        assert_freivalds(c, qx_or, qw_or, seed=M + 7 * li)
        # C is now verified in full, so the oracle's dequant of it is the
        # oracle's Y: every output of the product path, bit for bit
        for m0 in range(0, M, 1024):
            y_or_blk = oracle.dequant(c[m0:m0 + 1024], sx_or[m0:m0 + 1024], sw_or, dname)
            assert_y_close(y_np[m0:m0 + 1024], y_or_blk, dname)
        del c
        ys[M] = y_np
    # decode shapes: the first rows do not depend on how many rows follow
    ms = sorted(wl.M)
    for a, b in zip(ms, ms[1:]):
        assert np.array_equal(ys[a].view(np.uint16), ys[b][:a].view(np.uint16))


# ------------------------------------------- dense 16-bit baseline (fp16/bf16)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("M,N,K", [(37, 136, 80), (300, 520, 1040), (2048, 4096, 256),
                                   (4000, 8184, 272), (5, 16, 0), (1, 264, 4104),
                                   (2048, 12288, 4096), (3000, 6000, 272), (2000, 22000, 272)])
def test_gemm_float(dtype, M, N, K):
    """fp32-accumulated dense product: within K 2^-24 sum|a b| of the exact
    value before the final rounding, plus one unit of the output format."""
    g = torch.Generator(device="cpu").manual_seed(M + N + K)
    a = torch.randn((M, K), generator=g).to(dtype).to(DEV)
    b = (torch.randn((N, K), generator=g) * 0.05).to(dtype).to(DEV)
    y = w8.gemm_float(a, b)
    name = dt_name(a)
    y64, bound = oracle.gemm_float(np_bits(a), np_bits(b), name)
    got = y_values(np_bits(y), name)
    if name == "f16":
        ulp = np.spacing(np.abs(y64).astype(np.float16)).astype(np.float64)
    else:
        e = np.floor(np.log2(np.maximum(np.abs(y64), 2.0 ** -126)))
        ulp = 2.0 ** (e - 7)
    tol = K * 2.0 ** -24 * bound + ulp
    assert (np.abs(got - y64) <= tol).all()
