"""GPU parity of w8a8_calibrate_smooth: one launch that folds a calibration
batch into the running max|X_j|, takes max|W_j| and forms s and inv_s.

The maxima must equal the oracle's bit for bit; s and inv_s are held to the
same bar as w8a8_smooth_factors (bit-equal unless the fp64 value sits on an
fp32 rounding midpoint), and to the bits of the three-call path
(channel_amax twice, smooth_factors), which uses the same device code.  The
blocks of one call meet only through device atomics, so repeated calls on
one scratch check that every call sees all of its blocks' maxima and leaves
the scratch zero.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import w8a8_int8_amd as w8
from tests.test_gpu_parity import assert_s_parity, dt_name, host, np_bits

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def inputs(cal_rows, N, K, dtype, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    xc = torch.randn((cal_rows, K), generator=g)
    w = torch.randn((N, K), generator=g) * 0.05
    if K:
        idx = torch.randperm(K, generator=g)[:4]
        xc[:, idx] *= 60.0
        if K > 16:
            xc[:, :3] = 0.0  # dead activation channels (s = 1 when the start is 0 too)
            w[:, 5:7] = 0.0  # dead weight channels
    start = torch.rand(K, generator=g) * 2.0
    start[: min(K, 4)] = 0.0
    return xc.to(dtype).to(DEV), w.to(dtype).to(DEV), start.to(DEV)


def three_call(xc, w, start, alpha):
    ax = w8.channel_amax(xc, start.clone())
    aw = w8.channel_amax(w)
    s, inv_s = w8.smooth_factors(ax, aw, alpha)
    return ax, aw, s, inv_s


CASES = [(2048, 12288, 4096, torch.float16, 0.5), (2048, 4096, 11008, torch.float16, 0.5),
         (37, 136, 136, torch.bfloat16, 0.3), (0, 520, 1032, torch.float16, 0.8),
         (300, 0, 4104, torch.bfloat16, 0.5), (5, 7, 8, torch.float16, 1.0),
         (1000, 3000, 28672, torch.bfloat16, 0.0), (129, 22016, 4096, torch.float16, 0.5),
         (0, 0, 264, torch.float16, 0.5), (4096, 28672, 8192, torch.bfloat16, 0.5)]


@pytest.mark.parametrize("cal_rows,N,K,dtype,alpha", CASES)
def test_calibrate_smooth(cal_rows, N, K, dtype, alpha):
    xc, w, start = inputs(cal_rows, N, K, dtype, seed=cal_rows + 7 * N + K)
    scratch = w8.calibrate_smooth_scratch(K, DEV)
    ax = start.clone()
    aw, s, inv_s = w8.calibrate_smooth(xc if cal_rows else None, w, alpha, ax, scratch=scratch)
    torch.cuda.synchronize()
    assert not scratch.any()  # the call leaves its scratch zero
    ax_or = oracle.channel_amax(np_bits(xc), dt_name(xc), amax=host(start)) if cal_rows \
        else host(start)
    aw_or = oracle.channel_amax(np_bits(w), dt_name(w)) if N else np.zeros(K, np.float32)
    assert np.array_equal(host(ax).view(np.uint32), ax_or.view(np.uint32))
    assert np.array_equal(host(aw).view(np.uint32), aw_or.view(np.uint32))
    assert assert_s_parity(host(s), host(inv_s), ax_or, aw_or, alpha) == 0
    # the same bits as the three-call path
    ax3, aw3, s3, inv3 = three_call(xc, w, start, alpha)
    for a, b in ((ax, ax3), (aw, aw3), (s, s3), (inv_s, inv3)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_calibrate_smooth_repeated_calls_share_one_scratch():
    """60 calls of varying shapes on one scratch: each sees all of its maxima,
    none sees a maximum of an earlier call, and the scratch ends zero."""
    rng = np.random.default_rng(5)
    Kmax = 11008
    scratch = w8.calibrate_smooth_scratch(Kmax, DEV)
    for i in range(60):
        K = 8 * int(rng.integers(1, Kmax // 8 + 1))
        cal_rows = int(rng.choice([0, 1, int(rng.integers(2, 3000))]))
        N = int(rng.choice([0, 1, int(rng.integers(2, 6000))]))
        dtype = torch.float16 if i % 2 else torch.bfloat16
        alpha = float(rng.choice([0.0, 0.5, 0.85, 1.0]))
        xc, w, start = inputs(cal_rows, N, K, dtype, seed=100 + i)
        ax = start.clone()
        aw, s, inv_s = w8.calibrate_smooth(xc if cal_rows else None, w, alpha, ax,
                                           scratch=scratch)
        ax3, aw3, s3, inv3 = three_call(xc, w, start, alpha)
        for a, b in ((ax, ax3), (aw, aw3), (s, s3), (inv_s, inv3)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (i, cal_rows, N, K)
    torch.cuda.synchronize()
    assert not scratch.any()


def test_calibrate_smooth_running_over_batches():
    """Calibration batches through channel_amax, the last one through the
    fused call: amax_x is the running maximum of all of them."""
    K, N = 4096, 2048
    xs = [inputs(r, 0, K, torch.float16, seed=r)[0] for r in (512, 3, 1000)]
    _, w, _ = inputs(0, N, K, torch.float16, seed=9)
    ax = torch.zeros(K, device=DEV)
    for x in xs[:-1]:
        w8.channel_amax(x, ax)
    aw, s, inv_s = w8.calibrate_smooth(xs[-1], w, 0.5, ax)
    want = None
    for x in xs:
        want = oracle.channel_amax(np_bits(x), "f16", amax=want)
    assert np.array_equal(host(ax).view(np.uint32), want.view(np.uint32))
    aw_or = oracle.channel_amax(np_bits(w), "f16")
    assert assert_s_parity(host(s), host(inv_s), want, aw_or, 0.5) == 0


LAYER_SETS = [
    # the Llama-2-7B block's four layers, one 2048-token batch each
    [(2048, 12288, 4096), (2048, 4096, 4096), (2048, 22016, 4096), (2048, 4096, 11008)],
    # one layer; mixed and ragged shapes, empty calibration batch and empty weight
    [(129, 520, 1032)],
    [(37, 136, 136), (0, 520, 1032), (300, 0, 4104), (5, 7, 8), (0, 0, 264)],
    # ten layers: two launches (eight, then two)
    [(64 + 9 * i, 256 + 40 * i, 8 * (32 + 17 * i)) for i in range(10)],
]


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("si", range(len(LAYER_SETS)))
def test_calibrate_smooth_layers(si, dtype):
    """Several layers in one launch: every layer's maxima against the oracle
    bit for bit, s and inv_s to the smoothing-factor bar, and the same bits
    as one calibrate_smooth call per layer; every scratch ends zero."""
    alpha = 0.5 if si != 2 else 0.8
    shapes = LAYER_SETS[si]
    ins = [inputs(c, n, k, dtype, seed=1000 * si + 10 * i + (dtype == torch.bfloat16))
           for i, (c, n, k) in enumerate(shapes)]
    f32 = dict(dtype=torch.float32, device=DEV)
    groups, outs = [], []
    for (c, n, k), (xc, w, start) in zip(shapes, ins):
        ax = start.clone()
        o = (ax, torch.empty(k, **f32), torch.empty(k, **f32), torch.empty(k, **f32),
             w8.calibrate_smooth_scratch(k, DEV))
        outs.append(o)
        groups.append((xc if c else None, w) + o)
    w8.calibrate_smooth_layers(groups, alpha)
    torch.cuda.synchronize()
    for (c, n, k), (xc, w, start), (ax, aw, s, inv_s, scratch) in zip(shapes, ins, outs):
        assert not scratch.any()
        ax_or = oracle.channel_amax(np_bits(xc), dt_name(xc), amax=host(start)) if c \
            else host(start)
        aw_or = oracle.channel_amax(np_bits(w), dt_name(w)) if n else np.zeros(k, np.float32)
        assert np.array_equal(host(ax).view(np.uint32), ax_or.view(np.uint32)), (c, n, k)
        assert np.array_equal(host(aw).view(np.uint32), aw_or.view(np.uint32)), (c, n, k)
        assert assert_s_parity(host(s), host(inv_s), ax_or, aw_or, alpha) == 0
        ax1 = start.clone()
        aw1, s1, inv1 = w8.calibrate_smooth(xc if c else None, w, alpha, ax1)
        for a, b in ((ax, ax1), (aw, aw1), (s, s1), (inv_s, inv1)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (c, n, k)


def test_calibrate_smooth_layers_repeated():
    """The grouped call over the same layers and scratches 20 times in a row,
    with fresh calibration batches: the running maxima follow the per-layer
    calls, and the scratches stay zero between calls."""
    shapes = [(512, 1024, 4096), (256, 4096, 1024), (1000, 2048, 2048)]
    f32 = dict(dtype=torch.float32, device=DEV)
    st = [(torch.zeros(k, **f32), torch.empty(k, **f32), torch.empty(k, **f32),
           torch.empty(k, **f32), w8.calibrate_smooth_scratch(k, DEV)) for _, _, k in shapes]
    ref = [torch.zeros(k, **f32) for _, _, k in shapes]
    ws = [inputs(0, n, k, torch.float16, seed=50 + i)[1] for i, (_, n, k) in enumerate(shapes)]
    for it in range(20):
        xcs = [inputs(c, 0, k, torch.float16, seed=7000 + 10 * it + i)[0]
               for i, (c, _, k) in enumerate(shapes)]
        w8.calibrate_smooth_layers([(xc, w) + o for xc, w, o in zip(xcs, ws, st)], 0.5)
        for i, (xc, w) in enumerate(zip(xcs, ws)):
            aw1, s1, inv1 = w8.calibrate_smooth(xc, w, 0.5, ref[i])
            ax, aw, s, inv_s, _ = st[i]
            for a, b in ((ax, ref[i]), (aw, aw1), (s, s1), (inv_s, inv1)):
                assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (it, i)
    torch.cuda.synchronize()
    for o in st:
        assert not o[4].any()
