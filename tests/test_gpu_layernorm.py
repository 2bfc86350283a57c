"""GPU parity of the smoothing folded into a LayerNorm (w8a8_fold_norm_weight on
gamma and beta, w8a8_layernorm_quant_rows).

The row statistics are defined from exact integer sums of the fp16 row, so
the kernel's codes and row scales must equal the oracle's bit for bit, at
every size, for every eps, and on rows built to stress the sums (constant,
zero, +-65504, subnormal, a large common offset).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import w8a8_int8_amd as w8
from w8a8_int8_amd import _lib, synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def case(rows, cols, seed, offset=0.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn((rows, cols), generator=g) * torch.exp(torch.rand((rows, 1), generator=g) * 6 - 3)
    x += offset
    if cols:
        idx = torch.randperm(cols, generator=g)[:3]
        x[:, idx] *= 40.0
    x = x.clamp(-60000, 60000)
    gamma = torch.rand(cols, generator=g) * 1.5 + 0.25
    beta = torch.rand(cols, generator=g) - 0.5
    inv_s = torch.exp(torch.rand(cols, generator=g) * 6 - 4)
    return x.half().to(DEV), gamma.to(DEV), beta.to(DEV), inv_s.to(DEV)


def sample(n, k, seed):
    rng = np.random.default_rng(seed)
    return np.array(sorted(set([0, 1, 2, 3, n - 1]) | set(rng.integers(0, n, k).tolist())))


def check(x, gamma, beta, inv_s, eps, rows_idx=None):
    g, b = w8.fold_layernorm(gamma, beta, inv_s)
    g_or = oracle.fold_norm_weight(host(gamma), host(inv_s))
    b_or = oracle.fold_norm_weight(host(beta), host(inv_s))
    assert np.array_equal(host(g).view(np.uint32), g_or.view(np.uint32))
    assert np.array_equal(host(b).view(np.uint32), b_or.view(np.uint32))
    q, d = w8.layernorm_quant_rows(x, g, b, eps)
    xh, qh, dh = host(x), host(q), host(d)
    if rows_idx is not None:
        xh, qh, dh = xh[rows_idx], qh[rows_idx], dh[rows_idx]
    q_or, d_or = oracle.layernorm_smooth_quant_rows(xh, g_or, b_or, eps)
    assert np.array_equal(qh, q_or)
    assert np.array_equal(dh.view(np.uint32), d_or.view(np.uint32))
    return q, d


def stress_rows(x):
    """Rows 0-3: constant, zero, alternating +-65504, subnormals and a big offset."""
    cols = x.shape[1]
    x[0] = 3.25
    x[1] = 0.0
    x[2] = torch.tensor([65504.0, -65504.0] * (cols // 2), dtype=torch.float16)
    x[3] = 6e-8
    x[3, ::3] = -1e-7
    x[3, 0] = 2000.0
    return x


# Row lengths reach every launch form: one chunk per thread (16-512), two
# (1024), three on blocks of up to 512 threads (1040, 8208, 11008, ragged)
# and above (16384 on 704 threads, 20480 on 1024), four on up to 512 threads
# (4096, 5120, 7168) and on 1024 (28672), eight (65536).
@pytest.mark.parametrize("rows,cols", [(4, 16), (5, 48), (9, 4096), (7, 11008), (64, 512), (1025, 4096), (2050, 7168),
                                       (33, 28672), (5, 65536), (4, 1024), (4, 1040), (6, 5120),
                                       (5, 8208), (5, 16384), (4, 20480)])
def test_layernorm_quant_rows(rows, cols):
    x, gamma, beta, inv_s = case(rows, cols, rows * 7 + cols, offset=0.3)
    x = stress_rows(x)
    big = rows * cols > 2_000_000
    check(x, gamma, beta, inv_s, 1e-5, sample(rows, 24, cols) if big else None)


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.5, 1e4])
def test_layernorm_quant_rows_eps(eps):
    x, gamma, beta, inv_s = case(70, 1024, 11, offset=-2.0)
    check(x, gamma, beta, inv_s, eps)
    check(stress_rows(x), gamma, beta, inv_s, eps)


def test_layernorm_quant_rows_repeat_bit_identical():
    x, gamma, beta, inv_s = case(300, 7168, 5)
    g, b = w8.fold_layernorm(gamma, beta, inv_s)
    q1, d1 = w8.layernorm_quant_rows(x, g, b, 1e-5)
    q1, d1 = q1.clone(), d1.clone()
    q2, d2 = w8.layernorm_quant_rows(x, g, b, 1e-5)
    assert torch.equal(q1, q2) and torch.equal(d1.view(torch.int32), d2.view(torch.int32))


def test_layernorm_quant_rows_rejects_bf16_and_empty():
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device=DEV)
    g = torch.ones(64, device=DEV)
    with pytest.raises(_lib.W8A8Error, match="status 4"):
        w8.layernorm_quant_rows(x, g, g, 1e-5)
    q, d = w8.layernorm_quant_rows(torch.zeros((0, 64), dtype=torch.float16, device=DEV), g, g, 1e-5)
    assert q.shape == (0, 64) and d.shape == (0,)


def test_layernorm_quant_feeds_gemm_opt30b_qkv():
    """Full-size OPT-30B qkv layer (4096 tokens x 7168): LayerNorm-folded
    quantization of the hidden state feeding the INT8 GEMM.  Codes and row
    scales on sampled rows bit for bit; Y on the same rows bit for bit against
    the oracle's dequant of the exact product."""
    wl = synth.WORKLOADS["opt30b_prefill"]
    li = 0
    L = wl.layers[li]
    M = wl.M[0]
    xc = synth.calibration(wl, li, wl.cal_batch, device=DEV)
    w = synth.weights(wl, li, device=DEV)
    h = synth.activations(wl, li, M, device=DEV)
    g = torch.Generator(device="cpu").manual_seed(7)
    gamma = (torch.rand(L.K, generator=g) + 0.5).to(DEV)
    beta = (torch.rand(L.K, generator=g) * 0.2 - 0.1).to(DEV)
    p = w8.prepare_weight(w, w8.channel_amax(xc), 0.5)
    gf, bf = w8.fold_layernorm(gamma, beta, p["inv_s"])
    q, d = w8.layernorm_quant_rows(h, gf, bf, 1e-5)
    y = w8.gemm_dequant(q, d, p["qw"], p["sw"], torch.float16)
    torch.cuda.synchronize()
    rows = sample(M, 16, 2)
    g_or = oracle.fold_norm_weight(host(gamma), host(p["inv_s"]))
    b_or = oracle.fold_norm_weight(host(beta), host(p["inv_s"]))
    q_or, d_or = oracle.layernorm_smooth_quant_rows(host(h)[rows], g_or, b_or, 1e-5)
    assert np.array_equal(host(q)[rows], q_or)
    assert np.array_equal(host(d)[rows].view(np.uint32), d_or.view(np.uint32))
    c = oracle.gemm_i32(q_or, host(p["qw"]))
    y_or = oracle.dequant(c, d_or, host(p["sw"]), "f16")
    assert np.array_equal(synth.to_numpy_bits(y)[rows].view(np.uint16), y_or.view(np.uint16))
