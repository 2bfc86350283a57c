"""Seeded random shapes through every entry point, against the CPU oracle.

Shapes are drawn small (the oracle finishes each in well under a second) but
cover empty inputs, ragged tails of every tile size, the few-token GEMM paths
(row streaming, LDS-transposed pieces and split-K), zero rows, dead channels, both 16-bit input types, the
FP8 quantizer, the RMS-norm fold and the dense 16-bit product.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import w8a8_int8_amd as w8
from w8a8_int8_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CASES = 24


def bits(t):
    return synth.to_numpy_bits(t)


def dt(t):
    return "f16" if t.dtype == torch.float16 else "bf16"


def host(t):
    return t.detach().cpu().numpy()


def rand_x(rng, rows, cols, dtype):
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    if cols:
        idx = rng.choice(cols, size=min(cols, 1 + cols // 64), replace=False)
        x[:, idx] *= rng.uniform(20, 120, idx.size).astype(np.float32)
    if rows > 3:
        x[rng.integers(0, rows)] = 0.0
    return torch.from_numpy(x).to(dtype).to(DEV)


@pytest.mark.parametrize("case", range(CASES))
def test_fuzz_quant_and_amax(case):
    rng = np.random.default_rng(1000 + case)
    dtype = torch.float16 if case % 2 == 0 else torch.bfloat16
    rows = int(rng.choice([0, 1, 2, 3, int(rng.integers(4, 700))]))
    cols = 16 * int(rng.integers(0 if case % 5 else 1, 300))
    x = rand_x(rng, rows, cols, dtype)
    c = torch.from_numpy(np.exp(rng.uniform(-6, 6, cols)).astype(np.float32)).to(DEV)
    q, d = w8.scale_quant_rows(x, c)
    q_or, d_or = oracle.scale_quant_rows(bits(x), dt(x), host(c))
    assert np.array_equal(host(q), q_or)
    assert np.array_equal(host(d).view(np.uint32), d_or.view(np.uint32))
    if cols:
        start = np.abs(rng.standard_normal(cols)).astype(np.float32) * (case % 3 == 0)
        amax = w8.channel_amax(x, torch.from_numpy(start.copy()).to(DEV))
        want = oracle.channel_amax(bits(x), dt(x), amax=start) if rows else start
        assert np.array_equal(host(amax).view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("case", range(CASES))
def test_fuzz_gemm(case):
    rng = np.random.default_rng(2000 + case)
    M = int(rng.choice([0, 1, int(rng.integers(2, 17)), int(rng.integers(17, 33)),
                        int(rng.integers(33, 600))]))
    N = 8 * int(rng.integers(0 if case % 7 else 1, 90))
    K = 16 * int(rng.integers(0, 90))
    qa = torch.from_numpy(rng.integers(-127, 128, (M, K), dtype=np.int8)).to(DEV)
    qb = torch.from_numpy(rng.integers(-127, 128, (N, K), dtype=np.int8)).to(DEV)
    c_or = oracle.gemm_i32(host(qa), host(qb))
    assert np.array_equal(host(w8.gemm_i32(qa, qb)), c_or)
    sa = torch.from_numpy(rng.uniform(1e-4, 0.05, M).astype(np.float32)).to(DEV)
    sb = torch.from_numpy(rng.uniform(1e-5, 2e-3, N).astype(np.float32)).to(DEV)
    out = torch.float16 if case % 2 == 0 else torch.bfloat16
    y = w8.gemm_dequant(qa, sa, qb, sb, out)
    y_or = oracle.dequant(c_or, host(sa), host(sb), "f16" if case % 2 == 0 else "bf16")
    assert np.array_equal(bits(y).view(np.uint16), y_or.view(np.uint16))


@pytest.mark.parametrize("case", range(12))
def test_fuzz_linear_pipeline(case):
    rng = np.random.default_rng(3000 + case)
    dtype = torch.float16 if case % 2 == 0 else torch.bfloat16
    K = 16 * int(rng.integers(1, 200))
    N = 8 * int(rng.integers(1, 120))
    M = int(rng.choice([1, int(rng.integers(2, 33)), int(rng.integers(33, 500))]))
    alpha = float(rng.choice([0.0, 0.5, 0.8, 1.0, rng.uniform()]))
    xc = rand_x(rng, int(rng.integers(1, 400)), K, dtype)
    w = torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)).to(dtype).to(DEV)
    x = rand_x(rng, M, K, dtype)
    if K > 16:
        w[:, 3] = 0  # a dead weight channel: s = 1 there
    amax_x = w8.channel_amax(xc)
    p = w8.prepare_weight(w, amax_x, alpha)
    y = w8.linear(x, p["inv_s"], p["qw"], p["sw"])
    ax = oracle.channel_amax(bits(xc), dt(x))
    po = oracle.prepare_weight(bits(w), dt(x), ax, alpha)
    lo = oracle.linear(bits(x), dt(x), po["inv_s"], po["qw"], po["sw"])
    assert np.array_equal(host(p["s"]).view(np.uint32), po["s"].view(np.uint32))
    assert np.array_equal(host(p["qw"]), po["qw"])
    assert np.array_equal(bits(y).view(np.uint16), lo["y"].view(np.uint16))


def test_repeat_runs_are_bitwise_identical():
    """Atomic max order and block scheduling do not change any result."""
    wl = synth.WORKLOADS["llama2_7b_prefill"]
    xc = synth.calibration(wl, 1, 2048, chunk=3, device=DEV)
    w = synth.weights(wl, 1, device=DEV)
    x = synth.activations(wl, 1, 2048, device=DEV)
    outs = []
    for _ in range(3):
        amax = w8.channel_amax(xc)
        p = w8.prepare_weight(w, amax, 0.5)
        outs.append((host(amax), host(p["qw"]), bits(w8.linear(x, p["inv_s"], p["qw"], p["sw"]))))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("case", range(12))
def test_fuzz_e4m3_quant(case):
    rng = np.random.default_rng(4000 + case)
    dtype = torch.float16 if case % 2 == 0 else torch.bfloat16
    rows = int(rng.choice([0, 1, int(rng.integers(2, 40))]))
    cols = 16 * int(rng.integers(0 if case % 5 else 1, 120))
    x = rand_x(rng, rows, cols, dtype)
    c = torch.from_numpy(np.exp(rng.uniform(-6, 6, cols)).astype(np.float32)).to(DEV)
    q, d = w8.scale_quant_rows_e4m3(x, c)
    q_or, d_or = oracle.scale_quant_rows_e4m3(bits(x), dt(x), host(c))
    assert np.array_equal(host(q), q_or)
    assert np.array_equal(host(d).view(np.uint32), d_or.view(np.uint32))


@pytest.mark.parametrize("case", range(12))
def test_fuzz_rmsnorm_quant(case):
    rng = np.random.default_rng(5000 + case)
    dtype = torch.float16 if case % 2 == 0 else torch.bfloat16
    rows = int(rng.choice([1, int(rng.integers(2, 300))]))
    cols = 16 * int(rng.integers(1, 300))
    h = rand_x(rng, rows, cols, dtype)
    gamma = torch.from_numpy(rng.uniform(0.1, 3.0, cols).astype(np.float32)).to(DEV)
    inv_s = torch.from_numpy(np.exp(rng.uniform(-5, 3, cols)).astype(np.float32)).to(DEV)
    eps = float(rng.choice([0.0, 1e-6, 1e-5, 0.1]))
    g = w8.fold_norm_weight(gamma, inv_s)
    q, d = w8.rmsnorm_quant_rows(h, g, eps)
    g_or = oracle.fold_norm_weight(host(gamma), host(inv_s))
    assert np.array_equal(host(g).view(np.uint32), g_or.view(np.uint32))
    q_or, d_or = oracle.rmsnorm_smooth_quant_rows(bits(h), dt(h), g_or, eps)
    assert np.array_equal(host(q), q_or)
    dh = host(d).astype(np.float64)
    assert (np.abs(dh - d_or) <= d_or * (cols / 2 + 6) * 2.0 ** -24).all()


@pytest.mark.parametrize("case", range(12))
def test_fuzz_layernorm_quant(case):
    """LayerNorm fold: codes and row scales bit for bit, random shapes, row
    offsets up to 10^3 and eps."""
    rng = np.random.default_rng(5500 + case)
    rows = int(rng.choice([1, int(rng.integers(2, 120))]))
    cols = 16 * int(rng.integers(1, 300))
    x = rand_x(rng, rows, cols, torch.float16)
    x = (x.float() + torch.from_numpy(rng.uniform(-1e3, 1e3, (rows, 1)).astype(np.float32)).to(DEV)).half()
    gamma = torch.from_numpy(rng.uniform(0.1, 3.0, cols).astype(np.float32)).to(DEV)
    beta = torch.from_numpy(rng.uniform(-1.0, 1.0, cols).astype(np.float32)).to(DEV)
    inv_s = torch.from_numpy(np.exp(rng.uniform(-5, 3, cols)).astype(np.float32)).to(DEV)
    eps = float(rng.choice([0.0, 1e-6, 1e-5, 0.1]))
    g, b = w8.fold_layernorm(gamma, beta, inv_s)
    q, d = w8.layernorm_quant_rows(x, g, b, eps)
    g_or = oracle.fold_norm_weight(host(gamma), host(inv_s))
    b_or = oracle.fold_norm_weight(host(beta), host(inv_s))
    q_or, d_or = oracle.layernorm_smooth_quant_rows(host(x), g_or, b_or, eps)
    assert np.array_equal(host(q), q_or)
    assert np.array_equal(host(d).view(np.uint32), d_or.view(np.uint32))


@pytest.mark.parametrize("case", range(12))
def test_fuzz_gemm_float(case):
    """Dense 16-bit product: within K 2^-24 sum|a b| of the exact value, plus
    one unit of the output format."""
    rng = np.random.default_rng(6000 + case)
    dtype = torch.float16 if case % 2 == 0 else torch.bfloat16
    M = int(rng.choice([0, 1, int(rng.integers(2, 40)), int(rng.integers(40, 600))]))
    N = 8 * int(rng.integers(1, 90))
    K = 8 * int(rng.integers(0, 200))
    a = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(dtype).to(DEV)
    b = torch.from_numpy((rng.standard_normal((N, K)) * 0.05).astype(np.float32)).to(dtype).to(DEV)
    y = w8.gemm_float(a, b)
    y64, bound = oracle.gemm_float(bits(a), bits(b), dt(a))
    yb = bits(y)
    got = yb.astype(np.float64) if dtype == torch.float16 else oracle.widen(yb, "bf16").astype(np.float64)
    e = np.floor(np.log2(np.maximum(np.abs(y64), 2.0 ** -14 if dtype == torch.float16 else 2.0 ** -126)))
    ulp = 2.0 ** (e - (10 if dtype == torch.float16 else 7))
    assert (np.abs(got - y64) <= K * 2.0 ** -24 * bound + ulp).all()


@pytest.mark.parametrize("case", range(8))
def test_fuzz_linear_split_k(case):
    """Token counts and K for which the runtime forward splits K: 3-32 tokens
    under 2048 channels with rows of 64 or more 256-byte pieces, 17-32 tokens
    up to 12280 channels with rows of 32 or more."""
    rng = np.random.default_rng(7000 + case)
    dtype = torch.float16 if case % 2 == 0 else torch.bfloat16
    if case < 4:
        M = int(rng.integers(3, 33))
        K = 16 * int(rng.integers(1009, 2048))
        N = 8 * int(rng.integers(1, 256))
    else:
        M = int(rng.integers(17, 33))
        K = 16 * int(rng.integers(497, 1024))
        N = 8 * int(rng.integers(256, 1536))
    w = torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)).to(dtype).to(DEV)
    xc = rand_x(rng, 64, K, dtype)
    x = rand_x(rng, M, K, dtype)
    p = w8.prepare_weight(w, w8.channel_amax(xc), 0.5)
    y = w8.linear(x, p["inv_s"], p["qw"], p["sw"])
    qx_or, sx_or = oracle.scale_quant_rows(bits(x), dt(x), host(p["inv_s"]))
    y_or = oracle.dequant(oracle.gemm_i32(qx_or, host(p["qw"])), sx_or, host(p["sw"]), dt(x))
    assert np.array_equal(bits(y).view(np.uint16), y_or.view(np.uint16))
