"""GPU parity of the smoothing folded into the RMS norm (w8a8_fold_norm_weight,
w8a8_rmsnorm_quant_rows).

The INT8 codes must equal the oracle's bit for bit (the norm's 1 / rms only
enters the row scale); the row scale, whose sum of squares the device forms in
fp32 in its own order, must lie within (cols / 2 + 6) * 2^-24 relative of the
oracle's value computed with an exactly rounded sum.
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


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def dt_name(t: torch.Tensor) -> str:
    return {torch.float16: "f16", torch.bfloat16: "bf16"}[t.dtype]


def case(rows, cols, dtype, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    h = torch.randn((rows, cols), generator=g) * torch.exp(torch.rand((rows, 1), generator=g) * 4 - 2)
    if cols:
        idx = torch.randperm(cols, generator=g)[:3]
        h[:, idx] *= 60.0
    gamma = torch.rand(cols, generator=g) * 1.5 + 0.25
    inv_s = torch.exp(torch.rand(cols, generator=g) * 6 - 4)
    return h.to(dtype).to(DEV), gamma.to(DEV), inv_s.to(DEV)


def sample(n, k, seed):
    rng = np.random.default_rng(seed)
    return np.array(sorted(set([0, n - 1]) | set(rng.integers(0, n, k).tolist())))


def check(h, gamma, inv_s, eps, rows_idx=None):
    g = w8.fold_norm_weight(gamma, inv_s)
    g_or = oracle.fold_norm_weight(host(gamma), host(inv_s))
    assert np.array_equal(host(g).view(np.uint32), g_or.view(np.uint32))
    q, d = w8.rmsnorm_quant_rows(h, g, eps)
    hb = synth.to_numpy_bits(h)
    qh, dh = host(q), host(d).astype(np.float64)
    if rows_idx is not None:
        hb, qh, dh = hb[rows_idx], qh[rows_idx], dh[rows_idx]
    q_or, d_or = oracle.rmsnorm_smooth_quant_rows(hb, dt_name(h), g_or, eps)
    assert np.array_equal(qh, q_or)
    cols = h.shape[1]
    tol = (cols / 2 + 6) * 2.0 ** -24
    assert (np.abs(dh - d_or) <= d_or * tol).all()
    assert np.array_equal(dh == 0, d_or == 0)
    return q, d


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("rows,cols", [(1, 16), (3, 48), (64, 512), (1025, 4096), (2050, 7168),
                                       (33, 28672), (5, 65536), (1027, 9008)])
def test_rmsnorm_quant_rows(dtype, rows, cols):
    h, gamma, inv_s = case(rows, cols, dtype, rows * 7 + cols)
    if rows > 2:
        h[1] = 0  # a zero row: codes 0, scale 0
    big = rows * cols > 2_000_000
    rs = sample(rows, 24, cols) if big else None
    if big and rows > 2:
        rs = np.union1d(rs, [1])
    check(h, gamma, inv_s, 1e-5, rs)


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.5, 1e4])
def test_rmsnorm_quant_rows_eps(eps):
    h, gamma, inv_s = case(70, 1024, torch.float16, 11)
    h[5] = 0
    check(h, gamma, inv_s, eps)


@pytest.mark.parametrize("dtype,exp", [(torch.float16, -20), (torch.bfloat16, -66)])
@pytest.mark.parametrize("cols", [512, 4096, 11008])
def test_rmsnorm_quant_rows_tiny_rows(dtype, exp, cols):
    """Rows of tiny values with eps = 0, where a sum of squares lost to
    flushing would show as an infinite row scale: fp16 subnormal inputs (their
    squares are normal fp32 values), and bf16 values near 2^-66, whose squares
    are fp32 subnormals (exact: 16 significant bits above 2^-149)."""
    g = torch.Generator(device="cpu").manual_seed(cols + exp)
    h = torch.randn((9, cols), generator=g) * 2.0 ** exp
    gamma = torch.rand(cols, generator=g) * 1.5 + 0.25
    inv_s = torch.exp(torch.rand(cols, generator=g) * 6 - 4)
    h = h.to(dtype)
    assert h.abs().max() > 0
    if dtype == torch.float16:
        assert (h.float().abs() < 2.0 ** -14).all()  # every input subnormal
    else:
        assert (h.float() ** 2 < 2.0 ** -126).all()  # every square subnormal in fp32
    _, d = check(h.to(DEV), gamma.to(DEV), inv_s.to(DEV), 0.0)
    assert torch.isfinite(d).all()


def test_rmsnorm_quant_rows_codes_equal_folded_smoothing_quantizer():
    """The same codes as the smoothing quantizer with the folded weight g."""
    h, gamma, inv_s = case(300, 4096, torch.bfloat16, 3)
    g = w8.fold_norm_weight(gamma, inv_s)
    q, _ = w8.rmsnorm_quant_rows(h, g, 1e-5)
    q2, _ = w8.scale_quant_rows(h, g)
    assert torch.equal(q, q2)


def test_rmsnorm_quant_feeds_gemm_llama2_7b_qkv():
    """Full-size Llama-2-7B qkv layer (2048 tokens): norm-folded quantization
    of the hidden state feeding the INT8 GEMM; Y on sampled rows against the
    oracle within the row-scale tolerance and one output ulp."""
    wl = synth.WORKLOADS["llama2_7b_prefill"]
    li = 0
    L = wl.layers[li]
    M = wl.M[0]
    xc = synth.calibration(wl, li, wl.cal_batch, device=DEV)
    w = synth.weights(wl, li, device=DEV)
    h = synth.activations(wl, li, M, device=DEV)
    g = torch.Generator(device="cpu").manual_seed(5)
    gamma = (torch.rand(L.K, generator=g) + 0.5).to(DEV)
    amax_x = w8.channel_amax(xc)
    p = w8.prepare_weight(w, amax_x, 0.5)
    q, d = w8.rmsnorm_quant_rows(h, w8.fold_norm_weight(gamma, p["inv_s"]), 1e-5)
    y = w8.gemm_dequant(q, d, p["qw"], p["sw"], torch.float16)
    torch.cuda.synchronize()
    rows = sample(M, 24, 1)
    g_or = oracle.fold_norm_weight(host(gamma), host(p["inv_s"]))
    q_or, d_or = oracle.rmsnorm_smooth_quant_rows(synth.to_numpy_bits(h)[rows], "f16", g_or, 1e-5)
    assert np.array_equal(host(q)[rows], q_or)
    tol = (L.K / 2 + 6) * 2.0 ** -24
    assert (np.abs(host(d)[rows].astype(np.float64) - d_or) <= d_or * tol).all()
    # Y: exact int32 product, then the two scalings; the weight side is the
    # oracle's own fold and quantization of the same weight
    w_np = synth.to_numpy_bits(w)
    amax_w = oracle.channel_amax(w_np, "f16")
    s_or, inv_or = oracle.smooth_factors(oracle.channel_amax(synth.to_numpy_bits(xc), "f16"), amax_w, 0.5)
    assert np.array_equal(inv_or.view(np.uint32), host(p["inv_s"]).view(np.uint32))
    qw_or, sw_or = oracle.scale_quant_rows(w_np, "f16", s_or)
    c = oracle.gemm_i32(q_or, qw_or).astype(np.float64)
    y64 = c * d_or[:, None] * sw_or.astype(np.float64)[None, :]
    got = host(y)[rows].astype(np.float64)
    ulp = np.spacing(np.abs(y64).astype(np.float16)).astype(np.float64)
    assert (np.abs(got - y64) <= np.abs(y64) * (tol + 2.0 ** -22) + ulp).all()
