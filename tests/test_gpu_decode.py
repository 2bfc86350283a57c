"""GPU parity of the runtime forward at few tokens (M <= 32): the
row-streaming kernel up to 2 tokens, the few-token kernel (weight pieces
transposed through LDS) up to 32, and from 17 to 32 tokens on layers under
12288 channels with long rows its split-K form: int32 partial slices handed
over in memory, summed exactly by the last block of each channel group.
Integer accumulation is order free, so the output must equal the oracle's bit
for bit, and equal the unsplit gemm_dequant path's.
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


_LAYERS = {}


def layer(N, K, dtype, seed):
    key = (N, K, dtype, seed)
    if key not in _LAYERS:
        _LAYERS.clear()  # keep one layer's weights resident at a time
        _LAYERS[key] = _make_layer(N, K, dtype, seed)
    return _LAYERS[key]


def _make_layer(N, K, dtype, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    w = (torch.randn((N, K), generator=g) * 0.02).to(dtype).to(DEV)
    xc = torch.randn((64, K), generator=g)
    if K:
        xc[:, torch.randperm(K, generator=g)[:4]] *= 60.0
    xc = xc.to(dtype).to(DEV)
    p = w8.prepare_weight(w, w8.channel_amax(xc), 0.5)
    p["qw_host"] = host(p["qw"])
    return p


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 15, 16, 17, 31, 32])
@pytest.mark.parametrize("N,K", [(4096, 16384), (16384, 4096), (12288, 4096), (136, 80),
                                 (520, 1040), (264, 65536), (8, 16), (4104, 4112),
                                 (2056, 8208), (1024, 16384), (8192, 8192), (2040, 4096)])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_linear_decode_split_k(dtype, N, K, M):
    p = layer(N, K, dtype, N + K)
    g = torch.Generator(device="cpu").manual_seed(M * 7 + N)
    x = torch.randn((M, K), generator=g)
    x[:, :3] *= 50.0
    x = x.to(dtype).to(DEV)
    # the workspace needs no initialisation: fill it with garbage
    ws = torch.full((w8.linear_workspace_bytes(M, N, K),), 0x5A, dtype=torch.uint8, device=DEV)
    y = w8.linear(x, p["inv_s"], p["qw"], p["sw"], workspace=ws)
    qx = ws[:M * K].view(torch.int8).view(M, K)
    off = (M * K + 255) // 256 * 256
    sx = ws[off:off + 4 * M].view(torch.float32)
    # the unsplit kernel on the same codes gives the same bits
    y2 = w8.gemm_dequant(qx, sx, p["qw"], p["sw"], dtype)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    name = "f16" if dtype == torch.float16 else "bf16"
    qx_or, sx_or = oracle.scale_quant_rows(synth.to_numpy_bits(x), name, host(p["inv_s"]))
    assert np.array_equal(host(qx), qx_or)
    c = oracle.gemm_i32(qx_or, p["qw_host"])
    y_or = oracle.dequant(c, sx_or, host(p["sw"]), name)
    assert np.array_equal(synth.to_numpy_bits(y).view(np.uint16), y_or.view(np.uint16))


@pytest.mark.parametrize("M", [33, 48, 64, 65, 96, 128, 129])
@pytest.mark.parametrize("N,K", [(4096, 4096), (4104, 1040), (8192, 2064), (12288, 1024), (12296, 272),
                                 (520, 1040), (8, 16)])
def test_linear_mid_tokens(N, K, M):
    """33 to 128 tokens: the few-token kernel with four or eight token
    fragments on layers of up to 12288 / 8192 channels, the tiled kernel
    beyond; bit for bit against the oracle and the gemm_dequant call."""
    dtype = torch.float16 if M % 2 else torch.bfloat16
    p = layer(N, K, dtype, N + K)
    g = torch.Generator(device="cpu").manual_seed(M * 5 + N)
    x = torch.randn((M, K), generator=g)
    x[:, :2] *= 40.0
    x = x.to(dtype).to(DEV)
    y = w8.linear(x, p["inv_s"], p["qw"], p["sw"])
    name = "f16" if dtype == torch.float16 else "bf16"
    qx_or, sx_or = oracle.scale_quant_rows(synth.to_numpy_bits(x), name, host(p["inv_s"]))
    y_or = oracle.dequant(oracle.gemm_i32(qx_or, p["qw_host"]), sx_or, host(p["sw"]), name)
    assert np.array_equal(synth.to_numpy_bits(y).view(np.uint16), y_or.view(np.uint16))
    qx = torch.from_numpy(qx_or).to(DEV)
    sx = torch.from_numpy(sx_or).to(DEV)
    y2 = w8.gemm_dequant(qx, sx, p["qw"], p["sw"], dtype)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("N,K,M", [(1024, 16384, 32), (4096, 16384, 24)])
def test_linear_decode_repeat_calls_bit_identical(N, K, M):
    """The partial slices are overwritten and the counters cleared on every
    call: a second call with other activations, then the first again,
    reproduces the first output."""
    p = layer(N, K, torch.float16, 3)
    g = torch.Generator(device="cpu").manual_seed(9)
    xa = torch.randn((M, K), generator=g).half().to(DEV)
    xb = (torch.randn((M, K), generator=g) * 3).half().to(DEV)
    ws = torch.empty(w8.linear_workspace_bytes(M, N, K), dtype=torch.uint8, device=DEV)
    ya = w8.linear(xa, p["inv_s"], p["qw"], p["sw"], workspace=ws).clone()
    w8.linear(xb, p["inv_s"], p["qw"], p["sw"], workspace=ws)
    ya2 = w8.linear(xa, p["inv_s"], p["qw"], p["sw"], workspace=ws)
    assert torch.equal(ya.view(torch.int16), ya2.view(torch.int16))


def test_linear_workspace_too_small_is_rejected():
    N, K, M = 1024, 16384, 32
    p = layer(N, K, torch.float16, 5)
    x = torch.zeros((M, K), dtype=torch.float16, device=DEV)
    need = w8.linear_workspace_bytes(M, N, K)
    ws = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(_lib.W8A8Error, match="status 5"):
        w8.linear(x, p["inv_s"], p["qw"], p["sw"], workspace=ws)
