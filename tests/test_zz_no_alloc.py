"""w8a8_linear_noalloc (the runtime forward with the library's static scratch,
for callers that cannot allocate) against w8a8_linear, through the C ABI.

Two or more calls in a row share the one static array per GPU; each later
call is smaller than the one before, so a call that read stale scratch
contents (activation codes, scales or split-K partial sums of the previous
call) would differ from w8a8_linear.  Outputs must be bit-identical.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import w8a8_int8_amd as w8
from w8a8_int8_amd import _lib, synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCRATCH = 64 << 20
E_TOO_LARGE = 7


def _layer(M, N, K, dtype, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn((M, K), generator=g)
    x[:, torch.randperm(K, generator=g)[:4]] *= 60.0
    x = x.to(dtype).to(DEV)
    w = (torch.randn((N, K), generator=g) * 0.02).to(dtype).to(DEV)
    amax_x = w8.channel_amax(x)
    p = w8.prepare_weight(w, amax_x, 0.5)
    return x, p


def _call_noalloc(x, p, y):
    lib = _lib.load()
    M, K = x.shape
    N = p["qw"].shape[0]
    dt = _lib.W8A8_F16 if x.dtype == torch.float16 else _lib.W8A8_BF16
    return lib.w8a8_linear_noalloc(x.data_ptr(), dt, p["inv_s"].data_ptr(), p["qw"].data_ptr(),
                                   p["sw"].data_ptr(), y.data_ptr(), M, N, K,
                                   torch.cuda.current_stream().cuda_stream)


def _bits(t):
    return synth.to_numpy_bits(t).view(np.uint16)


@pytest.mark.parametrize("shapes,dtype", [
    # prefill, two split-K few-token calls (partial slices and counters in the
    # scratch; the second with fewer splits and smaller slices), an unsplit
    # 32-token call, then one token
    ([(2048, 4096, 4096), (32, 4096, 16384), (24, 1024, 16384), (32, 4096, 4096), (1, 4104, 1024)],
     torch.float16),
    # the largest Llama-2-7B activation (2048 x 11008), then 17-32 tokens on a narrow
    # layer with long rows (split), a narrow short-row call (unsplit), one at 5 tokens
    # split on a narrower layer, and one on a tiny layer
    ([(2048, 4096, 11008), (20, 1536, 8192), (20, 1536, 4096), (5, 1024, 16384), (5, 520, 1040)],
     torch.bfloat16),
])
def test_noalloc_matches_linear_on_calls_in_a_row(shapes, dtype):
    for i, (M, N, K) in enumerate(shapes):
        assert w8.linear_workspace_bytes(M, N, K) <= SCRATCH
        x, p = _layer(M, N, K, dtype, seed=100 * i + M)
        want = w8.linear(x, p["inv_s"], p["qw"], p["sw"])
        y = torch.full((M, N), float("nan"), dtype=dtype, device=DEV)
        assert _call_noalloc(x, p, y) == 0
        torch.cuda.synchronize()
        assert np.array_equal(_bits(y), _bits(want)), (M, N, K)


def test_noalloc_rejects_calls_beyond_its_scratch():
    M, N, K = 4096, 16, 16384  # M K = 64 MiB: with the scales, more than the scratch
    assert w8.linear_workspace_bytes(M, N, K) > SCRATCH
    x = torch.zeros((M, K), dtype=torch.float16, device=DEV)
    p = dict(inv_s=torch.ones(K, device=DEV), qw=torch.zeros((N, K), dtype=torch.int8, device=DEV),
             sw=torch.ones(N, device=DEV))
    y = torch.zeros((M, N), dtype=torch.float16, device=DEV)
    assert _call_noalloc(x, p, y) == E_TOO_LARGE
    torch.cuda.synchronize()
    assert not y.any()  # nothing was enqueued
