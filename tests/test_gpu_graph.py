"""The path under HIP graph capture: one layer's calibration + smoothing
factors (one launch), weight fold + quantization and the runtime forward,
captured once and replayed several times with new inputs written between the
replays.  Every replay must give the bits of the same calls made eagerly on
the same inputs (the library issues no memset and allocates nothing, and the
calibration scratch is left zero by every call, so replays need no reset)."""
from __future__ import annotations

import pytest
import torch

import w8a8_int8_amd as w8

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def fill(t: torch.Tensor, seed: int, scale: float = 1.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    t.copy_((torch.randn(t.shape, generator=g) * scale).to(t.dtype))


# 8 and 24 tokens on 4096 or more channels: the few-token GEMM; 24 tokens on
# 1024 channels with 8192 columns: its split-K form (partial slices in the
# workspace, counters cleared by the quantization launch); 512 tokens: the
# tiled GEMM.  form "pair": the benchmark step's calls (both quantizations in
# one launch, then gemm_dequant) instead of the runtime forward.
@pytest.mark.parametrize("M,N,K,form", [(8, 12288, 4096, "linear"), (24, 4096, 4096, "linear"),
                                        (24, 1024, 8192, "linear"), (512, 12288, 4096, "linear"),
                                        (512, 4096, 4096, "pair"), (24, 4096, 4096, "pair")])
def test_path_replays_match_eager(M, N, K, form):
    xc = torch.empty((2048, K), dtype=torch.float16, device=DEV)
    w = torch.empty((N, K), dtype=torch.float16, device=DEV)
    x = torch.empty((M, K), dtype=torch.float16, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    ax, aw, s, inv_s = (torch.zeros(K, **f32) for _ in range(4))
    qw = torch.empty((N, K), dtype=torch.int8, device=DEV)
    sw = torch.empty(N, **f32)
    y = torch.empty((M, N), dtype=torch.float16, device=DEV)
    ws = torch.empty(w8.linear_workspace_bytes(M, N, K), dtype=torch.uint8, device=DEV)
    scratch = w8.calibrate_smooth_scratch(K, DEV)

    qx = torch.empty((M, K), dtype=torch.int8, device=DEV)
    sx = torch.empty(M, **f32)

    def path():
        ax.zero_()  # a fill kernel, not a memset node
        w8.calibrate_smooth(xc, w, 0.5, ax, aw, s, inv_s, scratch)
        if form == "pair":
            w8.scale_quant_pair(w, s, x, inv_s, qw, sw, qx, sx)
            w8.gemm_dequant(qx, sx, qw, sw, torch.float16, y)
        else:
            w8.scale_quant_rows(w, s, qw, sw)
            w8.linear(x, inv_s, qw, sw, y, ws)

    fill(xc, 1, 3.0); fill(w, 2, 0.02); fill(x, 3, 3.0)
    path()  # warm up outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path()
    for rep in range(4):
        fill(xc, 10 + rep, 3.0); fill(w, 20 + rep, 0.02); fill(x, 30 + rep, 3.0)
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (ax, aw, s, inv_s, qw, sw, y)]
        assert not scratch.any()
        path()  # eager, same inputs
        torch.cuda.synchronize()
        want = (ax, aw, s, inv_s, qw, sw, y)
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), rep
