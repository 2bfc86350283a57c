"""Seeded synthetic inputs for the W8A8 linear-layer path.

This module only draws data: calibration activations, runtime activations and
weights with the shapes and value distributions of the workloads below.  It
holds none of the method's arithmetic (no scaling, no quantization, no GEMM),
so the CPU oracle and the HIP path can both consume its output.

Value model (jisaku.com glossary page "SmoothQuant", section on the activation
outlier problem): most activation channels are roughly unit normal, while a few
channels carry values one to two orders of magnitude larger; weights have no
such outliers (section on why weights are outlier-free).  Recipe:

* a layer's outlier channels are a seeded set of ``n_out`` distinct input
  channels; channel j gets one factor ``sign_j * c_j`` with ``c_j ~ U[lo, hi]``
  and a random sign, shared by calibration and runtime activations;
* activations: ``z ~ N(0, 1)`` in fp32, outlier columns multiplied by their
  factor, then rounded to the layer dtype (fp16 or bf16, round to nearest even);
* weights (stored N x K, output channel major, K contiguous): ``N(0, sigma)``
  in fp32, rounded to the layer dtype.

Every draw comes from a ``torch.Generator`` seeded from (workload, layer,
stream, chunk); the same call on the same device returns the same bits.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional, Sequence, Tuple

import torch

# stream ids of the seeded generators
STREAM_OUTLIERS = 0
STREAM_CALIB = 1
STREAM_X = 2
STREAM_W = 3


@dataclasses.dataclass(frozen=True)
class Layer:
    name: str
    K: int  # input channels
    N: int  # output channels


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: Tuple[int, ...]  # runtime token counts
    layers: Tuple[Layer, ...]
    dtype: str  # "f16" or "bf16": activation, weight and output dtype
    n_out: Optional[int]  # fixed outlier count, or None to use out_frac
    out_frac: float  # fraction of input channels that are outliers
    lo: float
    hi: float
    w_std: float
    alphas: Tuple[float, ...]
    cal_tokens: int  # calibration set size in tokens
    cal_batch: int  # tokens per calibration batch

    def outliers(self, K: int) -> int:
        if self.n_out is not None:
            return self.n_out
        return int(self.out_frac * K + 0.5)


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny_512", (64,), (Layer("linear", 512, 512),), "f16", 4, 0.0,
                 20.0, 120.0, 0.02, (0.5,), 256, 256),
        Workload("llama2_7b_prefill", (2048,),
                 (Layer("qkv", 4096, 12288), Layer("o_proj", 4096, 4096),
                  Layer("gate_up", 4096, 22016), Layer("down", 11008, 4096)),
                 "f16", None, 0.005, 20.0, 120.0, 0.02, (0.5,), 512 * 2048, 2048),
        Workload("opt6.7b_decode", (1, 8, 32),
                 (Layer("fc1", 4096, 16384), Layer("fc2", 16384, 4096),
                  Layer("qkv", 4096, 12288)),
                 "f16", None, 0.005, 20.0, 120.0, 0.02, (0.5, 0.8), 512 * 2048, 2048),
        Workload("opt30b_prefill", (4096,),
                 (Layer("qkv", 7168, 21504), Layer("out_proj", 7168, 7168),
                  Layer("fc1", 7168, 28672), Layer("fc2", 28672, 7168)),
                 "f16", None, 0.01, 50.0, 150.0, 0.015, (0.5,), 512 * 2048, 2048),
        Workload("llama2_70b_prefill", (8192,),
                 (Layer("qkv", 8192, 10240), Layer("gate_up", 8192, 57344),
                  Layer("down", 28672, 8192)),
                 "bf16", None, 0.005, 20.0, 120.0, 0.01, (0.5,), 512 * 2048, 2048),
    )
}


def torch_dtype(dtype: str) -> torch.dtype:
    return {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def seed_of(*parts) -> int:
    """A 63-bit seed from the given parts (stable across runs and machines)."""
    h = hashlib.sha256(repr(tuple(parts)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of("w8a8-synth-v1", *parts))
    return g


def outlier_spec(wl: Workload, layer: int, K: Optional[int] = None):
    """(channel index int64[n], factor float32[n]) of one layer's outliers (CPU)."""
    K = wl.layers[layer].K if K is None else K
    n = min(wl.outliers(K), K)
    g = _gen("cpu", wl.name, layer, STREAM_OUTLIERS)
    idx = torch.randperm(K, generator=g)[:n].sort().values
    c = torch.rand(n, generator=g, dtype=torch.float64) * (wl.hi - wl.lo) + wl.lo
    sign = torch.where(torch.rand(n, generator=g) < 0.5, -1.0, 1.0).to(torch.float64)
    return idx, (c * sign).to(torch.float32)


def _activations(wl: Workload, layer: int, rows: int, stream: int, chunk: int,
                 device, K: Optional[int] = None) -> torch.Tensor:
    K = wl.layers[layer].K if K is None else K
    g = _gen(device, wl.name, layer, stream, chunk, rows, K)
    z = torch.randn((rows, K), generator=g, device=device, dtype=torch.float32)
    idx, fac = outlier_spec(wl, layer, K)
    if idx.numel():
        idx = idx.to(device)
        z[:, idx] *= fac.to(device)
    return z.to(torch_dtype(wl.dtype))


def calibration(wl: Workload, layer: int, rows: int, chunk: int = 0,
                device="cpu", K: Optional[int] = None) -> torch.Tensor:
    """One calibration batch (rows x K) of layer ``layer``; ``chunk`` picks the batch."""
    return _activations(wl, layer, rows, STREAM_CALIB, chunk, device, K)


def activations(wl: Workload, layer: int, rows: int, device="cpu",
                K: Optional[int] = None, chunk: int = 0) -> torch.Tensor:
    """Runtime activations X (rows x K) of layer ``layer``."""
    return _activations(wl, layer, rows, STREAM_X, chunk, device, K)


def weights(wl: Workload, layer: int, device="cpu", N: Optional[int] = None,
            K: Optional[int] = None) -> torch.Tensor:
    """Weight W stored N x K (output channel major) of layer ``layer``."""
    L = wl.layers[layer]
    N = L.N if N is None else N
    K = L.K if K is None else K
    g = _gen(device, wl.name, layer, STREAM_W, N, K)
    w = torch.randn((N, K), generator=g, device=device, dtype=torch.float32)
    w *= wl.w_std
    return w.to(torch_dtype(wl.dtype))


def to_numpy_bits(t: torch.Tensor):
    """Host numpy view of a fp16 (as float16) or bf16 (as uint16 bit patterns) tensor."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float16:
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()


def layer_shapes(wl: Workload) -> Sequence[Tuple[str, int, int]]:
    return [(L.name, L.K, L.N) for L in wl.layers]
