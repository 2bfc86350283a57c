"""Benchmark of the SmoothQuant W8A8 linear-layer path on one MI355X.

One step = one pass of the whole path over one batch, for every linear layer
of the Llama-2-7B-shaped decoder block (prefill, M = 2048 tokens):
  1. channel amax: fold one fresh 2048-token calibration batch into the
     layer's running max|X_j| (streaming calibration; step i uses batch i)
  2. max|W_j| over the weight, smoothing factors s and 1/s (1 and these, for
     every layer at once, in one launch: w8a8_calibrate_smooth_layers), fold s
     into W and quantize it per output channel
  3. smooth X (X / s) and quantize it per token (2's fold + quantize and this
     in one launch, w8a8_scale_quant_pair)
  4.+5. INT8 GEMM with the fused dequant epilogue -> fp16 Y
All inputs are resident in HBM before the timed region.

Order of a run: inputs built on the GPU; the per-kernel pass (each kernel
timed alone, seconds of GPU work, which also brings the GPU from its idle
clock to its working clock: the ramp takes 15-20 ms of load, longer than the
warm-up steps); W warm-up steps; K timed steps; then `steady_state` (more
steps with no pause, reported apart), the calibration-volume or decode pass,
the other workloads and the CPU oracle.

value = the step's INT8 GEMM work (2 M N K summed over the layers) divided by
the whole step's wall time, in TOPS.  The per-kernel breakdown also times the
dense fp16 product of each layer (same tiling on the 16-bit matrix cores) to
state the W8A8-vs-FP16 speedup at kernel level.  The roofline object reports the GEMM
kernel (the dominant kernel) against the dense INT8 MFMA peak, with its
average launch duration taken from HIP events recorded around every GEMM
launch of every fourth timed step (--event-every), created without the
system-scope fence; each event pair still idles the GPU for a few
microseconds, so the other timed steps carry none.  cpu_baseline times the CPU oracle on the
host cores over one step of the same workload.

python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                [--other-workloads A,B] [--ceilings]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0  # MI355X dense INT8 MFMA, 10^12 int ops / s
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
PEAK_DENSE16_TFLOPS = 2500.0  # MI355X dense fp16 / bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense FP8 MFMA
METRIC = "W8A8 GEMM TOPS + smooth/quant GB/s (% of MI355X peak), Llama-2-7B shapes"
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama2_7b_prefill")
    ap.add_argument("--alpha", type=float, default=0.5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--event-every", type=int, default=4,
                    help="record the GEMM timing events on every N-th timed step (each event pair "
                         "costs the step a few microseconds of idle GPU)")
    ap.add_argument("--kernel-reps", type=int, default=20,
                    help="repetitions per kernel in the per-kernel breakdown pass")
    ap.add_argument("--other-workloads", default="opt30b_prefill,llama2_70b_prefill,opt6.7b_decode",
                    help="comma-separated workloads whose kernels are also timed (per-kernel pass "
                         "only, into the `other_workloads` key); empty for none")
    ap.add_argument("--steady-steps", type=int, default=200,
                    help="after the timed steps, this many more steps with no pause, reported apart "
                         "(`steady_state`) and not in `value`: a check that the timed steps ran at "
                         "the settled clock")
    ap.add_argument("--ceilings", action="store_true",
                    help="only run the hardware probes (read-only streaming, copy, INT8 MFMA from "
                         "registers with the shader clock) and print their figures")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this size first (outside the timed "
                         "region): the reference for scaling hardware byte counters")
    return ap.parse_args()


def gemm_source_hash() -> str:
    """Hash of the GEMM sources' code (comments and blank lines dropped), which
    ties a committed counter summary to the kernels it was taken from."""
    h = hashlib.sha256()
    for f in ("gemm.hip", "common.h"):
        with open(os.path.join(ROOT, "w8a8_int8_amd", "csrc", f)) as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def pmc_traffic(workload: str, kernel: str = "gemm_i8"):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary,
    or None when there is none or the GEMM source changed since it was taken."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("gemm_source_hash") != gemm_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class TimingEvents:
    """HIP events for timing kernels on torch's current stream, created with
    hipEventDisableSystemFence.  A default event's record carries a
    system-scope release: cache write-back and invalidation at every record,
    which on this GPU holds back the next kernel by about 6 us.  These events
    only time (no host code reads memory through them), so they drop it."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes

        import torch

        torch.cuda.init()
        path = None
        with open("/proc/self/maps") as f:  # the HIP runtime torch already uses
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("HIP runtime not loaded")
        self.hip = ctypes.CDLL(path)
        self.ct = ctypes
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.torch = torch

    def create(self):
        ev = self.ct.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.ct.byref(ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags: {rc}")
        return _Event(self, ev)


class _Event:
    def __init__(self, owner, handle):
        self.o, self.h = owner, handle

    def record(self):
        rc = self.o.hip.hipEventRecord(self.h, self.o.torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord: {rc}")

    def elapsed_time(self, end):
        ms = self.o.ct.c_float()
        rc = self.o.hip.hipEventElapsedTime(self.o.ct.byref(ms), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime: {rc}")
        return ms.value

    def destroy(self):
        self.o.hip.hipEventDestroy(self.h)


class Layer:
    """Device buffers of one linear layer; all inputs generated up front."""

    def __init__(self, wl, li, n_batches, alpha, dev):
        import torch

        import w8a8_int8_amd as w8
        from w8a8_int8_amd import synth

        L = wl.layers[li]
        self.name, self.K, self.N, self.M = L.name, L.K, L.N, wl.M[0]
        self.alpha = alpha
        self.cal = [synth.calibration(wl, li, wl.cal_batch, chunk=i, device=dev)
                    for i in range(n_batches)]
        self.w = synth.weights(wl, li, device=dev)
        self.x_all = synth.activations(wl, li, max(wl.M), device=dev)
        self.x = self.x_all[:self.M]
        f32 = dict(dtype=torch.float32, device=dev)
        self.amax_x = torch.zeros(self.K, **f32)
        self.amax_w = torch.zeros(self.K, **f32)
        self.scratch = w8.calibrate_smooth_scratch(self.K, dev)
        self.s = torch.empty(self.K, **f32)
        self.inv_s = torch.empty(self.K, **f32)
        self.qw = torch.empty((self.N, self.K), dtype=torch.int8, device=dev)
        self.sw = torch.empty(self.N, **f32)
        self.qx = torch.empty((self.M, self.K), dtype=torch.int8, device=dev)
        self.sx = torch.empty(self.M, **f32)
        self.y = torch.empty((self.M, self.N), dtype=self.x.dtype, device=dev)
        self.w8 = w8

    def gemm_ops(self):
        return 2.0 * self.M * self.N * self.K

    def gemm_bytes(self, M=None):
        """Algorithmic HBM bytes of one GEMM launch: both INT8 operands once,
        the 16-bit output once, the two scale vectors."""
        M = self.M if M is None else M
        return float(M * self.K + self.N * self.K + 2 * M * self.N + 4 * (M + self.N))

    def calib_args(self, i):
        """This layer's entry of the grouped calibration call for step i."""
        return (self.cal[i % len(self.cal)], self.w, self.amax_x, self.amax_w, self.s, self.inv_s,
                self.scratch)

    def step(self, i, ev=None):
        """One pass of the path for this layer alone: calibration batch i
        folded into the running max|X_j|, max|W_j| and the smoothing factors
        (one launch), then quantize_forward."""
        self.w8.calibrate_smooth(self.cal[i % len(self.cal)], self.w, self.alpha, self.amax_x,
                                 self.amax_w, self.s, self.inv_s, self.scratch)
        self.quantize_forward(ev)

    def quantize_forward(self, ev=None):
        """The weight folded and quantized and the activations smoothed and
        quantized (one launch), and the INT8 GEMM with its dequant epilogue."""
        w8 = self.w8
        w8.scale_quant_pair(self.w, self.s, self.x, self.inv_s, self.qw, self.sw, self.qx, self.sx)
        if ev is not None:
            ev[0].record()
        w8.gemm_dequant(self.qx, self.sx, self.qw, self.sw, self.x.dtype, self.y)
        if ev is not None:
            ev[1].record()


def steady_state(run_step, step_i, n, every, te, layers, gemm_avg, ops_per_step, ops_per_launch):
    """The same step, n more times right after the timed ones, with no pause
    in between, timed in blocks of n // 4 steps.  After an idle spell the GPU
    runs at a lower clock for the first 15-20 ms of load; the last block shows
    the step at the settled clock, a check on the timed steps.
    Informational: `value` and `roofline` come from the timed steps alone."""
    import torch

    blk = max(1, n // 4)
    evs = {k: [(te.create(), te.create()) for _ in layers]
           for k in range(3 * blk, 4 * blk) if k % every == 0}
    ms = []
    for b in range(4):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(b * blk, (b + 1) * blk):
            run_step(step_i + k, evs.get(k))
        torch.cuda.synchronize()
        ms.append((time.perf_counter() - t0) / blk * 1e3)
    avg = gemm_avg(evs)
    return {
        "steps": 4 * blk,
        "ms_per_step_by_block": [round(t, 4) for t in ms],
        "last_block": {
            "ms_per_step": round(ms[-1], 4),
            "TOPS": round(ops_per_step / (ms[-1] * 1e-3) / 1e12, 3),
            "gemm_avg_launch_us": round(avg * 1e6, 3),
            "gemm_frac_mfma": round(ops_per_launch / avg / 1e12 / PEAK_INT8_TOPS, 4),
        },
        "note": "informational, not `value`: the same step continued without pause after the "
                "timed steps, in four blocks; the last block at the settled clock",
    }


def graph_time(fn, n):
    """Mean seconds per call of fn(i), i < n, from one replay of a HIP graph
    that holds the n calls (after one eager call and one warm-up replay), so
    that the host's launch cost, larger than the small kernels here, does not
    enter."""
    import torch

    fn(0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(n):
            fn(i)
    graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    graph.replay()
    b.record()
    b.synchronize()
    return a.elapsed_time(b) / n * 1e-3


def rotation(t, min_total=512 << 20, cap=32):
    """t and copies of it, together at least min_total bytes: a kernel timed
    over them in turn reads HBM, not the 256 MB last-level cache."""
    n = max(1, min(cap, -(-min_total // (t.numel() * t.element_size()))))
    return [t] + [t.clone() for _ in range(n - 1)]


def kernel_breakdown(layers, reps, lean=False):
    """Per-kernel mean durations, each kernel type timed alone (graph_time).
    The bandwidth-bound kernels rotate over copies of their input (rotation).
    lean: only the path's own kernels and the dense 16-bit product (no norm
    folds, no FP8 variant)."""
    import torch

    timed = graph_time

    def hbm(t, by):
        return dict(us=t * 1e6, GBs=by / t / 1e9, frac_hbm=by / t / 1e9 / PEAK_HBM_GBS)

    w8 = layers[0].w8
    out = {}
    for L in layers:
        d = {}
        cal = L.cal if sum(c.numel() * 2 for c in L.cal) >= (512 << 20) else rotation(L.cal[0])
        nb = len(cal)
        t = timed(lambda i: w8.channel_amax(cal[i % nb], L.amax_x), reps)
        d["channel_amax_calib"] = hbm(t, cal[0].numel() * 2)
        ws = rotation(L.w)
        xs = rotation(L.x)
        nw, nx = len(ws), len(xs)
        t = timed(lambda i: w8.channel_amax(ws[i % nw], L.amax_w), reps)
        d["channel_amax_weight"] = hbm(t, L.w.numel() * 2)
        # the step's form: one calibration batch, the weight maxima and s in one launch
        t = timed(lambda i: w8.calibrate_smooth(cal[i % nb], ws[i % nw], L.alpha, L.amax_x,
                                                L.amax_w, L.s, L.inv_s, L.scratch), reps)
        d["calibrate_smooth"] = hbm(t, cal[0].numel() * 2 + L.w.numel() * 2)
        t = timed(lambda i: w8.scale_quant_rows(ws[i % nw], L.s, L.qw, L.sw), reps)
        d["fold_quant_weight"] = hbm(t, L.w.numel() * 3 + 4 * (L.N + L.K))
        t = timed(lambda i: w8.scale_quant_rows(xs[i % nx], L.inv_s, L.qx, L.sx), reps)
        d["smooth_quant_act"] = hbm(t, L.x.numel() * 3 + 4 * (L.M + L.K))
        # the step's form: both in one launch
        t = timed(lambda i: w8.scale_quant_pair(ws[i % nw], L.s, xs[i % nx], L.inv_s, L.qw, L.sw,
                                                L.qx, L.sx), reps)
        d["quant_pair"] = hbm(t, (L.w.numel() + L.x.numel()) * 3 + 4 * (L.N + L.M + 2 * L.K))
        t = timed(lambda i: w8.gemm_dequant(L.qx, L.sx, L.qw, L.sw, L.x.dtype, L.y), reps)
        ops = L.gemm_ops()
        d["gemm_dequant"] = dict(us=t * 1e6, TOPS=ops / t / 1e12, frac_mfma=ops / t / 1e12 / PEAK_INT8_TOPS)
        t16 = timed(lambda i: w8.gemm_float(L.x, L.w, L.y), reps)
        d["dense16_gemm"] = dict(us=t16 * 1e6, TFLOPS=ops / t16 / 1e12,
                                 frac_mfma=ops / t16 / 1e12 / PEAK_DENSE16_TFLOPS)
        if lean:
            del ws, xs
            out[f"{L.name}_{L.K}x{L.N}"] = {k: {kk: round(vv, 4) for kk, vv in v.items()}
                                            for k, v in d.items()}
            continue
        # the smoothing folded into the RMS norm in front of the layer (x taken as the norm's input)
        g = w8.fold_norm_weight(torch.ones(L.K, dtype=torch.float32, device=L.x.device), L.inv_s)
        t = timed(lambda i: w8.rmsnorm_quant_rows(xs[i % nx], g, 1e-5, L.qx, L.sx), reps)
        d["rmsnorm_smooth_quant_act"] = hbm(t, L.x.numel() * 3 + 4 * (L.M + L.K))
        if L.x.dtype == torch.float16:
            # the same fold into a LayerNorm (OPT-family decoders), fp16 only
            b = w8.fold_norm_weight(torch.zeros(L.K, dtype=torch.float32, device=L.x.device), L.inv_s)
            t = timed(lambda i: w8.layernorm_quant_rows(xs[i % nx], g, b, 1e-5, L.qx, L.sx), reps)
            d["layernorm_smooth_quant_act"] = hbm(t, L.x.numel() * 3 + 4 * (L.M + 2 * L.K))
        # FP8 (E4M3) form of the same layer: codes from the same smoothed tensors
        qw8, sw8 = w8.scale_quant_rows_e4m3(L.w, L.s)
        qx8, sx8 = w8.scale_quant_rows_e4m3(L.x, L.inv_s)
        t = timed(lambda i: w8.scale_quant_rows_e4m3(xs[i % nx], L.inv_s, qx8, sx8), reps)
        d["smooth_quant_act_e4m3"] = hbm(t, L.x.numel() * 3 + 4 * (L.M + L.K))
        t8 = timed(lambda i: w8.gemm_dequant_e4m3(qx8, sx8, qw8, sw8, L.x.dtype, L.y), reps)
        d["gemm_dequant_e4m3"] = dict(us=t8 * 1e6, TFLOPS=ops / t8 / 1e12,
                                      frac_mfma=ops / t8 / 1e12 / PEAK_FP8_TFLOPS)
        del qw8, sw8, qx8, sx8, ws, xs
        out[f"{L.name}_{L.K}x{L.N}"] = {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in d.items()}
    # W8A8 vs the dense 16-bit product on the same shapes, summed over the layers
    t_w8 = sum(v["gemm_dequant"]["us"] for v in out.values())
    t_q = sum(v["smooth_quant_act"]["us"] for v in out.values())
    t_16 = sum(v["dense16_gemm"]["us"] for v in out.values())
    out["w8a8_vs_dense16"] = {"gemm_speedup": round(t_16 / t_w8, 3),
                              "gemm_plus_act_quant_speedup": round(t_16 / (t_w8 + t_q), 3)}
    if not lean:
        t_8 = sum(v["gemm_dequant_e4m3"]["us"] for v in out.values() if "gemm_dequant_e4m3" in v)
        out["e4m3_vs_int8"] = {"gemm_time_ratio": round(t_8 / t_w8, 3)}
    return out


def calibration_volume(wl, layers, reps):
    """Step 1 at the calibration volume the page recommends (512 samples of
    2048 tokens, 1,048,576 tokens per layer): (a) the streaming form, one call
    per 2048-token batch as the batches arrive, 512 calls cycling over the
    layer's distinct batches (at least 420 MB, past the 256 MB last-level
    cache), timed from a captured graph; (b) one call per slice of at least
    1 GiB of tokens, two distinct slices in turn."""
    import torch

    from w8a8_int8_amd import synth

    w8 = layers[0].w8
    out = {}
    for li, L in enumerate(layers):
        if L.name not in ("qkv", "down"):
            continue
        nb = len(L.cal)
        t = graph_time(lambda i: w8.channel_amax(L.cal[i % nb], L.amax_x), 512)
        by = L.cal[0].numel() * 2
        d = {"per_batch_stream": dict(batches=512, distinct_batches=nb, us_per_batch=round(t * 1e6, 3),
                                      total_ms=round(t * 512e3, 3), GBs=round(by / t / 1e9, 1),
                                      frac_hbm=round(by / t / 1e9 / PEAK_HBM_GBS, 4))}
        rows = max(wl.cal_batch, -(-(1 << 30) // (2 * L.K)))
        rows = -(-rows // wl.cal_batch) * wl.cal_batch
        slices = [synth.calibration(wl, li, rows, chunk=10_000 + j, device=L.x.device)
                  for j in range(2)]
        t = graph_time(lambda i: w8.channel_amax(slices[i % 2], L.amax_x), max(4, reps // 4))
        by = slices[0].numel() * 2
        d["one_call_per_slice"] = dict(tokens=rows, GB=round(by / 1e9, 3), us=round(t * 1e6, 2),
                                       GBs=round(by / t / 1e9, 1),
                                       frac_hbm=round(by / t / 1e9 / PEAK_HBM_GBS, 4),
                                       full_set_ms=round(t * (wl.cal_tokens / rows) * 1e3, 3))
        del slices
        torch.cuda.empty_cache()
        out[f"{L.name}_{L.K}"] = d
    return out


def other_workload(name, alpha, reps, dev):
    """The per-kernel pass (lean) on another workload, or its few-token sweep."""
    import torch

    from w8a8_int8_amd import synth

    wl = synth.WORKLOADS[name]
    layers = [Layer(wl, li, 1, alpha, dev) for li in range(len(wl.layers))]
    for L in layers:
        L.step(0)
    torch.cuda.synchronize()
    if wl.M[0] <= 32:
        res = {"decode_sweep": decode_sweep(wl, layers, max(reps, 20))}
    else:
        res = {"M": wl.M[0], "act_dtype": wl.dtype, **kernel_breakdown(layers, reps, lean=True)}
    del layers
    torch.cuda.empty_cache()
    return res


def decode_sweep(wl, layers, reps):
    """Every token count of a few-token workload through each layer: the
    runtime forward (smooth + quant, then the split-K GEMM) and the unsplit
    GEMM kernel alone, against the HBM roofline (both stream the INT8 weight
    once).  The calls rotate over copies of the weight totalling >= 512 MB, so
    that the 256 MB last-level cache cannot serve it, and run from a captured
    HIP graph, so that host-side launch cost does not enter."""
    import torch

    w8 = layers[0].w8
    out = {}
    for L in layers:
        copies = max(2, min(16, -(-(512 << 20) // (L.N * L.K))))
        qws = [L.qw] + [L.qw.clone() for _ in range(copies - 1)]
        for M in wl.M:
            x = L.x_all[:M]
            y = torch.empty((M, L.N), dtype=L.x.dtype, device=L.x.device)
            ws = torch.empty(max(w8.linear_workspace_bytes(M, L.N, L.K), 1), dtype=torch.uint8,
                             device=L.x.device)
            qx = ws[:M * L.K].view(torch.int8).view(M, L.K)
            off = (M * L.K + 255) // 256 * 256
            sx = ws[off:off + 4 * M].view(torch.float32)
            w8.linear(x, L.inv_s, L.qw, L.sw, y, ws)

            run = lambda fn: graph_time(fn, reps)  # noqa: E731

            t_lin = run(lambda i: w8.linear(x, L.inv_s, qws[i % copies], L.sw, y, ws))
            t_q = run(lambda i: w8.scale_quant_rows(x, L.inv_s, qx, sx))
            t_g = run(lambda i: w8.gemm_dequant(qx, sx, qws[i % copies], L.sw, L.x.dtype, y))
            by = L.gemm_bytes(M)
            out[f"{L.name}_{L.K}x{L.N}_M{M}"] = {
                "linear_us": round(t_lin * 1e6, 3),
                "act_quant_us": round(t_q * 1e6, 3),
                "linear_gemm_GBs": round(by / (t_lin - t_q) / 1e9, 1) if t_lin > t_q else None,
                "unsplit_gemm_us": round(t_g * 1e6, 3),
                "unsplit_gemm_GBs": round(by / t_g / 1e9, 1),
            }
        del qws
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, layers, alpha, min_seconds=10.0):
    """The CPU oracle, as it stands, over one step of the same workload."""
    import oracle
    from w8a8_int8_amd import synth

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    dname = wl.dtype
    host = [(synth.to_numpy_bits(L.cal[0]), synth.to_numpy_bits(L.w), synth.to_numpy_bits(L.x))
            for L in layers]
    ops = 0.0
    steps = 0
    t0 = time.perf_counter()
    # whole steps until at least min_seconds of host work (bounded: <= 8 steps)
    while steps < 8 and (steps == 0 or time.perf_counter() - t0 < min_seconds):
        for (xc, w, x), L in zip(host, layers):
            ax = oracle.channel_amax(xc, dname)
            p = oracle.prepare_weight(w, dname, ax, alpha)
            oracle.linear(x, dname, p["inv_s"], p["qw"], p["sw"])
            ops += L.gemm_ops()
        steps += 1
    dt = time.perf_counter() - t0
    return {"value": round(ops / dt / 1e12, 6), "unit": "TOPS", "cores": int(threads),
            "affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
            "threads_note": "the exact integer product runs as an fp64 BLAS product on `cores` "
                            "threads; the other oracle steps are numpy on one thread",
            "kind": "oracle", "seconds": round(dt, 3), "steps": steps,
            "sample": (f"{steps} full step(s) of {wl.name} on the host: for each of the "
                       f"{len(layers)} layers, amax over one {wl.cal_batch}-token calibration "
                       f"batch, weight amax + smoothing factors + fold/quant, and the forward "
                       f"(smooth+quant, exact INT8 GEMM, dequant) at M={wl.M[0]}")}


def ceilings(dev):
    """The GPU's practical ceilings, from the probes in libw8a8_probe.so (not
    part of the path): read-only streaming and a plain copy over buffers past
    the 256 MB last-level cache, and back-to-back INT8 MFMAs from registers
    with each block's shader clock, for three operand patterns."""
    import ctypes

    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "w8a8_int8_amd", "libw8a8_probe.so"))
    vp, sz, ci = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.w8a8probe_read.argtypes = [vp, sz, vp, ci, ci, vp]
    lib.w8a8probe_copy.argtypes = [vp, vp, sz, ci, vp]
    lib.w8a8probe_mfma.argtypes = [ci, ci, ci, ci, ci, ci, vp, vp, vp]
    st = lambda: torch.cuda.current_stream().cuda_stream  # noqa: E731
    out = {}
    n = 2 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    src.view(torch.int32).copy_(torch.arange(n // 4, dtype=torch.int32, device=dev))
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    reads = {}
    for chunked in (0, 1):
        for blocks in (1024, 2048, 4096, 8192, 16384):
            t = graph_time(lambda i: lib.w8a8probe_read(src.data_ptr(), n, sink.data_ptr(), blocks,
                                                        chunked, st()), 10)
            reads[("chunked_" if chunked else "grid_stride_") + str(blocks)] = round(n / t / 1e9, 1)
    out["read_only_stream_GBs"] = {"bytes": n, "by_layout_and_blocks": reads,
                                   "best": max(reads.values())}
    # the same read at the sizes of single kernels of the path (rotated over
    # copies past the last-level cache), the best layout and block count:
    # a fixed cost per launch dominates the small sizes
    sizes = {}
    for mb in (16, 25, 50, 100, 200, 400, 800):
        nb = mb << 20
        parts = max(2, -(-(768 << 20) // nb))
        bufs = [src[(j % (n // nb)) * nb:(j % (n // nb) + 1) * nb] for j in range(min(parts, n // nb))]
        best = 0.0
        for blocks in (1024, 2048, 4096, 8192):
            t = graph_time(lambda i: lib.w8a8probe_read(bufs[i % len(bufs)].data_ptr(), nb, sink.data_ptr(),
                                                        blocks, 1, st()), 20)
            best = max(best, nb / t / 1e9)
        sizes[f"{mb}MiB"] = round(best, 1)
    out["read_only_stream_GBs"]["by_size_best"] = sizes
    # the same read of one buffer over and over (its second and later reads
    # can come from the 256 MB last-level cache) beside the rotated read, at
    # the sizes of the path's weights: what a second pass over W could gain
    llc = {}
    for mb in (64, 100, 150, 200, 300):
        nb = mb << 20
        nbuf = n // nb
        t_same = graph_time(lambda i: lib.w8a8probe_read(src.data_ptr(), nb, sink.data_ptr(), 4096, 1,
                                                         st()), 20)
        t_rot = graph_time(lambda i: lib.w8a8probe_read(src[(i % nbuf) * nb:].data_ptr(), nb,
                                                        sink.data_ptr(), 4096, 1, st()), 20)
        llc[f"{mb}MiB"] = {"same_buffer": round(nb / t_same / 1e9, 1), "rotated": round(nb / t_rot / 1e9, 1)}
    out["read_only_stream_GBs"]["reread_vs_rotated_4096_blocks"] = llc
    half = n // 2
    dst = torch.empty(half, dtype=torch.uint8, device=dev)
    copies = {}
    for blocks in (2048, 4096, 8192, 16384):
        t = graph_time(lambda i: lib.w8a8probe_copy(src.data_ptr(), dst.data_ptr(), half, blocks, st()), 10)
        copies[str(blocks)] = round(2 * half / t / 1e9, 1)
    t = graph_time(lambda i: dst.copy_(src[:half]), 10)
    out["copy_GBs"] = {"bytes_each_way": half, "by_blocks": copies, "best": max(copies.values()),
                       "torch_copy": round(2 * half / t / 1e9, 1)}
    del src, dst
    blocks = 256
    clocks = torch.zeros(2 * blocks, dtype=torch.int64, device=dev)
    mf = {}
    for shape, waves, chains in ((0, 8, 4), (0, 8, 8), (0, 4, 8), (1, 8, 4), (1, 8, 8), (1, 8, 16)):
        per = 65536.0 if shape == 0 else 32768.0  # int ops per instruction
        # the same int ops per SIMD in every case
        iters = int(20000 * 4 // chains * 8 // waves * (65536.0 / per))
        name = "32x32x32" if shape == 0 else "16x16x64"
        for pattern, label in ((0, "zero_operands"), (1, "random_bytes"), (2, "codes_below_32")):
            lib.w8a8probe_mfma(blocks, 200, pattern, waves, chains, shape, clocks.data_ptr(),
                               sink.data_ptr(), st())
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            lib.w8a8probe_mfma(blocks, iters, pattern, waves, chains, shape, clocks.data_ptr(),
                               sink.data_ptr(), st())
            b.record()
            b.synchronize()
            t = a.elapsed_time(b) * 1e-3
            c = clocks.view(blocks, 2).double().cpu()
            ghz = (c[:, 0] / c[:, 1] * 0.1).median().item()  # s_memrealtime ticks at 100 MHz
            ops = blocks * waves * iters * chains * per
            mf[f"{name}_{waves}waves_{chains}chains_{label}"] = {
                "POPS": round(ops / t / 1e15, 3), "frac_of_5_POPS": round(ops / t / 1e15 / 5.0, 4),
                "clock_GHz": round(ghz, 3),
                "frac_of_clock_scaled_peak": round(ops / t / 1e15 / (5.0 * ghz / 2.4), 4)}
    out["mfma_i8_only"] = {"blocks": blocks, **mf}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by rows/columns without collectives on the hot path; "
              "see the design notes)", file=sys.stderr)
        sys.exit(2)
    import torch

    import w8a8_int8_amd as w8
    from w8a8_int8_amd import _lib, synth

    _lib.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    if args.ceilings:
        print(json.dumps({"ceilings": ceilings(dev)}), flush=True)
        return
    wl = synth.WORKLOADS[args.workload]
    n_batches = max(1, min(args.steps + args.warmup, wl.cal_tokens // wl.cal_batch))
    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    layers = [Layer(wl, li, n_batches, args.alpha, dev) for li in range(len(wl.layers))]

    def run_step(i, evs_row=None):
        # every layer's calibration batch, weight maxima and smoothing factors
        # in one launch, then per layer the two quantizations and the GEMM
        w8.calibrate_smooth_layers([L.calib_args(i) for L in layers], args.alpha)
        for li, L in enumerate(layers):
            L.quantize_forward(None if evs_row is None else evs_row[li])

    torch.cuda.synchronize()
    print(f"[bench] {wl.name}: {len(layers)} layers, M={wl.M[0]}, buffers ready", file=sys.stderr,
          flush=True)

    # The per-kernel pass (each kernel of the workload timed alone, a few
    # seconds of GPU work) runs before the warm-up steps.  After an idle spell
    # the GPU needs 15-20 ms of continuous load to reach its working clock,
    # more than the warm-up steps take, so the timed steps would otherwise sit
    # in that ramp.  The timing events are created before the warm-up steps
    # too, so that no host work leaves the GPU idle between warm-up and timed
    # steps (an idle gap of 10 ms or more lets the clock drop back).
    kernels = kernel_breakdown(layers, args.kernel_reps)
    torch.cuda.synchronize()
    print("[bench] per-kernel pass done", file=sys.stderr, flush=True)
    te = TimingEvents()
    every = max(1, args.event_every)
    ev_steps = [k for k in range(args.steps) if k % every == 0]
    evs = {k: [(te.create(), te.create()) for _ in layers] for k in ev_steps}

    step_i = 0
    for _ in range(args.warmup):
        run_step(step_i)
        step_i += 1
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        run_step(step_i, evs.get(k))
        step_i += 1
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    ms_per_step = elapsed / args.steps * 1e3
    ops_per_step = sum(L.gemm_ops() for L in layers)
    value = ops_per_step / (elapsed / args.steps) / 1e12

    def gemm_avg(evs):
        gemm_s = [sum(a.elapsed_time(b) for a, b in row) * 1e-3 for row in evs.values()]
        for row in evs.values():
            for a, b in row:
                a.destroy()
                b.destroy()
        return sum(gemm_s) / (len(gemm_s) * len(layers))

    gemm_launch_avg = gemm_avg(evs)
    ops_per_launch = ops_per_step / len(layers)
    achieved = ops_per_launch / gemm_launch_avg / 1e12
    # few tokens (decode): the GEMM streams the weight and is HBM-bound
    decode = wl.M[0] <= 32
    # the kernel the launcher picks for that token count (one or two tokens:
    # whole weight rows streamed; up to 32: weight pieces transposed in LDS)
    decode_kernel = "k_gemv_rows" if wl.M[0] <= 2 else "k_gemm_fewtok"
    steady = None
    if args.steady_steps > 0 and not decode:
        steady = steady_state(run_step, step_i, args.steady_steps, every, te, layers, gemm_avg,
                              ops_per_step, ops_per_launch)
        step_i += args.steady_steps
    bytes_per_launch = sum(L.gemm_bytes() for L in layers) / len(layers)
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)

    # the step's form of the calibration: every layer in one launch (timed
    # here, after the timed steps: memory-bound work just before the warm-up
    # steps would leave them at a lower clock)
    t = graph_time(lambda i: w8.calibrate_smooth_layers([L.calib_args(i) for L in layers], args.alpha),
                   args.kernel_reps)
    by = sum(L.cal[0].numel() * 2 + L.w.numel() * 2 for L in layers)
    kernels["calibrate_smooth_layers"] = {
        "us": round(t * 1e6, 3), "GBs": round(by / t / 1e9, 1),
        "frac_hbm": round(by / t / 1e9 / PEAK_HBM_GBS, 4),
        "one_launch_per_layer_us": round(sum(v["calibrate_smooth"]["us"] for v in kernels.values()
                                             if isinstance(v, dict) and "calibrate_smooth" in v), 3)}
    if decode:
        kernels["decode_sweep"] = decode_sweep(wl, layers, max(args.kernel_reps, 20))
    else:
        kernels["calibration_volume"] = calibration_volume(wl, layers, args.kernel_reps)
    print("[bench] decode sweep / calibration volume done", file=sys.stderr, flush=True)
    others = {}
    for name in [n for n in args.other_workloads.split(",") if n and n != wl.name]:
        others[name] = other_workload(name, args.alpha, args.kernel_reps, dev)
        print(f"[bench] per-kernel pass of {name} done", file=sys.stderr, flush=True)

    traffic = pmc_traffic(wl.name)
    rec = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic (seeded outlier-bearing activations, N(0, sigma) weights)",
        "config": {
            "workload": wl.name,
            "M": wl.M[0],
            "layers": [f"{L.name}:{L.K}->{L.N}" for L in layers],
            "calibration_tokens_per_step": wl.cal_batch,
            "alpha": args.alpha,
            "act_dtype": wl.dtype,
        },
        "roofline": {
            "kernel": "gemm_dequant (k_gemm_i8)",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_INT8_TOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_INT8_TOPS, 4),
            "traffic": traffic,
            "ops_per_launch": ops_per_launch,
            "avg_launch_us": round(gemm_launch_avg * 1e6, 3),
            "event_steps": len(ev_steps),
        } if not decode else {
            "kernel": f"gemm_dequant ({decode_kernel})",
            "bound": "hbm",
            "achieved": round(bytes_per_launch / gemm_launch_avg / 1e9, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(bytes_per_launch / gemm_launch_avg / 1e9 / PEAK_HBM_GBS, 4),
            "traffic": pmc_traffic(wl.name, decode_kernel.replace("k_", "")),
            "bytes_per_launch": bytes_per_launch,
            "avg_launch_us": round(gemm_launch_avg * 1e6, 3),
            "event_steps": len(ev_steps),
        },
        "kernels": kernels,
    }
    if steady is not None:
        rec["steady_state"] = steady
    if others:
        rec["other_workloads"] = others
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(wl, layers, args.alpha)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
