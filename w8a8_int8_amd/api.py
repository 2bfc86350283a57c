"""Python binding of libw8a8 over torch tensors.

Argument marshalling only: each function checks devices, dtypes and
contiguity, allocates missing outputs with torch (device memory plumbing) and
calls the C entry point of the same name on the current HIP stream.  Every
step of the computation runs in the library's HIP kernels; there is no
fallback path.

Names follow the usage example on the jisaku.com glossary page "SmoothQuant"
(section "インストール・使用例"): ``channel_amax`` collects the activation
statistics (``get_act_scales``), ``smooth_factors`` + ``prepare_weight``
smooth and quantize a layer (``smooth_lm``, ``quantize_model``), and
``linear`` runs the W8A8 forward.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib

_DT = {torch.float16: _lib.W8A8_F16, torch.bfloat16: _lib.W8A8_BF16}


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.data_ptr()


def _dev(*ts: torch.Tensor) -> None:
    for t in ts:
        if t.device.type != "cuda":
            raise ValueError(f"expected a GPU tensor, got one on {t.device}")
        if not t.is_contiguous():
            raise ValueError("expected a contiguous tensor")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"expected float16 or bfloat16, got {t.dtype}")
    return _DT[t.dtype]


def _need(t: torch.Tensor, dtype: torch.dtype, shape) -> None:
    if t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"expected {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


def channel_amax(x: torch.Tensor, amax: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Fold max|x| over the rows of ``x`` (rows x cols) into ``amax`` (fp32[cols]).

    A new ``amax`` starts at zero; passing the previous result continues a
    running maximum over calibration batches.
    """
    _dev(x)
    rows, cols = x.shape
    if amax is None:
        amax = torch.zeros(cols, dtype=torch.float32, device=x.device)
    _dev(amax)
    _need(amax, torch.float32, (cols,))
    lib = _lib.load()
    _lib.check("w8a8_channel_amax", lib.w8a8_channel_amax(
        _ptr(x), _dtype_code(x), rows, cols, _ptr(amax), _stream()))
    return amax


def smooth_factors(amax_x: torch.Tensor, amax_w: torch.Tensor, alpha: float,
                   s: Optional[torch.Tensor] = None, inv_s: Optional[torch.Tensor] = None):
    """(s, inv_s): s_j = amax_x[j]**alpha / amax_w[j]**(1 - alpha), inv_s = 1 / s."""
    _dev(amax_x, amax_w)
    K = amax_x.shape[0]
    _need(amax_x, torch.float32, (K,))
    _need(amax_w, torch.float32, (K,))
    s = torch.empty(K, dtype=torch.float32, device=amax_x.device) if s is None else s
    inv_s = torch.empty(K, dtype=torch.float32, device=amax_x.device) if inv_s is None else inv_s
    _dev(s, inv_s)
    lib = _lib.load()
    _lib.check("w8a8_smooth_factors", lib.w8a8_smooth_factors(
        _ptr(amax_x), _ptr(amax_w), K, float(alpha), _ptr(s), _ptr(inv_s), _stream()))
    return s, inv_s


def calibrate_smooth_scratch(K: int, device) -> torch.Tensor:
    """Zero-filled scratch for calibrate_smooth over K channels (reusable: every
    call leaves it zero)."""
    n = _lib.load().w8a8_calibrate_smooth_scratch_bytes(K)
    if n == 0:
        raise ValueError(f"no calibrate_smooth scratch for K = {K}")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def calibrate_smooth(x_cal: Optional[torch.Tensor], w: torch.Tensor, alpha: float,
                     amax_x: torch.Tensor, amax_w: Optional[torch.Tensor] = None,
                     s: Optional[torch.Tensor] = None, inv_s: Optional[torch.Tensor] = None,
                     scratch: Optional[torch.Tensor] = None):
    """One launch of: channel_amax(x_cal, amax_x) (skipped for None), amax_w =
    channel max of the N x K weight ``w``, and smooth_factors.  Returns
    (amax_w, s, inv_s)."""
    _dev(w, amax_x)
    N, K = w.shape
    cal_rows = 0 if x_cal is None else x_cal.shape[0]
    if x_cal is not None:
        _dev(x_cal)
        _need(x_cal, w.dtype, (cal_rows, K))
    _need(amax_x, torch.float32, (K,))
    f32 = dict(dtype=torch.float32, device=w.device)
    amax_w = torch.empty(K, **f32) if amax_w is None else amax_w
    s = torch.empty(K, **f32) if s is None else s
    inv_s = torch.empty(K, **f32) if inv_s is None else inv_s
    scratch = calibrate_smooth_scratch(K, w.device) if scratch is None else scratch
    _dev(amax_w, s, inv_s, scratch)
    for t in (amax_w, s, inv_s):
        _need(t, torch.float32, (K,))
    _need(scratch, torch.uint8, (scratch.numel(),))
    lib = _lib.load()
    _lib.check("w8a8_calibrate_smooth", lib.w8a8_calibrate_smooth(
        _ptr(x_cal), cal_rows, _ptr(w), N, _dtype_code(w), K, float(alpha), _ptr(amax_x),
        _ptr(amax_w), _ptr(s), _ptr(inv_s), _ptr(scratch), scratch.numel(), _stream()))
    return amax_w, s, inv_s


def calibrate_smooth_layers(layers, alpha: float) -> None:
    """calibrate_smooth for several layers in one launch (up to 8 per launch):
    ``layers`` is a sequence of (x_cal or None, w, amax_x, amax_w, s, inv_s,
    scratch) with every tensor given, all of one dtype; the outputs are
    written in place, the same bits as one calibrate_smooth per layer."""
    arr = (_lib.CalibLayer * max(1, len(layers)))()
    dtype = None
    for i, (x_cal, w, amax_x, amax_w, s, inv_s, scratch) in enumerate(layers):
        _dev(w, amax_x, amax_w, s, inv_s, scratch)
        N, K = w.shape
        dtype = w.dtype if dtype is None else dtype
        if w.dtype != dtype:
            raise TypeError("calibrate_smooth_layers: every layer must have the same dtype")
        cal_rows = 0 if x_cal is None else x_cal.shape[0]
        if x_cal is not None:
            _dev(x_cal)
            _need(x_cal, w.dtype, (cal_rows, K))
        for t in (amax_x, amax_w, s, inv_s):
            _need(t, torch.float32, (K,))
        _need(scratch, torch.uint8, (scratch.numel(),))
        arr[i] = _lib.CalibLayer(_ptr(x_cal), cal_rows, _ptr(w), N, K, float(alpha), _ptr(amax_x),
                                 _ptr(amax_w), _ptr(s), _ptr(inv_s), _ptr(scratch), scratch.numel())
    lib = _lib.load()
    code = _dtype_code(layers[0][1]) if layers else 0
    _lib.check("w8a8_calibrate_smooth_layers", lib.w8a8_calibrate_smooth_layers(
        ctypes.addressof(arr), len(layers), code, _stream()))


def scale_quant_rows(x: torch.Tensor, col_scale: torch.Tensor,
                     q: Optional[torch.Tensor] = None, row_scale: Optional[torch.Tensor] = None):
    """(q int8 rows x cols, row_scale fp32[rows]) of x * col_scale per row."""
    _dev(x, col_scale)
    rows, cols = x.shape
    _need(col_scale, torch.float32, (cols,))
    q = torch.empty((rows, cols), dtype=torch.int8, device=x.device) if q is None else q
    row_scale = (torch.empty(rows, dtype=torch.float32, device=x.device)
                 if row_scale is None else row_scale)
    _dev(q, row_scale)
    _need(q, torch.int8, (rows, cols))
    _need(row_scale, torch.float32, (rows,))
    lib = _lib.load()
    _lib.check("w8a8_scale_quant_rows", lib.w8a8_scale_quant_rows(
        _ptr(x), _dtype_code(x), rows, cols, _ptr(col_scale), _ptr(q), _ptr(row_scale),
        _stream()))
    return q, row_scale


def scale_quant_pair(w: torch.Tensor, s: torch.Tensor, x: torch.Tensor, inv_s: torch.Tensor,
                     qw: Optional[torch.Tensor] = None, sw: Optional[torch.Tensor] = None,
                     qx: Optional[torch.Tensor] = None, sx: Optional[torch.Tensor] = None):
    """(qw, sw, qx, sx): scale_quant_rows(w, s) and scale_quant_rows(x, inv_s) in one launch."""
    _dev(w, s, x, inv_s)
    N, K = w.shape
    M = x.shape[0]
    if x.dtype != w.dtype:
        raise TypeError(f"w is {w.dtype} but x is {x.dtype}")
    _need(x, w.dtype, (M, K))
    _need(s, torch.float32, (K,))
    _need(inv_s, torch.float32, (K,))
    qw = torch.empty((N, K), dtype=torch.int8, device=w.device) if qw is None else qw
    sw = torch.empty(N, dtype=torch.float32, device=w.device) if sw is None else sw
    qx = torch.empty((M, K), dtype=torch.int8, device=w.device) if qx is None else qx
    sx = torch.empty(M, dtype=torch.float32, device=w.device) if sx is None else sx
    _dev(qw, sw, qx, sx)
    _need(qw, torch.int8, (N, K))
    _need(sw, torch.float32, (N,))
    _need(qx, torch.int8, (M, K))
    _need(sx, torch.float32, (M,))
    lib = _lib.load()
    _lib.check("w8a8_scale_quant_pair", lib.w8a8_scale_quant_pair(
        _ptr(w), N, _ptr(s), _ptr(qw), _ptr(sw), _ptr(x), M, _ptr(inv_s), _ptr(qx), _ptr(sx),
        _dtype_code(w), K, _stream()))
    return qw, sw, qx, sx


def fold_norm_weight(gamma: torch.Tensor, inv_s: torch.Tensor,
                     g: Optional[torch.Tensor] = None) -> torch.Tensor:
    """g = gamma * inv_s (fp32): the smoothing folded into an RMS norm's weight."""
    _dev(gamma, inv_s)
    K = gamma.shape[0]
    _need(gamma, torch.float32, (K,))
    _need(inv_s, torch.float32, (K,))
    g = torch.empty(K, dtype=torch.float32, device=gamma.device) if g is None else g
    _dev(g)
    _need(g, torch.float32, (K,))
    lib = _lib.load()
    _lib.check("w8a8_fold_norm_weight", lib.w8a8_fold_norm_weight(
        _ptr(gamma), _ptr(inv_s), K, _ptr(g), _stream()))
    return g


def rmsnorm_quant_rows(h: torch.Tensor, g: torch.Tensor, eps: float,
                       q: Optional[torch.Tensor] = None,
                       row_scale: Optional[torch.Tensor] = None):
    """Per-token INT8 of RMSNorm(h) with the folded weight g = gamma * inv_s.

    Returns (q int8 rows x cols, row_scale fp32[rows]); q * row_scale[:, None]
    approximates h / rms(h) * gamma * inv_s.
    """
    _dev(h, g)
    rows, cols = h.shape
    _need(g, torch.float32, (cols,))
    q = torch.empty((rows, cols), dtype=torch.int8, device=h.device) if q is None else q
    row_scale = (torch.empty(rows, dtype=torch.float32, device=h.device)
                 if row_scale is None else row_scale)
    _dev(q, row_scale)
    _need(q, torch.int8, (rows, cols))
    _need(row_scale, torch.float32, (rows,))
    lib = _lib.load()
    _lib.check("w8a8_rmsnorm_quant_rows", lib.w8a8_rmsnorm_quant_rows(
        _ptr(h), _dtype_code(h), rows, cols, _ptr(g), float(eps), _ptr(q), _ptr(row_scale),
        _stream()))
    return q, row_scale


def fold_layernorm(gamma: torch.Tensor, beta: torch.Tensor, inv_s: torch.Tensor):
    """(g, b) = (gamma * inv_s, beta * inv_s) in fp32: the smoothing folded into
    a LayerNorm's affine pair (two calls of w8a8_fold_norm_weight)."""
    return fold_norm_weight(gamma, inv_s), fold_norm_weight(beta, inv_s)


def layernorm_quant_rows(x: torch.Tensor, g: torch.Tensor, b: torch.Tensor, eps: float,
                         q: Optional[torch.Tensor] = None,
                         row_scale: Optional[torch.Tensor] = None):
    """Per-token INT8 of LayerNorm(x; gamma, beta) * inv_s for fp16 x, given
    the folded g = gamma * inv_s and b = beta * inv_s (fold_layernorm).

    Returns (q int8 rows x cols, row_scale fp32[rows]); q * row_scale[:, None]
    approximates LayerNorm(x) * inv_s.
    """
    _dev(x, g, b)
    rows, cols = x.shape
    _need(g, torch.float32, (cols,))
    _need(b, torch.float32, (cols,))
    q = torch.empty((rows, cols), dtype=torch.int8, device=x.device) if q is None else q
    row_scale = (torch.empty(rows, dtype=torch.float32, device=x.device)
                 if row_scale is None else row_scale)
    _dev(q, row_scale)
    _need(q, torch.int8, (rows, cols))
    _need(row_scale, torch.float32, (rows,))
    lib = _lib.load()
    _lib.check("w8a8_layernorm_quant_rows", lib.w8a8_layernorm_quant_rows(
        _ptr(x), _dtype_code(x), rows, cols, _ptr(g), _ptr(b), float(eps), _ptr(q),
        _ptr(row_scale), _stream()))
    return q, row_scale


def gemm_i32(qa: torch.Tensor, qb: torch.Tensor, c: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Exact int32 C = qa @ qb.T for qa (M x K) and qb (N x K) int8."""
    _dev(qa, qb)
    M, K = qa.shape
    N = qb.shape[0]
    _need(qb, torch.int8, (N, K))
    _need(qa, torch.int8, (M, K))
    c = torch.empty((M, N), dtype=torch.int32, device=qa.device) if c is None else c
    _dev(c)
    _need(c, torch.int32, (M, N))
    lib = _lib.load()
    _lib.check("w8a8_gemm_i32", lib.w8a8_gemm_i32(_ptr(qa), _ptr(qb), _ptr(c), M, N, K, _stream()))
    return c


def gemm_dequant(qa: torch.Tensor, sa: torch.Tensor, qb: torch.Tensor, sb: torch.Tensor,
                 out_dtype: torch.dtype = torch.float16,
                 y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = (C * sa[:, None]) * sb[None, :] rounded to ``out_dtype``, C = qa @ qb.T."""
    _dev(qa, sa, qb, sb)
    M, K = qa.shape
    N = qb.shape[0]
    _need(qa, torch.int8, (M, K))
    _need(qb, torch.int8, (N, K))
    _need(sa, torch.float32, (M,))
    _need(sb, torch.float32, (N,))
    y = torch.empty((M, N), dtype=out_dtype, device=qa.device) if y is None else y
    _dev(y)
    _need(y, out_dtype, (M, N))
    lib = _lib.load()
    _lib.check("w8a8_gemm_dequant", lib.w8a8_gemm_dequant(
        _ptr(qa), _ptr(sa), _ptr(qb), _ptr(sb), _ptr(y), _DT[out_dtype], M, N, K, _stream()))
    return y


def scale_quant_rows_e4m3(x: torch.Tensor, col_scale: torch.Tensor,
                          q: Optional[torch.Tensor] = None,
                          row_scale: Optional[torch.Tensor] = None):
    """(q uint8 E4M3 codes rows x cols, row_scale fp32[rows]) of x * col_scale per row."""
    _dev(x, col_scale)
    rows, cols = x.shape
    _need(col_scale, torch.float32, (cols,))
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device) if q is None else q
    row_scale = (torch.empty(rows, dtype=torch.float32, device=x.device)
                 if row_scale is None else row_scale)
    _dev(q, row_scale)
    _need(q, torch.uint8, (rows, cols))
    _need(row_scale, torch.float32, (rows,))
    lib = _lib.load()
    _lib.check("w8a8_scale_quant_rows_e4m3", lib.w8a8_scale_quant_rows_e4m3(
        _ptr(x), _dtype_code(x), rows, cols, _ptr(col_scale), _ptr(q), _ptr(row_scale),
        _stream()))
    return q, row_scale


def gemm_dequant_e4m3(qa: torch.Tensor, sa: torch.Tensor, qb: torch.Tensor, sb: torch.Tensor,
                      out_dtype: torch.dtype = torch.float16,
                      y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """FP8 form of gemm_dequant: qa, qb hold E4M3 codes (uint8), fp32 accumulation."""
    _dev(qa, sa, qb, sb)
    M, K = qa.shape
    N = qb.shape[0]
    _need(qa, torch.uint8, (M, K))
    _need(qb, torch.uint8, (N, K))
    _need(sa, torch.float32, (M,))
    _need(sb, torch.float32, (N,))
    y = torch.empty((M, N), dtype=out_dtype, device=qa.device) if y is None else y
    _dev(y)
    _need(y, out_dtype, (M, N))
    lib = _lib.load()
    _lib.check("w8a8_gemm_dequant_e4m3", lib.w8a8_gemm_dequant_e4m3(
        _ptr(qa), _ptr(sa), _ptr(qb), _ptr(sb), _ptr(y), _DT[out_dtype], M, N, K, _stream()))
    return y


def gemm_float(a: torch.Tensor, b: torch.Tensor, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Dense 16-bit baseline y = a @ b.T (fp16 or bf16 operands, fp32 accumulation)."""
    _dev(a, b)
    M, K = a.shape
    N = b.shape[0]
    _need(b, a.dtype, (N, K))
    y = torch.empty((M, N), dtype=a.dtype, device=a.device) if y is None else y
    _dev(y)
    _need(y, a.dtype, (M, N))
    lib = _lib.load()
    _lib.check("w8a8_gemm_float", lib.w8a8_gemm_float(
        _ptr(a), _ptr(b), _ptr(y), _dtype_code(a), M, N, K, _stream()))
    return y


def linear_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(_lib.load().w8a8_linear_workspace_bytes(M, N, K))


def linear(x: torch.Tensor, inv_s: torch.Tensor, qw: torch.Tensor, sw: torch.Tensor,
           y: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """W8A8 forward of one smoothed linear layer: y = dequant(quant(x * inv_s) @ qw.T)."""
    _dev(x, inv_s, qw, sw)
    M, K = x.shape
    N = qw.shape[0]
    _need(inv_s, torch.float32, (K,))
    _need(qw, torch.int8, (N, K))
    _need(sw, torch.float32, (N,))
    y = torch.empty((M, N), dtype=x.dtype, device=x.device) if y is None else y
    _dev(y)
    _need(y, x.dtype, (M, N))
    need = linear_workspace_bytes(M, N, K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _dev(workspace)
    lib = _lib.load()
    _lib.check("w8a8_linear", lib.w8a8_linear(
        _ptr(x), _dtype_code(x), _ptr(inv_s), _ptr(qw), _ptr(sw), _ptr(y), M, N, K,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream()))
    return y


def linear_noalloc(x: torch.Tensor, inv_s: torch.Tensor, qw: torch.Tensor, sw: torch.Tensor,
                   y: torch.Tensor) -> torch.Tensor:
    """``linear`` with the library's static scratch instead of a workspace
    (w8a8_linear_noalloc): ``y`` is required, so nothing is allocated."""
    _dev(x, inv_s, qw, sw, y)
    M, K = x.shape
    N = qw.shape[0]
    _need(inv_s, torch.float32, (K,))
    _need(qw, torch.int8, (N, K))
    _need(sw, torch.float32, (N,))
    _need(y, x.dtype, (M, N))
    lib = _lib.load()
    _lib.check("w8a8_linear_noalloc", lib.w8a8_linear_noalloc(
        _ptr(x), _dtype_code(x), _ptr(inv_s), _ptr(qw), _ptr(sw), _ptr(y), M, N, K, _stream()))
    return y


def prepare_weight(w: torch.Tensor, amax_x: torch.Tensor, alpha: float) -> dict:
    """Offline weight path of one layer: max|W_j|, (s, inv_s), folded INT8 weight.

    ``w`` is N x K (output channel major).  Returns dict(amax_w, s, inv_s, qw, sw).
    """
    amax_w = channel_amax(w)
    s, inv_s = smooth_factors(amax_x, amax_w, alpha)
    qw, sw = scale_quant_rows(w, s)
    return dict(amax_w=amax_w, s=s, inv_s=inv_s, qw=qw, sw=sw)
