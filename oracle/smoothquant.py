"""CPU oracle of the SmoothQuant W8A8 linear-layer path.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module.  It shares no code with the HIP library
and is never on the product path.

It is the plain, slow, step-by-step definition of what the path computes,
written from the jisaku.com glossary page "SmoothQuant" (cited below by section
name); where that page is silent, each docstring states the reading taken.
Every floating-point step that decides an INT8 code is done
in IEEE fp32 (numpy float32 ufuncs: one correctly rounded operation each, no
fused multiply-add); the smoothing factors are formed in fp64 and rounded once
to fp32.  Integer results (codes, accumulators) are exact.

Layouts: activations X are M x K (token major), weights W are N x K (output
channel major, the page's W_j is column j of this array, i.e. input channel j).
bf16 data is carried as uint16 bit patterns.

Parity status of each function is stated in its docstring ("pinned by" names
the test that ties it to something other than itself).
"""
from __future__ import annotations

import math

import numpy as np

QMAX = 127  # symmetric INT8 grid [-127, 127]: -128 is never produced


# ---------------------------------------------------------------- dtypes


def widen(x, dtype: str) -> np.ndarray:
    """fp16 / bf16 storage -> float32 values (exact widening).

    ``dtype`` "f16": ``x`` is a float16 array.  "bf16": ``x`` holds uint16 bit
    patterns; the fp32 value has the same sign, exponent and the 7 stored
    mantissa bits followed by 16 zero bits.
    Pinned by tests/test_oracle_pins.py::test_widen_bf16_bits.
    """
    if dtype == "f16":
        assert x.dtype == np.float16
        return x.astype(np.float32)
    if dtype == "bf16":
        assert x.dtype == np.uint16
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(dtype)


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Written from the IEEE definition: keep the upper 16 bits of the fp32
    pattern, rounding by the discarded lower 16 bits (above half: up; exactly
    half: up only if the kept last bit is 1).  Inputs are finite.
    Pinned by tests/test_oracle_pins.py::test_round_to_bf16_*.
    """
    bits = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    hi = bits >> np.uint64(16)
    lo = bits & np.uint64(0xFFFF)
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & np.uint64(1)) == 1))
    return (hi + up.astype(np.uint64)).astype(np.uint16)


def narrow(v: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> output storage dtype (the activation dtype) with round to nearest even."""
    if dtype == "f16":
        return v.astype(np.float16)  # numpy's conversion is correctly rounded
    if dtype == "bf16":
        return round_to_bf16(v)
    raise ValueError(dtype)


# ---------------------------------------------------------------- step (1)


def channel_amax(x, dtype: str, amax=None) -> np.ndarray:
    """Per-input-channel max |x| over all rows (running max over batches).

    Section "ハイパーパラメータ α" uses max(|X_j|) (over calibration tokens,
    channel j) and max(|W_j|) (over output channels, input channel j); the
    usage example's ``get_act_scales`` collects the activation statistic.  For
    X (T x K) and for W (N x K) this is the max over axis 0.  ``amax``
    (float32[K]) is the running value from earlier batches; the max is exact
    and order free, so batches may be folded in any order.
    Pinned by test_channel_amax_* (brute force, resumability, membership).
    """
    a = np.abs(widen(x, dtype)).max(axis=0).astype(np.float32)
    if amax is not None:
        a = np.maximum(a, np.asarray(amax, dtype=np.float32))
    return a


# ---------------------------------------------------------------- step (2)


def smooth_factor(a: float, b: float, alpha: float) -> float:
    """s_j = max|X_j|**alpha / max|W_j|**(1 - alpha) (section "ハイパーパラメータ α").

    Formed in fp64 with the C library's pow and one division, then rounded
    once to fp32 (the page does not fix the precision).  A channel whose
    activation or weight maximum is zero gets s = 1, so there is no inf/NaN.
    Pinned by test_smooth_factor_alpha_limits / _alpha_half / _balance / _dead.
    """
    if a == 0.0 or b == 0.0:
        return 1.0
    return float(np.float32(math.pow(a, alpha) / math.pow(b, 1.0 - alpha)))


def smooth_factors(amax_x, amax_w, alpha: float):
    """Vector form of :func:`smooth_factor` plus inv_s = RN32(1 / s), the stored reciprocal.

    Returns (s, inv_s), both float32[K].
    """
    amax_x = np.asarray(amax_x, dtype=np.float32)
    amax_w = np.asarray(amax_w, dtype=np.float32)
    assert amax_x.shape == amax_w.shape
    s = np.empty(amax_x.shape, dtype=np.float32)
    for j in range(amax_x.shape[0]):
        s[j] = smooth_factor(float(amax_x[j]), float(amax_w[j]), float(alpha))
    inv_s = np.float32(1.0) / s  # one fp32 division per channel
    return s, inv_s.astype(np.float32)


# ------------------------------------------------------ smoothing itself


def smooth_fp64(x64: np.ndarray, w64: np.ndarray, s: np.ndarray):
    """The smoothing identity in fp64 (section "平滑化変換の数学").

    X~ = X diag(s)^-1 divides input channel j of X by s_j; W~ = diag(s) W
    multiplies input channel j of W by s_j (W is N x K here, so that is column
    j).  Returns (X~, W~) in fp64.
    Pinned by test_smoothing_identity_fp64.
    """
    s64 = np.asarray(s, dtype=np.float64)
    return x64 / s64[None, :], w64 * s64[None, :]


def apply_col_scale(v32: np.ndarray, c) -> np.ndarray:
    """v[t, j] * c[j] in fp32, one rounding per element.

    With c = inv_s on activations this is X diag(s)^-1 (a multiplication by
    the stored reciprocal, not a per-element division); with c = s on weights
    it is the fold diag(s) W, kept in fp32 and not rounded to the model dtype
    before it is quantized.
    """
    return (np.asarray(v32, dtype=np.float32) * np.asarray(c, dtype=np.float32)[None, :]).astype(np.float32)


# ------------------------------------------------------------ quantizer


def quantize_rows(v32: np.ndarray):
    """Symmetric per-row INT8 quantization.

    For each row: amax = max |v|; delta = RN32(amax / 127) is the stored
    dequant scale; r = RN32(127 / amax); code = clamp(RNE(RN32(v * r)),
    -127, 127).  A zero row gives all-zero codes and delta = 0.  Section
    "Activation外れ値問題" gives the INT8 range; the symmetric grid, the
    per-row (per-token / per-output-channel) granularity and round-half-even
    are readings where the page is silent.
    Returns (q int8[rows, cols], delta float32[rows]).
    Pinned by test_quantize_* (exhaustive nearest code, ties, range, bound).
    """
    v32 = np.asarray(v32, dtype=np.float32)
    rows = v32.shape[0]
    q = np.zeros(v32.shape, dtype=np.int8)
    delta = np.zeros(rows, dtype=np.float32)
    for t in range(rows):
        m = np.float32(np.abs(v32[t]).max()) if v32.shape[1] else np.float32(0)
        if m == 0:
            continue
        delta[t] = m / np.float32(QMAX)
        r = np.float32(QMAX) / m
        y = (v32[t] * r).astype(np.float32)
        q[t] = np.clip(np.rint(y), -QMAX, QMAX).astype(np.int8)
    return q, delta


def scale_quant_rows(x, dtype: str, col_scale):
    """Per-column scale then per-row quantization: steps (2b) and (3).

    (W, s) gives the folded per-output-channel INT8 weight; (X, inv_s) gives
    the smoothed per-token INT8 activation with its dynamic scale.
    """
    return quantize_rows(apply_col_scale(widen(x, dtype), col_scale))


# ---------------------------------------------------------------- step (4)


def gemm_i32(qa: np.ndarray, qb: np.ndarray) -> np.ndarray:
    """C[t, k] = sum_j qa[t, j] * qb[k, j], exact (section comparing GPTQ/AWQ:
    SmoothQuant multiplies the INT8 operands directly, with no dequantization
    before the product).

    Computed as an fp64 matrix product of the int8 values: every product and
    every partial sum is an integer of magnitude <= 127*127*K < 2**53, so each
    is exactly representable and any summation order gives the exact sum.  The
    result is checked to fit int32.
    Pinned by test_gemm_* (Python-integer triple loop, closed forms).
    """
    qa = np.asarray(qa, dtype=np.int8)
    qb = np.asarray(qb, dtype=np.int8)
    K = qa.shape[1]
    assert qb.shape[1] == K
    assert QMAX * QMAX * max(K, 1) < 2 ** 53
    c = qa.astype(np.float64) @ qb.astype(np.float64).T
    c = c.astype(np.int64)
    assert np.abs(c).max(initial=0) < 2 ** 31
    return c.astype(np.int32)


# ---------------------------------------------------------------- step (5)


def dequant(c: np.ndarray, sa, sb, out_dtype: str) -> np.ndarray:
    """Y[t, k] = out(RN32(RN32(f32(C[t, k]) * sa[t]) * sb[k])), left to right, no FMA.

    f32(C) rounds the int32 accumulator to nearest even; each product is one
    fp32 rounding, applied left to right; the final conversion to fp16 / bf16
    rounds to nearest even.  Per-token x per-output-channel scales factor out
    of the K sum, which is what lets the product run in INT8.
    Pinned by test_dequant_* (closed form, end-to-end error bound).
    """
    cf = np.asarray(c, dtype=np.int32).astype(np.float32)
    y = (cf * np.asarray(sa, dtype=np.float32)[:, None]).astype(np.float32)
    y = (y * np.asarray(sb, dtype=np.float32)[None, :]).astype(np.float32)
    return narrow(y, out_dtype)


# ------------------------------------------------- dense 16-bit baseline


def gemm_float(a, b, dtype: str):
    """The FP16 (or bf16) product the page compares W8A8 against (section
    "パフォーマンスベンチマーク(A100-80GB)"): y = a @ b.T for 16-bit operands.

    Returns (y64, bound): the product in fp64 (each 16-bit product is exact in
    fp64, the sum carries at most K * 2^-53 relative rounding) and
    sum_j |a[t, j] b[k, j]|, the scale of the accumulation error a
    reduced-precision sum may add.
    Pinned by test_gemm_float_* (integer-valued operands: exact).
    """
    a64 = widen(a, dtype).astype(np.float64)
    b64 = widen(b, dtype).astype(np.float64)
    return a64 @ b64.T, np.abs(a64) @ np.abs(b64).T


# ------------------------------------------------------ FP8 (E4M3) variant

E4M3_MAX = 448.0  # largest finite E4M3 value (1.75 * 2^8)


def e4m3_value(code: int) -> float:
    """Value of one 8-bit E4M3 code (OCP FP8: 1 sign, 4 exponent bits with bias
    7, 3 mantissa bits; exponent field 0 is subnormal; 0x7f / 0xff are NaN and
    there is no infinity)."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def round_to_e4m3(v32: np.ndarray) -> np.ndarray:
    """float32 -> E4M3 codes (uint8), round to nearest, ties to even.

    The page notes that the smoothing transform carries over to low-bit float
    formats (FAQ on FP4 / Blackwell); this is the FP8 grid of that variant.
    Written from the format: a finite |v| in binade [2^E, 2^(E+1)) has spacing
    2^(E-3) (subnormal spacing 2^-9 below 2^-6); the code is |v| / spacing
    rounded half-to-even, re-encoded as exponent and mantissa.  Inputs are
    finite with |v| < 464 (the midpoint above 448), which the quantizer
    guarantees.  Pinned by test_e4m3_*.
    """
    v = np.asarray(v32, dtype=np.float32).astype(np.float64)
    a = np.abs(v)
    assert np.all(a < 464.0)
    _, e = np.frexp(a)  # a = f * 2^e with f in [0.5, 1)
    E = np.maximum(e - 1, -6)  # binade exponent, subnormals share -6
    spacing = np.ldexp(1.0, E - 3)
    k = np.rint(a / spacing)  # exact division by a power of two; rint is half-to-even
    q = k * spacing  # the rounded magnitude (may step up into the next binade)
    codes = np.zeros(v.shape, dtype=np.uint8)
    for idx in np.ndindex(v.shape):
        mag = q[idx]
        if mag == 0.0:
            c = 0
        elif mag < 2.0 ** -6:
            c = int(round(mag / 2.0 ** -9))  # exact: an integer 1..7
        else:
            ex = int(np.floor(np.log2(mag)))
            man = mag / 2.0 ** ex - 1.0
            c = ((ex + 7) << 3) | int(round(man * 8))
        if v[idx] < 0 or (v[idx] == 0 and np.signbit(v[idx])):
            c |= 0x80
        codes[idx] = c
    return codes


def e4m3_to_float(codes: np.ndarray) -> np.ndarray:
    table = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def quantize_rows_e4m3(v32: np.ndarray):
    """Per-row FP8 (E4M3) quantization, the FP8 counterpart of quantize_rows:
    delta = RN32(amax / 448), r = RN32(448 / amax), code = E4M3(RN32(v * r)).
    A zero row gives zero codes and delta = 0.  Returns (codes uint8, delta).
    Pinned by test_quantize_e4m3_*.
    """
    v32 = np.asarray(v32, dtype=np.float32)
    rows = v32.shape[0]
    q = np.zeros(v32.shape, dtype=np.uint8)
    delta = np.zeros(rows, dtype=np.float32)
    for t in range(rows):
        m = np.float32(np.abs(v32[t]).max()) if v32.shape[1] else np.float32(0)
        if m == 0:
            continue
        delta[t] = m / np.float32(E4M3_MAX)
        r = np.float32(E4M3_MAX) / m
        q[t] = round_to_e4m3((v32[t] * r).astype(np.float32))
    return q, delta


def scale_quant_rows_e4m3(x, dtype: str, col_scale):
    """Per-column scale then per-row FP8 quantization (FP8 form of steps 2b/3)."""
    return quantize_rows_e4m3(apply_col_scale(widen(x, dtype), col_scale))


def gemm_e4m3(qa: np.ndarray, qb: np.ndarray):
    """C = decode(qa) @ decode(qb).T in fp64, and sum |a b| (the scale of the
    accumulation error an fp32 sum may add).  Every E4M3 product is exact in
    fp64.  Pinned by test_gemm_e4m3_brute_force.
    """
    a = e4m3_to_float(qa)
    b = e4m3_to_float(qb)
    return a @ b.T, np.abs(a) @ np.abs(b).T


# ------------------------------------- smoothing folded into an RMS norm
#
# The page's X~ = X s^-1 (section "平滑化変換の数学") is a per-channel
# multiplication; where X is the output of an RMS normalisation (the norm in
# front of the attention and MLP projections of LLaMA-family decoders) it can
# be folded into that norm's per-channel weight gamma.  The fold itself is an
# extension beyond the page.  Reading taken: the per-token quantizer is
# invariant to a positive factor common to a row, so the norm's 1 / rms(x_t)
# moves from the elements into the row's scale; the codes are those of
# x * RN32(gamma * inv_s), and the row scale is RN32(m / 127) / rms(x_t).


def rms_inv(x, dtype: str, eps: float) -> np.ndarray:
    """r_t = 1 / sqrt(mean_j x[t, j]^2 + eps), in fp64 (float64[rows]).

    The sum of squares is math.fsum's correctly rounded sum of the exact
    squares (each fp16 / bf16 square is exact in fp64), so r is within a few
    fp64 ulps of the real value; a zero row with eps = 0 gives +inf.
    Pinned by test_rms_inv_*.
    """
    x64 = widen(x, dtype).astype(np.float64)
    K = x64.shape[1]
    out = np.empty(x64.shape[0], dtype=np.float64)
    for t in range(x64.shape[0]):
        v = math.fsum((x64[t] * x64[t]).tolist()) / K + float(eps)
        out[t] = math.inf if v == 0.0 else 1.0 / math.sqrt(v)
    return out


def rmsnorm_fp64(x, dtype: str, gamma, eps: float) -> np.ndarray:
    """The plain RMS normalisation x[t, j] * r_t * gamma_j, in fp64."""
    r = rms_inv(x, dtype, eps)
    return widen(x, dtype).astype(np.float64) * r[:, None] * np.asarray(gamma, np.float64)[None, :]


def fold_norm_weight(gamma, inv_s) -> np.ndarray:
    """g_j = RN32(gamma_j * inv_s_j): the smoothing's X s^-1 folded into the
    per-channel weight of the norm that produces X."""
    return (np.asarray(gamma, np.float32) * np.asarray(inv_s, np.float32)).astype(np.float32)


def rmsnorm_smooth_quant_rows(x, dtype: str, g, eps: float):
    """Per-token INT8 of RMSNorm(x; gamma) * inv_s, given the folded g.

    The codes and m / 127 are those of scale_quant_rows(x, g); the row scale
    is delta_t = RN32(m_t / 127) * r_t, returned in fp64 (the reference the
    device's fp32 evaluation is held to).  A zero row has delta 0.
    Returns (q int8[rows, cols], delta float64[rows]).
    Pinned by test_rmsnorm_quant_* (against the plain fp64 definition within
    the quantization bound, closed forms, scale invariance).
    """
    q, d = scale_quant_rows(x, dtype, np.asarray(g, np.float32))
    r = rms_inv(x, dtype, eps)
    delta = np.zeros(len(d), dtype=np.float64)
    nz = d > 0
    delta[nz] = d[nz].astype(np.float64) * r[nz]
    return q, delta


# --------------------------------- smoothing folded into a LayerNorm
#
# The same fold for the LayerNorm in front of the projections of OPT-family
# decoders: y = (x - mean) / sqrt(var + eps) * gamma + beta, so
# y * inv_s = (x - mean) r * RN32(gamma * inv_s) + RN32(beta * inv_s).  The
# additive term keeps the row statistics inside every element, so here they
# enter the codes.  Reading taken (the page gives no normalisation at all):
# the statistics are the exact mean and population variance of the fp16 row,
# each rounded once per the steps below, so that they do not depend on a
# summation order; the rest is one IEEE fp32 operation per step.  fp16 input
# only: every fp16 value is an integer multiple of 2^-24, so the row sums are
# exact integers.


def layernorm_stats(x, eps: float):
    """Row statistics of the LayerNorm fold: (mean float32[rows], r float32[rows]).

    With X_j = x_j * 2^24 (an integer for every finite fp16 value), K = cols,
    S1 = sum X_j and S2 = sum X_j^2 (exact integers):
      mean = f32(f64(f64(S1) / (K * 2^24)))
      var  = f32(f64(f64(K * S2 - S1^2) / (K^2 * 2^48)))      (population variance)
      t    = RN32(var + eps);  r = RN32(1 / RN32(sqrt(t))), or r = 0 when t = 0
    where f64() is the correctly rounded conversion to double and f32() to
    float (each to nearest even).  Rows must have K >= 1.
    Pinned by test_layernorm_stats_* (exact rationals, closed forms).
    """
    assert x.dtype == np.float16 and x.ndim == 2 and x.shape[1] >= 1
    rows, K = x.shape
    X = (x.astype(np.float64) * float(1 << 24)).astype(np.int64)  # exact: |X| < 2^41
    eps32 = np.float32(eps)
    mean = np.zeros(rows, dtype=np.float32)
    r = np.zeros(rows, dtype=np.float32)
    for t in range(rows):
        xt = [int(v) for v in X[t]]
        s1 = sum(xt)
        s2 = sum(v * v for v in xt)
        mean[t] = np.float32(float(s1) / float(K << 24))
        var = np.float32(float(K * s2 - s1 * s1) / float((K * K) << 48))
        tt = np.float32(var + eps32)
        if tt > 0:
            r[t] = np.float32(1.0) / np.sqrt(tt)
    return mean, r


def layernorm_smooth_quant_rows(x, g, b, eps: float):
    """Per-token INT8 of LayerNorm(x; gamma, beta) * inv_s, given the folded
    g = RN32(gamma * inv_s) and b = RN32(beta * inv_s) (fold_norm_weight of
    each).  Per element v_j = RN32(RN32(RN32(RN32(x_j - mean) * r) * g_j) + b_j),
    left to right, no fused multiply-add; then quantize_rows(v).
    Returns (q int8[rows, cols], delta float32[rows]).
    Pinned by test_layernorm_quant_* (shift, scale and sign invariances,
    closed forms, the plain fp64 definition within the quantization bound).
    """
    mean, r = layernorm_stats(x, eps)
    x32 = x.astype(np.float32)
    d = (x32 - mean[:, None]).astype(np.float32)
    v = (d * r[:, None]).astype(np.float32)
    v = (v * np.asarray(g, np.float32)[None, :]).astype(np.float32)
    v = (v + np.asarray(b, np.float32)[None, :]).astype(np.float32)
    return quantize_rows(v)


def layernorm_fp64(x, gamma, beta, eps: float) -> np.ndarray:
    """The plain LayerNorm (x - mean) / sqrt(var + eps) * gamma + beta in fp64,
    with numpy's mean and population variance."""
    x64 = x.astype(np.float64)
    mu = x64.mean(axis=1, keepdims=True)
    var = ((x64 - mu) ** 2).mean(axis=1, keepdims=True)
    return (x64 - mu) / np.sqrt(var + eps) * np.asarray(gamma, np.float64)[None, :] + \
        np.asarray(beta, np.float64)[None, :]


# ------------------------------------------------------ composed flows


def prepare_weight(w, dtype: str, amax_x, alpha: float):
    """Offline weight path: amax_w, (s, inv_s), folded INT8 weight and scales.

    Mirrors the usage example's ``smooth_lm`` then ``quantize_model``.
    Returns dict(amax_w, s, inv_s, qw, sw).
    """
    amax_w = channel_amax(w, dtype)
    s, inv_s = smooth_factors(amax_x, amax_w, alpha)
    qw, sw = scale_quant_rows(w, dtype, s)
    return dict(amax_w=amax_w, s=s, inv_s=inv_s, qw=qw, sw=sw)


def linear(x, dtype: str, inv_s, qw, sw):
    """Runtime forward: smooth + per-token quant, INT8 GEMM, dequant.

    Returns dict(qx, sx, c, y).
    """
    qx, sx = scale_quant_rows(x, dtype, inv_s)
    c = gemm_i32(qx, qw)
    y = dequant(c, sx, sw, dtype)
    return dict(qx=qx, sx=sx, c=c, y=y)
