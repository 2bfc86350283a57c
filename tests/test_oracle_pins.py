"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test ties one oracle function to something other than its own formula:
exact rational arithmetic, brute force over all candidates, closed forms,
invariants, library routines, or values printed on the jisaku.com glossary
page "SmoothQuant" (cited by section).
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests.exact import (F, decimal_pow_ratio, rn16, rn32, rn32_decimal, rnbf16,
                         ulp32)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


def _bf16_bits(x32: np.ndarray) -> np.ndarray:
    """bf16 bit patterns via torch's own conversion (an independent routine)."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ dtypes


def test_widen_bf16_bits():
    bits = np.array([0x3F80, 0xC000, 0x3F00, 0x4049, 0x7F7F, 0x0001, 0x8000], dtype=np.uint16)
    want = [1.0, -2.0, 0.5, 3.140625, (2 - 2 ** -7) * 2.0 ** 127, 2.0 ** -133, -0.0]
    got = oracle.widen(bits, "bf16")
    assert got.dtype == np.float32
    for g, w in zip(got.tolist(), want):
        assert g == w and math.copysign(1, g) == math.copysign(1, w)


def test_widen_f16_exact():
    h = np.array([0.1, -65504, 6e-8, 1.5], dtype=np.float16)
    assert [F(v) for v in oracle.widen(h, "f16")] == [F(v) for v in h]


def test_round_to_bf16_ties_and_exact():
    one = 1.0
    cases = {
        one + 2 ** -8: 0x3F80,        # halfway, kept bit even -> down
        one + 3 * 2 ** -8: 0x3F82,    # halfway, kept bit odd -> up
        one + 2 ** -8 + 2 ** -20: 0x3F81,  # just above halfway -> up
        -(one + 2 ** -8): 0xBF80,
        0.0: 0x0000,
    }
    for v, bits in cases.items():
        assert int(oracle.round_to_bf16(np.array([v], np.float32))[0]) == bits


def test_round_to_bf16_vs_exact_and_torch():
    x = (rng.standard_normal(4000) * np.exp(rng.uniform(-30, 30, 4000))).astype(np.float32)
    got = oracle.round_to_bf16(x)
    assert np.array_equal(got, _bf16_bits(x))
    for v, g in zip(x[:300], got[:300]):
        want = rnbf16(F(v))
        assert oracle.widen(np.array([g], np.uint16), "bf16")[0] == np.float32(want)


# ------------------------------------------------------------ channel amax


def test_channel_amax_brute_force():
    x = (rng.standard_normal((37, 24)) * 10).astype(np.float16)
    x[3, 5] = -0.0
    got = oracle.channel_amax(x, "f16")
    for j in range(24):
        best = Fraction(0)
        for t in range(37):
            best = max(best, abs(F(x[t, j])))
        assert F(got[j]) == best
        # the maximum is one of the inputs of column j
        assert any(abs(F(x[t, j])) == best for t in range(37))


def test_channel_amax_resumable_bf16():
    x32 = (rng.standard_normal((64, 40)) * 3).astype(np.float32)
    xb = _bf16_bits(x32)
    whole = oracle.channel_amax(xb, "bf16")
    a = oracle.channel_amax(xb[:17], "bf16")
    b = oracle.channel_amax(xb[17:], "bf16", amax=a)
    c = oracle.channel_amax(xb[40:], "bf16")
    d = oracle.channel_amax(xb[:40], "bf16", amax=c)
    assert np.array_equal(whole, b) and np.array_equal(whole, d)


def test_channel_amax_on_weights_is_over_output_channels():
    # W is N x K; max|W_j| runs over the N output channels of input channel j.
    w = np.zeros((5, 3), np.float16)
    w[4, 0] = -7
    w[0, 2] = 2
    assert oracle.channel_amax(w, "f16").tolist() == [7.0, 0.0, 2.0]


# ------------------------------------------------------- smoothing factors


def _rand_amax(n):
    return np.exp(rng.uniform(-6, 6, n)).astype(np.float32)


def test_smooth_factor_alpha_limits():
    a, b = _rand_amax(500), _rand_amax(500)
    s1, inv1 = oracle.smooth_factors(a, b, 1.0)
    assert np.array_equal(s1, a)  # alpha = 1: s_j = max|X_j|
    s0, inv0 = oracle.smooth_factors(a, b, 0.0)
    for j in range(500):
        assert s0[j] == rn32(1 / F(b[j]))  # alpha = 0: s_j = 1 / max|W_j|
        assert inv1[j] == rn32(1 / F(s1[j])) and inv0[j] == rn32(1 / F(s0[j]))


@pytest.mark.parametrize("alpha", [0.5, 0.8, 0.3])
def test_smooth_factor_general_alpha_correctly_rounded(alpha):
    a, b = _rand_amax(300), _rand_amax(300)
    s, inv = oracle.smooth_factors(a, b, alpha)
    near = 0
    for j in range(300):
        want, dist = rn32_decimal(decimal_pow_ratio(float(a[j]), float(b[j]), alpha))
        if dist < 2.0 ** -45:
            near += 1  # fp64 evaluation may round either way this close to a midpoint
            assert abs(float(s[j]) - float(want)) <= ulp32(want)
        else:
            assert s[j] == want, (j, a[j], b[j])
        assert inv[j] == rn32(1 / F(s[j]))
    assert near == 0


def test_smooth_factor_balance():
    """max|X~_j| = a/s = (ab)**(1-alpha) and max|W~_j| = b*s = (ab)**alpha."""
    a, b = _rand_amax(200), _rand_amax(200)
    for alpha in (0.5, 0.8):
        s, _ = oracle.smooth_factors(a, b, alpha)
        a64, b64, s64 = a.astype(float), b.astype(float), s.astype(float)
        np.testing.assert_allclose(a64 / s64, (a64 * b64) ** (1 - alpha), rtol=2e-7)
        np.testing.assert_allclose(b64 * s64, (a64 * b64) ** alpha, rtol=2e-7)
        if alpha == 0.5:  # equal split of the difficulty
            np.testing.assert_allclose(a64 / s64, b64 * s64, rtol=3e-7)


def test_smooth_factor_alpha_semantics():
    """alpha = 1 normalises the activation channels (all difficulty goes to W);
    alpha = 0 normalises the weight channels (the printed formula governs where
    the page's labels of the two limits contradict it)."""
    a, b = _rand_amax(50), _rand_amax(50)
    s1, _ = oracle.smooth_factors(a, b, 1.0)
    assert np.allclose(a.astype(float) / s1, 1.0)
    s0, _ = oracle.smooth_factors(a, b, 0.0)
    assert np.allclose(b.astype(float) * s0, 1.0, rtol=1e-7)


def test_smooth_factor_dead_channel():
    s, inv = oracle.smooth_factors(np.array([0, 3, 0], np.float32),
                                   np.array([2, 0, 0], np.float32), 0.5)
    assert s.tolist() == [1, 1, 1] and inv.tolist() == [1, 1, 1]


def test_smoothing_identity_fp64():
    """Y = X W = (X diag(s)^-1)(diag(s) W), section on the smoothing math."""
    x = rng.standard_normal((33, 48))
    x[:, 7] *= 90
    w = rng.standard_normal((20, 48)) * 0.02  # N x K
    s = np.exp(rng.uniform(-4, 4, 48)).astype(np.float32)
    xt, wt = oracle.smooth_fp64(x, w, s)
    y = x @ w.T
    yt = xt @ wt.T
    scale = np.abs(x) @ np.abs(w).T
    assert np.max(np.abs(yt - y) / scale) <= 1e-12
    # smoothing really moved the outlier: channel 7 of X~ is X's channel 7 / s_7
    assert np.allclose(xt[:, 7] * s[7], x[:, 7])


# ----------------------------------------------------------------- quantizer


def _nearest_code(y: Fraction) -> int:
    """Brute force over all 255 symmetric codes; ties go to the even code."""
    best = None
    for c in range(-127, 128):
        d = abs(y - c)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def test_quantize_exhaustive_nearest_code():
    v = (rng.standard_normal((12, 40)) * np.exp(rng.uniform(-8, 8, (12, 1)))).astype(np.float32)
    v[3, 11] *= 300  # an outlier element
    q, d = oracle.quantize_rows(v)
    for t in range(12):
        m = max(abs(F(e)) for e in v[t])
        assert F(d[t]) == F(rn32(m / 127))
        r = rn32(Fraction(127) / m)
        for j in range(40):
            y = rn32(F(v[t, j]) * F(r))
            assert int(q[t, j]) == _nearest_code(F(y))


def test_quantize_crafted_ties():
    # amax = 127 gives r = 1 exactly and delta = 1: codes are RNE of the values.
    v = np.array([[127, 2.5, -2.5, 3.5, 0.5, -0.5, 1.5, -126.5]], np.float32)
    q, d = oracle.quantize_rows(v)
    assert q.tolist() == [[127, 2, -2, 4, 0, 0, 2, -126]] and d.tolist() == [1.0]


def test_quantize_range_and_extremes():
    v = (rng.standard_normal((200, 64)) * np.exp(rng.uniform(-10, 10, (200, 1)))).astype(np.float32)
    v[5] = 0
    q, d = oracle.quantize_rows(v)
    assert q.min() >= -127 and q.max() <= 127
    assert not (q == -128).any()
    assert d[5] == 0 and not q[5].any()
    for t in range(200):
        if t != 5:
            assert np.abs(q[t].astype(int)).max() == 127  # the amax element maps to +-127


def test_quantize_error_bound():
    v = (rng.standard_normal((50, 128)) * 4).astype(np.float32)
    q, d = oracle.quantize_rows(v)
    err = np.abs(v.astype(float) - q.astype(float) * d[:, None].astype(float))
    assert (err <= d[:, None] / 2 * (1 + 2 ** -13)).all()


def _fp32_neighbours(t: np.ndarray, spread: int = 6) -> np.ndarray:
    """Each fp32 value of t and its `spread` neighbours on either side."""
    t = np.ascontiguousarray(t, dtype=np.float32)
    steps = np.arange(-spread, spread + 1, dtype=np.int64)
    return (t.view(np.int32).astype(np.int64)[:, None] + steps[None, :]).astype(np.int32).view(
        np.float32).ravel()


def test_quantizer_reading_multiplies_by_the_rounded_reciprocal():
    """Reading R9: code = RNE(RN32(v * RN32(127 / m))), not RNE(RN32(v / RN32(m / 127))).

    The page fixes the INT8 range (section "Activation外れ値問題") but not how
    a value is divided by the step.  The two readings differ only where
    v * 127 / m lies within an fp32 ulp of a half-integer, so the cases are
    crafted: for several row maxima m, the fp32 neighbours of the preimages
    (k + 1/2) m / 127 of every midpoint, kept where numpy's fp32 arithmetic
    says the readings part.  Each kept case is then decided with exact
    rationals (tests/exact.py): the oracle must give the multiply reading's
    code, which must differ from the divide reading's."""
    f32 = np.float32
    cases = []
    for m in f32([3, 7, 11, 13, 0.3, 5e-3, 91.7, 1234.5, 3 * 2.0 ** -20]):
        k = np.arange(0, 127, dtype=np.float64)
        cand = _fp32_neighbours(((k + 0.5) * float(m) / 127).astype(f32))
        cand = cand[np.abs(cand) < m]
        a = np.rint((cand * (f32(127) / m)).astype(f32))
        b = np.rint((cand / (m / f32(127))).astype(f32))
        for j, c in enumerate(cand[a != b][:3]):
            cases.append((m, c if j % 2 == 0 else -c))
    assert len(cases) >= 20
    rows = np.zeros((len(cases), 2), dtype=np.float32)
    for t, (m, c) in enumerate(cases):
        rows[t] = (m, c)
    q, d = oracle.quantize_rows(rows)
    for t, (m, c) in enumerate(cases):
        r = rn32(Fraction(127) / F(m))
        delta = rn32(F(m) / 127)
        want = _nearest_code(F(rn32(F(c) * F(r))))
        alt = _nearest_code(F(rn32(F(c) / F(delta))))
        assert want != alt, (m, c)
        assert int(q[t, 1]) == want and int(q[t, 0]) == 127 and F(d[t]) == F(delta), (m, c)


def test_smoothing_reading_multiplies_by_the_stored_inverse():
    """Reading R7: X~ = X s^-1 (section "平滑化変換の数学") is applied as
    RN32(x * inv_s) with the stored inv_s, not as a division RN32(x / s) by
    s = RN32(1 / inv_s).  Crafted rows [127, x] with inv_s = [1, c]: the row
    maximum is 127, so r = 1 and the code of x is RNE(RN32(x * c)) itself.
    c runs over the fp32 neighbours of (k + 1/2) / x, kept where numpy's fp32
    arithmetic says the two readings part; exact rationals then decide each
    case, and the oracle must follow the multiply reading."""
    f32 = np.float32
    xs = np.array([3, 5.5, 7.25, 11, 13.125, 17, 29.5, 0.75, 1.375], dtype=np.float16)
    cases = []
    for xc in xs:
        k = np.arange(1, 126, dtype=np.float64)
        cand = _fp32_neighbours(((k + 0.5) / float(xc)).astype(f32))
        x32 = f32(xc)
        a = np.rint((x32 * cand).astype(f32))
        b = np.rint((x32 / (f32(1) / cand).astype(f32)).astype(f32))
        for j, c in enumerate(cand[a != b][:3]):
            cases.append((xc if j % 2 == 0 else -xc, c))
    assert len(cases) >= 20
    for xc, c in cases:
        x = np.array([[127, xc]], dtype=np.float16)
        inv_s = np.array([1.0, c], dtype=np.float32)
        q, d = oracle.scale_quant_rows(x, "f16", inv_s)
        want = _nearest_code(F(rn32(F(xc) * F(c))))
        alt = _nearest_code(F(rn32(F(xc) / F(rn32(Fraction(1) / F(c))))))
        assert want != alt, (xc, c)
        assert int(q[0, 1]) == want and float(d[0]) == 1.0, (xc, c)


def _wide_fp32(shape, seed):
    g = np.random.default_rng(seed)
    return (g.standard_normal(shape) * np.exp(g.uniform(-20, 20, shape))).astype(np.float32)


def test_apply_col_scale_is_one_rounded_product():
    """apply_col_scale(v, c)[t, j] == RN32(v[t, j] * c[j]) exactly (exact
    rationals), on values spread over 2^-29 .. 2^29."""
    v = _wide_fp32((6, 40), 31)
    c = _wide_fp32((40,), 32)
    got = oracle.apply_col_scale(v, c)
    assert got.dtype == np.float32
    for t in range(6):
        for j in range(40):
            assert F(got[t, j]) == F(rn32(F(v[t, j]) * F(c[j]))), (t, j)


def test_fold_norm_weight_is_one_rounded_product():
    """g_j = RN32(gamma_j * inv_s_j) exactly (exact rationals)."""
    gamma = _wide_fp32((300,), 33)
    inv_s = _wide_fp32((300,), 34)
    g = oracle.fold_norm_weight(gamma, inv_s)
    assert g.dtype == np.float32
    for j in range(300):
        assert F(g[j]) == F(rn32(F(gamma[j]) * F(inv_s[j]))), j


def test_golden_page_outlier_example():
    """The page's ordinary / outlier channel values (tests/golden, cited there).

    Per-token quantization without smoothing lets the outlier set the scale:
    the ordinary channel keeps at most a couple of levels.  After smoothing the
    outlier channel (alpha = 0.5 with unit weight maxima) the ordinary channel
    gets a much finer grid, the page's reason for moving difficulty into W.
    """
    rows = [l.split() for l in open(os.path.join(GOLDEN, "page_outlier_example.txt"))
            if l.strip() and not l.startswith("#")]
    x = np.array([[float(r[1]), float(r[2])] for r in rows], np.float16)
    x32 = oracle.widen(x, "f16")
    amax = oracle.channel_amax(x, "f16")
    assert amax.tolist() == [float(np.float16(1.2)), float(np.float16(127.4))]
    q, d = oracle.quantize_rows(x32)
    for t in range(5):
        m = max(abs(F(e)) for e in x32[t])
        r = rn32(Fraction(127) / m)
        for j in range(2):
            assert int(q[t, j]) == _nearest_code(F(rn32(F(x32[t, j]) * F(r))))
    # closed-form values for this example: the ordinary channel of token 0 is -1
    assert q[0].tolist() == [-1, 127] and q[3].tolist() == [2, 127]
    # smoothing with alpha = 0.5 and unit weight maxima: s = sqrt(amax_x)
    s, inv = oracle.smooth_factors(amax, np.ones(2, np.float32), 0.5)
    qs, ds = oracle.scale_quant_rows(x, "f16", inv)
    err_plain = np.abs(q[:, 0] * d - x32[:, 0])
    err_smooth = np.abs(qs[:, 0] * ds / inv[0] - x32[:, 0])
    assert err_smooth.max() < err_plain.max() / 4


# ---------------------------------------------------------------------- GEMM


def test_gemm_brute_force_python_ints():
    for (m, n, k) in [(1, 1, 1), (3, 5, 7), (9, 4, 64), (2, 3, 130)]:
        qa = rng.integers(-127, 128, (m, k), dtype=np.int8)
        qb = rng.integers(-127, 128, (n, k), dtype=np.int8)
        c = oracle.gemm_i32(qa, qb)
        assert c.dtype == np.int32 and c.shape == (m, n)
        for i in range(m):
            for j in range(n):
                assert int(c[i, j]) == sum(int(qa[i, t]) * int(qb[j, t]) for t in range(k))


def test_gemm_closed_forms():
    K = 28672
    ones = np.full((1, K), 127, np.int8)
    assert int(oracle.gemm_i32(ones, -ones)[0, 0]) == -16129 * K == -462450688
    qa = rng.integers(-127, 128, (6, 48), dtype=np.int8)
    ident = (np.eye(48, dtype=np.int16) * 127).astype(np.int8)
    assert np.array_equal(oracle.gemm_i32(qa, ident), qa.astype(np.int32) * 127)


def test_gemm_large_k_vs_integer_matmul():
    qa = rng.choice(np.array([-127, 127, -126, 125], np.int8), (4, 28672))
    qb = rng.integers(-127, 128, (5, 28672), dtype=np.int8)
    want = qa.astype(np.int64) @ qb.astype(np.int64).T  # numpy integer loop, no BLAS
    assert np.array_equal(oracle.gemm_i32(qa, qb), want)


# ------------------------------------------------------------------- dequant


def test_dequant_exact_rounding():
    c = rng.integers(-(2 ** 28), 2 ** 28, (8, 9)).astype(np.int32)
    c[0, 0] = 2 ** 24 + 1  # int -> fp32 tie: rounds to even (2**24)
    c[0, 1] = 2 ** 24 + 3  # -> 2**24 + 4
    sa = np.exp(rng.uniform(-12, -4, 8)).astype(np.float32)
    sb = np.exp(rng.uniform(-12, -4, 9)).astype(np.float32)
    y16 = oracle.dequant(c, sa, sb, "f16")
    ybf = oracle.dequant(c, sa, sb, "bf16")
    for i in range(8):
        for j in range(9):
            cf = rn32(Fraction(int(c[i, j])))
            if (i, j) == (0, 0):
                assert F(cf) == 2 ** 24
            if (i, j) == (0, 1):
                assert F(cf) == 2 ** 24 + 4
            t = rn32(F(cf) * F(sa[i]))
            y = rn32(F(t) * F(sb[j]))
            assert F(y16[i, j]) == F(rn16(F(y)))
            assert F(oracle.widen(ybf[i:i + 1, j], "bf16")[0]) == F(rnbf16(F(y)))


def test_linear_end_to_end_error_bound_and_method_sanity():
    """Oracle linear vs fp64 X W^T: within the quantization error bound, and
    smoothing (alpha = 0.5) beats no smoothing on outlier data (the page's
    claim that X~ is easier to quantize)."""
    M, K, N = 48, 256, 40
    x32 = rng.standard_normal((M, K)).astype(np.float32)
    out = rng.choice(K, 3, replace=False)
    x32[:, out] *= np.array([60, -90, 110], np.float32)
    x = x32.astype(np.float16)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    xf, wf = x.astype(float), w.astype(float)
    y64 = xf @ wf.T
    amax_x = oracle.channel_amax(x, "f16")
    errs = {}
    for alpha in (None, 0.5):
        if alpha is None:
            qw, sw = oracle.scale_quant_rows(w, "f16", np.ones(K, np.float32))
            inv = np.ones(K, np.float32)
            s = inv
        else:
            p = oracle.prepare_weight(w, "f16", amax_x, alpha)
            qw, sw, inv, s = p["qw"], p["sw"], p["inv_s"], p["s"]
        r = oracle.linear(x, "f16", inv, qw, sw)
        y = r["y"].astype(float)
        # per-element bound: sum_j (|x~| dw/2 + |w~| dx/2 + dx dw/4) + rounding
        xt = np.abs(xf * inv.astype(float)[None, :])
        wt = np.abs(wf * s.astype(float)[None, :])
        dx, dw = r["sx"].astype(float), sw.astype(float)
        bound = (xt.sum(1)[:, None] * dw[None, :] / 2 + dx[:, None] * wt.sum(1)[None, :] / 2
                 + K * dx[:, None] * dw[None, :] / 4)
        bound = bound * (1 + 1e-3) + np.abs(y64) * 2e-3 + 1e-3
        assert (np.abs(y - y64) <= bound).all()
        errs[alpha] = np.abs(y - y64).mean()
    assert errs[0.5] < errs[None] / 2


# ------------------------------------------------------- dense 16-bit baseline


def test_gemm_float_integer_operands_exact():
    """Integer-valued fp16/bf16 operands: every product and sum is an integer,
    so the fp64 result must equal the Python-integer sum."""
    for dtype in ("f16", "bf16"):
        a_i = rng.integers(-100, 101, (5, 48))
        b_i = rng.integers(-100, 101, (7, 48))
        if dtype == "f16":
            a, b = a_i.astype(np.float16), b_i.astype(np.float16)
        else:
            a, b = _bf16_bits(a_i.astype(np.float32)), _bf16_bits(b_i.astype(np.float32))
        y, bound = oracle.gemm_float(a, b, dtype)
        for i in range(5):
            for j in range(7):
                assert y[i, j] == sum(int(a_i[i, t]) * int(b_i[j, t]) for t in range(48))
                assert bound[i, j] == sum(abs(int(a_i[i, t]) * int(b_i[j, t])) for t in range(48))


def test_gemm_float_matches_int_gemm_on_codes():
    """On INT8 codes (exact in fp16) the dense baseline and the INT8 product agree."""
    qa = rng.integers(-127, 128, (6, 64), dtype=np.int8)
    qb = rng.integers(-127, 128, (9, 64), dtype=np.int8)
    y, _ = oracle.gemm_float(qa.astype(np.float16), qb.astype(np.float16), "f16")
    assert np.array_equal(y.astype(np.int64), oracle.gemm_i32(qa, qb).astype(np.int64))


# ------------------------------------------------------------ FP8 (E4M3)


def _e4m3_finite_values():
    vals = []
    for c in range(256):
        v = oracle.e4m3_value(c)
        if not math.isnan(v):
            vals.append((c, Fraction(v)))
    return vals


def test_e4m3_grid_facts():
    vals = dict(_e4m3_finite_values())
    assert len(vals) == 254  # 0x7f and 0xff are NaN
    assert vals[0x7E] == 448 and vals[0x08] == Fraction(1, 64) and vals[0x01] == Fraction(1, 512)
    assert vals[0x38] == 1 and vals[0x39] == Fraction(9, 8) and vals[0xB8] == -1


def test_e4m3_roundtrip_every_code():
    for c, v in _e4m3_finite_values():
        got = int(oracle.round_to_e4m3(np.array([float(v)], np.float32))[0])
        if v == 0:
            assert got in (0x00, 0x80) and float(v) == 0
        else:
            assert got == c


def test_e4m3_nearest_code_brute_force_and_ties():
    finite = [(c, v) for c, v in _e4m3_finite_values() if c not in (0x80,)]

    def nearest(x: Fraction) -> int:
        best = None
        for c, v in finite:
            d = abs(x - v)
            if best is None or d < best[0] or (d == best[0] and (c & 1) == 0):
                best = (d, c)
        return best[1]

    xs = list(rng.uniform(-460, 460, 400)) + list(rng.uniform(-2, 2, 300)) + \
        list(rng.uniform(-0.02, 0.02, 200))
    # crafted ties: midpoints between neighbours go to the even mantissa
    xs += [1 + 1 / 16, 1 + 3 / 16, -(1 + 1 / 16), 3 / 1024, 5 / 1024, 440.0, 456.0 - 1e-3]
    x32 = np.array(xs, np.float32)
    got = oracle.round_to_e4m3(x32)
    for x, g in zip(x32, got):
        want = nearest(Fraction(float(x)))
        if float(x) == 0:
            continue
        if want & 0x7F == 0:  # rounds to zero: keeps the sign of x
            want = 0x80 if x < 0 else 0x00
        assert int(g) == want, (float(x), int(g), want)
    assert int(oracle.round_to_e4m3(np.array([1 + 1 / 16], np.float32))[0]) == 0x38  # tie -> 1.0
    assert int(oracle.round_to_e4m3(np.array([1 + 3 / 16], np.float32))[0]) == 0x3A  # tie -> 1.25


def test_quantize_e4m3_range_and_bound():
    v = (rng.standard_normal((60, 96)) * np.exp(rng.uniform(-6, 6, (60, 1)))).astype(np.float32)
    v[4] = 0
    q, d = oracle.quantize_rows_e4m3(v)
    assert d[4] == 0 and not q[4].any()
    vals = oracle.e4m3_to_float(q)
    assert np.isfinite(vals).all() and np.abs(vals).max() <= 448
    for t in range(60):
        if t == 4:
            continue
        assert np.abs(vals[t]).max() == 448  # the amax element maps to +-448
        # relative rounding of E4M3 is at most 2^-4 (normals) plus the scale roundings
        err = np.abs(v[t].astype(float) - vals[t] * float(d[t]))
        assert (err <= np.abs(v[t]) * (2 ** -4 + 2 ** -20) + float(d[t]) * 2 ** -10).all()


def test_gemm_e4m3_brute_force():
    qa = rng.integers(0, 256, (4, 40)).astype(np.uint8)
    qb = rng.integers(0, 256, (5, 40)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x38  # no NaN codes
    qb[(qb & 0x7F) == 0x7F] = 0x38
    c, bound = oracle.gemm_e4m3(qa, qb)
    vals = {cc: Fraction(oracle.e4m3_value(cc)) for cc in range(256) if (cc & 0x7F) != 0x7F}
    for i in range(4):
        for j in range(5):
            exact = sum(vals[int(qa[i, t])] * vals[int(qb[j, t])] for t in range(40))
            assert Fraction(c[i, j]) == exact
            assert Fraction(bound[i, j]) == sum(abs(vals[int(qa[i, t])] * vals[int(qb[j, t])]) for t in range(40))


def test_e4m3_every_midpoint():
    """Each midpoint between neighbouring finite E4M3 magnitudes rounds to the
    neighbour with the even code (ties to even), and the fp32 values just
    either side of it round to the nearer neighbour; both signs."""
    pos = sorted((v, c) for c, v in _e4m3_finite_values() if c < 0x80)
    for (v0, c0), (v1, c1) in zip(pos, pos[1:]):
        mid = (v0 + v1) / 2
        m32 = np.float32(float(mid))
        assert Fraction(float(m32)) == mid  # exact in fp32
        even = c0 if c0 % 2 == 0 else c1
        below = np.nextafter(m32, np.float32(0))
        above = np.nextafter(m32, np.float32(1000))
        got = oracle.round_to_e4m3(np.array([m32, below, above, -m32, -below, -above], np.float32))
        assert [int(g) for g in got] == [even, c0, c1, even | 0x80, c0 | 0x80, c1 | 0x80], (mid, c0, c1)


# ------------------------------------------- smoothing folded into an RMS norm


def test_rms_inv_closed_forms():
    x = np.array([[2.0] * 8, [-0.25] * 8, [3.0, 4.0] * 4, [0.0] * 8], np.float16)
    r = oracle.rms_inv(x, "f16", 0.0)
    assert r[0] == 0.5 and r[1] == 4.0
    assert r[2] == 1.0 / math.sqrt(12.5)
    assert r[3] == math.inf
    r = oracle.rms_inv(x, "f16", 0.75)
    assert r[3] == 1.0 / math.sqrt(0.75) and r[0] == 1.0 / math.sqrt(4.75)


def test_rms_inv_against_decimal():
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    x = (rng.standard_normal((6, 40)) * np.exp(rng.uniform(-4, 4, (6, 1)))).astype(np.float16)
    eps = 1e-6
    r = oracle.rms_inv(x, "f16", eps)
    for t in range(6):
        ms = sum(Fraction(float(v)) ** 2 for v in x[t]) / 40 + Fraction(eps)
        want = 1 / (Decimal(ms.numerator) / Decimal(ms.denominator)).sqrt()
        assert abs(Decimal(r[t]) - want) <= abs(want) * Decimal(2) ** -51


def _rms_case(rows, cols, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((rows, cols)) * np.exp(g.uniform(-3, 3, (rows, 1)))
    x[:, g.choice(cols, 3, replace=False)] *= 60.0  # outlier channels
    gamma = g.uniform(0.2, 2.0, cols).astype(np.float32)
    inv_s = np.exp(g.uniform(-4, 2, cols)).astype(np.float32)
    return x.astype(np.float16), gamma, inv_s


def test_rmsnorm_quant_matches_plain_definition():
    """Dequantized codes against the plain fp64 RMSNorm(x; gamma) * inv_s:
    within half a quantization step (the quantizer's bound) plus the two fp32
    roundings of the fold and the scaling."""
    x, gamma, inv_s = _rms_case(24, 96, 7)
    for eps in (0.0, 1e-5, 3.0):
        q, delta = oracle.rmsnorm_smooth_quant_rows(x, "f16", oracle.fold_norm_weight(gamma, inv_s), eps)
        plain = oracle.rmsnorm_fp64(x, "f16", gamma, eps) * inv_s.astype(np.float64)[None, :]
        deq = q.astype(np.float64) * delta[:, None]
        tol = delta[:, None] / 2 * (1 + 2.0 ** -13) + np.abs(plain) * 2.0 ** -22
        assert (np.abs(deq - plain) <= tol).all()
        assert (np.abs(q).max(axis=1) == 127).all()


def test_rmsnorm_quant_scale_invariance_and_zero_row():
    x, gamma, inv_s = _rms_case(10, 64, 9)
    x[3] = 0
    g = oracle.fold_norm_weight(gamma, inv_s)
    q1, d1 = oracle.rmsnorm_smooth_quant_rows(x, "f16", g, 0.0)
    x2 = (x.astype(np.float32) * 4).astype(np.float16)  # exact: a power of two, no overflow
    q2, d2 = oracle.rmsnorm_smooth_quant_rows(x2, "f16", g, 0.0)
    assert np.array_equal(q1, q2) and np.array_equal(d1, d2)
    assert not q1[3].any() and d1[3] == 0.0
    # the codes are those of the smoothing quantizer with the folded weight
    qs, ds = oracle.scale_quant_rows(x, "f16", (gamma * inv_s).astype(np.float32))
    assert np.array_equal(q1, qs)


# -------------------------------------------- smoothing folded into a LayerNorm


def _ln_rows(rows, cols, seed, shift=0.0):
    g = np.random.default_rng(seed)
    x = g.standard_normal((rows, cols)) * np.exp(g.uniform(-4, 4, (rows, 1))) + shift
    x[:, g.choice(cols, 2, replace=False)] *= 40.0  # outlier channels
    return np.clip(x, -60000, 60000).astype(np.float16)


def test_layernorm_stats_exact_rationals():
    """Mean and population variance against exact rationals from the textbook
    two-pass form (sum of (x - mean)^2), a different route from the oracle's
    K S2 - S1^2.  Where the integer sums stay below 2^53 the oracle's steps
    round exactly once to fp64, so the fp32 results are those of the exact
    values rounded to fp64 then to fp32."""
    x = _ln_rows(12, 48, 3, shift=5.0)
    x[0, :4] = np.float16(6e-8)  # subnormals
    x[1] = np.float16(65504.0) * np.array([1, -1] * 24, np.float16)
    mean, r = oracle.layernorm_stats(x, 0.0)
    for t in range(x.shape[0]):
        xs = [F(float(v)) for v in x[t]]
        mu = sum(xs) / 48
        var = sum((v - mu) ** 2 for v in xs) / 48
        assert mean[t] == np.float32(float(mu)), t
        var32 = np.float32(float(var))
        want_r = np.float32(0.0) if var32 == 0 else np.float32(1.0) / np.sqrt(var32)
        assert r[t] == want_r, t


def test_layernorm_stats_closed_forms():
    x = np.array([[2.0, -2.0] * 8, [3.0, 5.0] * 8, [7.0] * 16, [0.0] * 16,
                  [-1.5, -0.5] * 8], np.float16)
    mean, r = oracle.layernorm_stats(x, 0.0)
    assert list(mean) == [0.0, 4.0, 7.0, 0.0, -1.0]
    assert list(r) == [0.5, 1.0, 0.0, 0.0, 2.0]
    mean, r = oracle.layernorm_stats(x, 0.25)
    assert r[2] == 2.0 and r[3] == 2.0 and r[1] == np.float32(1.0) / np.sqrt(np.float32(1.25))


def _ln_fold(cols, seed):
    g = np.random.default_rng(seed)
    gamma = g.uniform(0.2, 2.0, cols).astype(np.float32)
    beta = g.uniform(-0.5, 0.5, cols).astype(np.float32)
    inv_s = np.exp(g.uniform(-4, 2, cols)).astype(np.float32)
    return gamma, beta, inv_s


def test_layernorm_quant_matches_plain_definition():
    """Dequantized codes against the plain fp64 LayerNorm(x; gamma, beta) *
    inv_s: within half a quantization step plus the fp32 roundings of the
    statistics and of each elementwise step."""
    x = _ln_rows(20, 96, 11, shift=2.0)
    gamma, beta, inv_s = _ln_fold(96, 12)
    g, b = oracle.fold_norm_weight(gamma, inv_s), oracle.fold_norm_weight(beta, inv_s)
    for eps in (0.0, 1e-5, 2.0):
        q, delta = oracle.layernorm_smooth_quant_rows(x, g, b, eps)
        plain = oracle.layernorm_fp64(x, gamma, beta, eps) * inv_s.astype(np.float64)[None, :]
        deq = q.astype(np.float64) * delta.astype(np.float64)[:, None]
        x64 = x.astype(np.float64)
        mu = np.abs(x64.mean(axis=1, keepdims=True))
        rg = np.abs(plain - beta.astype(np.float64)[None, :] * inv_s[None, :]) / np.maximum(
            np.abs(x64 - x64.mean(axis=1, keepdims=True)), 1e-300)
        tol = (delta.astype(np.float64)[:, None] / 2 * (1 + 2.0 ** -13)
               + ((np.abs(x64) + mu) * rg + np.abs(b)[None, :]) * 2.0 ** -20)
        assert (np.abs(deq - plain) <= tol).all(), eps
        assert (np.abs(q).max(axis=1) == 127).all()


def test_layernorm_quant_shift_scale_sign_invariance():
    """LayerNorm ignores a shift of the row and, with eps = 0, a positive
    scale; a sign flip negates (x - mean).  Shifts by an integer of rows whose
    mean is an integer, and scales by 4, are exact in fp16 and in the
    statistics, so the codes and the row scales must not change at all."""
    g0 = np.random.default_rng(21)
    half = g0.integers(-40, 41, (8, 32)).astype(np.float64)
    x = np.concatenate([half, -half], axis=1) + g0.integers(-20, 21, (8, 1))  # integer means
    x = x.astype(np.float16)
    gamma, beta, inv_s = _ln_fold(64, 22)
    g, b = oracle.fold_norm_weight(gamma, inv_s), oracle.fold_norm_weight(beta, inv_s)
    q0, d0 = oracle.layernorm_smooth_quant_rows(x, g, b, 1e-3)
    q1, d1 = oracle.layernorm_smooth_quant_rows((x.astype(np.float32) + 13).astype(np.float16), g, b, 1e-3)
    assert np.array_equal(q0, q1) and np.array_equal(d0, d1)
    y = _ln_rows(8, 64, 23)
    q2, d2 = oracle.layernorm_smooth_quant_rows(y, g, b, 0.0)
    q3, d3 = oracle.layernorm_smooth_quant_rows((y.astype(np.float32) * 4).astype(np.float16), g, b, 0.0)
    assert np.array_equal(q2, q3) and np.array_equal(d2, d3)
    zero = np.zeros(64, np.float32)
    q4, d4 = oracle.layernorm_smooth_quant_rows(y, g, zero, 0.5)
    q5, d5 = oracle.layernorm_smooth_quant_rows(-y, g, zero, 0.5)
    assert np.array_equal(q4, -q5) and np.array_equal(d4, d5)


def test_layernorm_quant_constant_row_is_the_bias():
    """A constant row has x - mean = 0, so v = b and the codes are those of
    the folded bias alone (zero codes when b = 0)."""
    x = np.full((3, 32), 3.25, np.float16)
    gamma, beta, inv_s = _ln_fold(32, 31)
    g, b = oracle.fold_norm_weight(gamma, inv_s), oracle.fold_norm_weight(beta, inv_s)
    for eps in (0.0, 1e-5):
        q, d = oracle.layernorm_smooth_quant_rows(x, g, b, eps)
        qb, db = oracle.quantize_rows(np.tile(b, (3, 1)))
        assert np.array_equal(q, qb) and np.array_equal(d, db)
        q, d = oracle.layernorm_smooth_quant_rows(x, g, np.zeros(32, np.float32), eps)
        assert not q.any() and not d.any()
