"""Pins for the CPU oracle: page worked examples, exact brute force with
Python integers and fractions, closed forms and invariants of the method.

None of these checks re-types the oracle's own formulas in numpy: the brute
force below rounds exact rationals to binary32/bf16 with integer arithmetic,
so a wrong division order, tie rule, clamp, operand orientation, scale index
or bf16 rounding in the oracle fails at least one of them.
"""
import json
import math
import os
import struct
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

from conftest import GOLDEN
from oracle import w8a8_oracle as O

F32 = np.float32


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# exact reference arithmetic (independent of numpy's float ops)
# ---------------------------------------------------------------------------

def rn(fr: Fraction, p: int, emin: int = -126) -> Fraction:
    """Round a rational to the nearest p-bit binary float, ties to even."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    qe = max(e - (p - 1), emin - (p - 1))
    scaled = a / Fraction(2) ** qe
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * Fraction(2) ** qe


def rn32(fr):
    return rn(fr, 24)


def rnbf16(fr):
    return rn(fr, 8)


def half_away(fr: Fraction) -> int:
    s = -1 if fr < 0 else 1
    a = abs(fr)
    return s * int(math.floor(a + Fraction(1, 2)))


def bf16_bits_of(fr: Fraction) -> int:
    v = np.float32(float(fr))          # fr is a bf16 value: exact in float32
    assert Fraction(float(v)) == fr
    return int(np.array([v], dtype=F32).view(np.uint32)[0] >> 16)


def ref_quantize_row(x, s=None):
    """Brute-force per-token quantization of one row given as float32s."""
    xs = [rn32(Fraction(float(v)) / Fraction(float(sj))) if s is not None else Fraction(float(v))
          for v, sj in zip(x, s if s is not None else [1] * len(x))]
    a = max(abs(v) for v in xs)
    S = rn32(a / 127)
    if S == 0:
        return [0] * len(xs), S
    q = [max(-127, min(127, half_away(rn32(v / S)))) for v in xs]
    return q, S


# ---------------------------------------------------------------------------
# page worked examples
# ---------------------------------------------------------------------------

def test_page_weight_rtn_example():
    g = golden("half_weight_rtn.json")
    w_kn = np.array(g["W_KxN"], dtype=F32)
    wq, sw = O.quantize_weight_f32(w_kn.T)            # our layout is [N, K]
    np.testing.assert_allclose(sw, g["scales_printed"], atol=5e-7)
    np.testing.assert_array_equal(wq.T, np.array(g["q_arith_KxN"]))
    # the printed 62 differs only in that entry, and the page's own
    # reconstruction uses it: 62 * 0.007323 = 0.4540
    qp = np.array(g["q_printed_KxN"])
    assert (qp != wq.T).sum() == 1
    recon_page = qp * np.array(g["scales_printed"])[None, :]
    np.testing.assert_allclose(recon_page, g["recon_printed_KxN"], atol=g["tol_printed"])
    # reconstruction of our codes matches the page wherever the codes agree
    recon = wq.T.astype(np.float64) * sw.astype(np.float64)[None, :]
    agree = qp == wq.T
    np.testing.assert_allclose(recon[agree], np.array(g["recon_printed_KxN"])[agree], atol=1e-4)
    x = np.array(g["x"])
    np.testing.assert_allclose(x @ w_kn.astype(np.float64), g["y_original_printed"], atol=g["tol_printed"])
    np.testing.assert_allclose(x @ recon_page, g["y_recon_printed"], atol=g["tol_printed"])
    np.testing.assert_allclose(x @ recon, g["y_recon_arith"], atol=g["tol_printed"])


def test_page_activation_outlier_example():
    g = golden("half_activation_outlier.json")
    q, S = O.quantize_act_f32(np.array([g["x"]], dtype=F32))
    assert abs(float(S[0]) - g["scale_printed"]) < g["scale_tol"]
    assert q[0].tolist() == g["q_printed"]


def test_page_smoothquant_gamma_example():
    g = golden("half_smoothquant_gamma.json")
    act = np.array(g["normalized"], dtype=F32) * np.array(g["gamma"], dtype=F32)
    np.testing.assert_array_equal(act, np.array(g["activation_printed"], dtype=F32))
    smooth = np.array(g["smooth"], dtype=F32)
    xs = O.smooth_activations(act[None, :], smooth)
    np.testing.assert_array_equal(xs[0], np.array(g["smoothed_printed"], dtype=F32))
    # the page's fixed scale: exact ties 62.5 and 127.5 -> 63 and 127
    q_fixed = O.quantize_with_scale(xs, F32(g["scale_printed"]))
    assert q_fixed[0].tolist() == g["q_printed_at_scale_printed"]
    # dynamic per-token scale
    q, S = O.quantize_act_f32(act[None, :], smooth)
    assert q[0].tolist() == g["q_dynamic"]
    assert abs(float(S[0]) - 1.53 / 127) < 1e-8
    # without smoothing the three small channels collapse (outlier example)
    q0, _ = O.quantize_act_f32(act[None, :])
    assert q0[0].tolist() == [1, 1, 1, 127]


# ---------------------------------------------------------------------------
# rounding rule and clamp
# ---------------------------------------------------------------------------

def test_round_half_away_vs_fraction():
    r = np.random.default_rng(1)
    v = np.concatenate([
        (r.integers(-260, 260, 4000) + 0.5).astype(F32),               # exact ties
        r.uniform(-130, 130, 20000).astype(F32),
        np.array([0.0, -0.0, 0.49999997, -0.49999997, 0.5, -0.5, 1.5, 2.5, -2.5,
                  126.5, 127.49999, 127.5, -127.5, 1e-30, -1e-30], dtype=F32)])
    got = O.round_half_away(v)
    want = [half_away(Fraction(float(x))) for x in v]
    np.testing.assert_array_equal(got, want)


def test_crafted_ties_dynamic_scale_is_power_of_two():
    # row max 127 * 2**k makes S = 2**k exactly, so (n + 1/2) * 2**k are ties
    for k in (-10, 0, 3):
        row = np.array([127, 62.5, -62.5, 0.5, -0.5, 1.5, -1.5, 126.5, -126.5, 0.25],
                       dtype=F32) * F32(2.0 ** k)
        q, S = O.quantize_act_f32(row[None, :])
        assert float(S[0]) == 2.0 ** k
        assert q[0].tolist() == [127, 63, -63, 1, -1, 2, -2, 127, -127, 0]


def test_fixed_scale_clamps_and_saturates():
    xs = np.array([[1e30, -1e30, 200.0, -200.0, 127.4, 127.5, -127.5]], dtype=F32)
    q = O.quantize_with_scale(xs, F32(1.0))
    assert q[0].tolist() == [127, -127, 127, -127, 127, 127, -127]
    assert O.quantize_with_scale(xs, F32(0.0))[0].tolist() == [0] * 7


# ---------------------------------------------------------------------------
# activation quantization: brute force + invariants
# ---------------------------------------------------------------------------

def test_quantize_act_vs_fraction_brute_force():
    r = np.random.default_rng(2)
    for trial in range(40):
        K = int(r.integers(1, 24))
        x = r.standard_normal(K).astype(F32) * F32(10.0 ** r.integers(-3, 3))
        if trial % 3 == 0:
            x[r.integers(0, K)] *= F32(20)
        s = np.exp(r.uniform(-2, 2, K)).astype(F32) if trial % 2 else None
        q, S = O.quantize_act_f32(x[None, :], s)
        qref, Sref = ref_quantize_row(x, s)
        assert Fraction(float(S[0])) == Sref
        assert q[0].tolist() == qref, (trial, x, s)


def test_quantize_act_invariants():
    r = np.random.default_rng(3)
    M, K = 64, 512
    x = r.standard_normal((M, K)).astype(F32)
    x[:, r.choice(K, 5, replace=False)] *= F32(20)
    x[7] = 0.0                                            # zero row
    x[9, :] = F32(1e-39)                                  # subnormal row
    s = np.exp(r.uniform(-1, 1, K)).astype(F32)
    q, S = O.quantize_act_f32(x, s)
    xs = (x / s[None, :]).astype(F32)
    assert q.dtype == np.int8 and q.min() >= -127
    nz = np.any(xs != 0, axis=1)
    assert S[7] == 0 and np.all(q[7] == 0)
    # every nonzero row reaches +-127 exactly once its max is scaled
    assert np.all(np.max(np.abs(q[nz].astype(int)), axis=1) == 127)
    # dequantize(quantize(x)) is within S/2 (plus binary32 slack)
    err = np.abs(q.astype(np.float64) * S[:, None].astype(np.float64) - xs.astype(np.float64))
    assert np.all(err <= S[:, None].astype(np.float64) * 0.5 * (1 + 2.0 ** -20))
    # sign agreement and monotonicity within each row
    assert np.all((np.sign(q) == np.sign(xs)) | (q == 0))
    for m in range(0, M, 7):
        order = np.argsort(xs[m], kind="stable")
        assert np.all(np.diff(q[m][order].astype(int)) >= 0)
    # scaling a row by a power of two scales S and keeps q
    q2, S2 = O.quantize_act_f32(x * F32(8.0), s)
    np.testing.assert_array_equal(q2[nz], q[nz])
    np.testing.assert_array_equal(S2[nz & (S > 1e-30)], S[nz & (S > 1e-30)] * F32(8.0))
    # rows are independent
    qs, Ss = O.quantize_act_f32(x[10:20], s)
    np.testing.assert_array_equal(qs, q[10:20])
    np.testing.assert_array_equal(Ss, S[10:20])


def test_quantize_act_bf16_wrapper():
    bits = np.array([[0x3F80, 0xBF80, 0x4000, 0x0000]], dtype=np.uint16)   # 1, -1, 2, 0
    q, S = O.quantize_act(bits)
    assert float(S[0]) == np.float32(2.0) / np.float32(127)
    assert q[0].tolist() == [64, -64, 127, 0]    # 63.5 -> 64 (half away)


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------

def test_gemm_vs_python_ints():
    r = np.random.default_rng(4)
    for (M, N, K) in [(1, 1, 1), (3, 5, 7), (17, 9, 33), (2, 31, 64)]:
        a = r.integers(-127, 128, (M, K)).astype(np.int8)
        b = r.integers(-127, 128, (N, K)).astype(np.int8)
        got = O.gemm_i32(a, b)
        want = [[sum(int(a[m, k]) * int(b[n, k]) for k in range(K)) for n in range(N)]
                for m in range(M)]
        np.testing.assert_array_equal(got, want)
        assert got.shape == (M, N)


def test_gemm_closed_forms():
    K = 28672
    a = np.full((2, K), 127, np.int8)
    b = np.stack([np.full(K, 127, np.int8), np.full(K, -127, np.int8)])
    acc = O.gemm_i32(a, b)
    assert acc.tolist() == [[16129 * K, -16129 * K]] * 2
    # one-hot weight rows pick columns of the activation codes
    r = np.random.default_rng(5)
    x = r.integers(-127, 128, (6, 40)).astype(np.int8)
    idx = [3, 0, 39, 17]
    w = np.zeros((4, 40), np.int8)
    w[np.arange(4), idx] = 1
    np.testing.assert_array_equal(O.gemm_i32(x, w), x[:, idx].astype(np.int32))


# ---------------------------------------------------------------------------
# epilogue and bf16 rounding
# ---------------------------------------------------------------------------

def test_round_to_bf16_known_cases():
    cases = {1 + 2 ** -8: 0x3F80,                 # tie -> even (1.0)
             1 + 3 * 2 ** -8: 0x3F82,             # tie -> even (1 + 2**-6)
             1 + 2 ** -8 + 2 ** -30: 0x3F81,      # just above the tie
             -(1 + 2 ** -8): 0xBF80,
             2.0 ** -133: 0x0001,                 # smallest subnormal
             3.4e38: 0x7F80,                      # rounds past bf16 max -> inf
             0.0: 0x0000}
    got = O.round_to_bf16(np.array(list(cases.keys())))
    assert got.tolist() == list(cases.values())


def test_epilogue_vs_fraction():
    r = np.random.default_rng(6)
    M, N = 5, 7
    acc = r.integers(-2 ** 28, 2 ** 28, (M, N)).astype(np.int32)
    acc[0, 0] = 0
    s_tok = (r.uniform(1e-4, 1e-1, M)).astype(F32)
    s_chan = (r.uniform(1e-5, 1e-2, N)).astype(F32)
    y64, y = O.dequant_epilogue(acc, s_tok, s_chan)
    for m in range(M):
        for n in range(N):
            exact = Fraction(int(acc[m, n])) * Fraction(float(s_tok[m])) * Fraction(float(s_chan[n]))
            chain = rn32(rn32(rn32(Fraction(int(acc[m, n]))) * Fraction(float(s_tok[m])))
                         * Fraction(float(s_chan[n])))
            assert int(y[m, n]) == bf16_bits_of(rnbf16(chain))
            assert abs(Fraction(float(y64[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 52)
            # the chain stays within one bf16 ulp of the exact value's rounding
            assert abs(int(y[m, n]) - bf16_bits_of(rnbf16(exact))) <= 1
    assert int(y[0, 0]) == 0


def test_epilogue_is_a_binary32_chain():
    # acc = 2^24 + 2^16 + 1 is not a binary32 value: it converts to
    # 2^24 (1 + 2^-8), exactly halfway between two bf16 values, and rounds to
    # the even one (2^24); the exact product is just above halfway (2^24 + 2^17)
    acc = np.array([[2 ** 24 + 2 ** 16 + 1]], dtype=np.int32)
    y64, y = O.dequant_epilogue(acc, np.ones(1, F32), np.ones(1, F32))
    assert int(y[0, 0]) == 0x4B80
    assert bf16_bits_of(rnbf16(Fraction(int(acc[0, 0])))) == 0x4B81


def test_epilogue_scale_orientation():
    acc = np.array([[257, 259], [256, -257]], dtype=np.int32)
    s_tok = np.array([2.0 ** -8, 2.0 ** -7], dtype=F32)
    s_chan = np.array([1.0, 2.0], dtype=F32)
    _, y = O.dequant_epilogue(acc, s_tok, s_chan)
    # y = acc * s_tok[m] * s_chan[n]
    assert y.tolist() == [[0x3F80, 0x4002], [0x4000, 0xC080]]


# ---------------------------------------------------------------------------
# smoothing factors and weight preparation
# ---------------------------------------------------------------------------

def _sqrt_rn32(fr: Fraction) -> Fraction:
    getcontext().prec = 60
    d = (Decimal(fr.numerator) / Decimal(fr.denominator)).sqrt()
    return rn32(Fraction(d))


def test_smoothing_factors_vs_exact():
    r = np.random.default_rng(7)
    ax = np.abs(r.standard_normal(200)).astype(F32) * F32(20)
    aw = np.abs(r.standard_normal(200)).astype(F32) * F32(0.05)
    ax[0], aw[1] = 0, 0
    ax[2], aw[2] = 4.0, 1.0
    s = O.smoothing_factors(ax, aw)
    assert s[0] == 1 and s[1] == 1 and s[2] == 2
    for j in range(3, 200):
        ratio = rn32(Fraction(float(ax[j])) / Fraction(float(aw[j])))
        assert Fraction(float(s[j])) == _sqrt_rn32(ratio)


def test_smoothing_balances_activation_and_weight_ranges():
    # alpha = 1/2: after smoothing, a channel's activation absmax and its
    # weight absmax are both sqrt(ax * aw)
    r = np.random.default_rng(8)
    K, M, N = 96, 32, 48
    out = r.choice(K, 4, replace=False)
    x = r.standard_normal((M, K)).astype(F32)
    x[:, out] *= F32(20)
    w = (r.standard_normal((N, K)) * 0.02).astype(F32)
    xb, wb = O.round_to_bf16(x), O.round_to_bf16(w)
    ax, aw = O.act_channel_absmax(xb), O.weight_channel_absmax(wb)
    s = O.smoothing_factors(ax, aw)
    x_s = O.smooth_activations(O.bf16_to_f32(xb), s)
    w_s = O.bf16_to_f32(wb) * s[None, :]
    target = np.sqrt(ax.astype(np.float64) * aw.astype(np.float64))
    np.testing.assert_allclose(np.max(np.abs(x_s), axis=0), target, rtol=1e-6)
    np.testing.assert_allclose(np.max(np.abs(w_s), axis=0), target, rtol=1e-6)
    # the product is unchanged (before the weight is re-rounded to bf16)
    xw = O.bf16_to_f32(xb).astype(np.float64) @ O.bf16_to_f32(wb).astype(np.float64).T
    np.testing.assert_allclose(x_s.astype(np.float64) @ w_s.astype(np.float64).T, xw,
                               rtol=1e-5, atol=1e-6 * np.abs(xw).max())
    # smoothing flattens the outlier channels seen by the per-token scale
    ratio_before = np.max(np.abs(O.bf16_to_f32(xb)), axis=1) / np.median(np.abs(O.bf16_to_f32(xb)), axis=1)
    ratio_after = np.max(np.abs(x_s), axis=1) / np.median(np.abs(x_s), axis=1)
    assert np.median(ratio_after) < 0.5 * np.median(ratio_before)


def test_smooth_weight_vs_fraction():
    r = np.random.default_rng(9)
    w = O.round_to_bf16((r.standard_normal((6, 10)) * 0.02).astype(F32))
    s = np.exp(r.uniform(-2, 2, 10)).astype(F32)
    ws = O.smooth_weight(w, s)
    w32 = O.bf16_to_f32(w)
    for n in range(6):
        for j in range(10):
            prod = rn32(Fraction(float(w32[n, j])) * Fraction(float(s[j])))
            assert int(ws[n, j]) == bf16_bits_of(rnbf16(prod))


def test_quantize_weight_per_output_channel_vs_fraction():
    r = np.random.default_rng(10)
    N, K = 7, 19
    w = O.round_to_bf16((r.standard_normal((N, K)) * 0.02).astype(F32))
    wq, sw = O.quantize_weight(w)
    w32 = O.bf16_to_f32(w)
    for n in range(N):
        qref, Sref = ref_quantize_row(w32[n])          # one scale per output channel
        assert Fraction(float(sw[n])) == Sref
        assert wq[n].tolist() == qref


# ---------------------------------------------------------------------------
# the whole layer
# ---------------------------------------------------------------------------

def test_linear_matches_brute_force_small():
    r = np.random.default_rng(11)
    M, N, K = 3, 4, 16
    x = O.round_to_bf16(r.standard_normal((M, K)).astype(F32))
    w = O.round_to_bf16((r.standard_normal((N, K)) * 0.02).astype(F32))
    s = O.smoothing_factors(O.act_channel_absmax(x), O.weight_channel_absmax(w))
    wq, sw = O.prepare_weight(w, s)
    out = O.linear(x, s, wq, sw)
    x32 = O.bf16_to_f32(x)
    for m in range(M):
        qref, Sref = ref_quantize_row(x32[m], s)
        assert out["xq"][m].tolist() == qref
        for n in range(N):
            acc = sum(qref[k] * int(wq[n, k]) for k in range(K))
            assert int(out["acc"][m, n]) == acc
            exact = Fraction(acc) * Sref * Fraction(float(sw[n]))
            assert int(out["y"][m, n]) == bf16_bits_of(rnbf16(exact))


def test_w8a8_output_close_to_unquantized_and_smoothing_helps():
    # sanity (not parity): relative Frobenius error of the W8A8 layer against
    # the float product, with and without smoothing, on outlier data
    r = np.random.default_rng(12)
    M, N, K = 32, 64, 256
    x = r.standard_normal((M, K)).astype(F32)
    x[:, r.choice(K, 3, replace=False)] *= F32(30)
    xb = O.round_to_bf16(x)
    wb = O.round_to_bf16((r.standard_normal((N, K)) * 0.02).astype(F32))
    ref = O.bf16_to_f32(xb).astype(np.float64) @ O.bf16_to_f32(wb).astype(np.float64).T

    def rel(smooth):
        wq, sw = O.prepare_weight(wb, smooth)
        y = O.linear(xb, smooth, wq, sw)["y64"]
        return np.linalg.norm(y - ref) / np.linalg.norm(ref)

    s = O.smoothing_factors(O.act_channel_absmax(xb), O.weight_channel_absmax(wb))
    e_plain, e_smooth = rel(None), rel(s)
    assert e_smooth < 0.05
    assert e_smooth < e_plain


# ---------------------------------------------------------------------------
# static per-tensor scale: calibration ([PTQ]) and fixed-scale quantization
# ---------------------------------------------------------------------------

def test_minmax_calibration_closed_form():
    # [PTQ] "1. Min-Max Calibration": S = max(|min|, |max|) / 127
    x = np.array([[-3.0, 1.0, 0.5], [2.0, -0.5, -2.5]], dtype=F32)
    amax, S = O.minmax_calibration(O.act_channel_absmax(O.round_to_bf16(x)))
    assert Fraction(float(amax)) == 3 and Fraction(float(S)) == rn32(Fraction(3, 127))
    # with smoothing the maxima of x / s count: 3/2, 1/4, 2.5/0.5 = 5
    s = np.array([2.0, 4.0, 0.5], dtype=F32)
    amax, S = O.minmax_calibration(O.act_channel_absmax(O.round_to_bf16(x)), s)
    assert Fraction(float(amax)) == 5 and Fraction(float(S)) == rn32(Fraction(5, 127))


def test_minmax_from_channel_maxima_equals_tensor_maximum():
    # max over tokens of RN(x / s) equals RN(max|x| / s): the per-channel route
    # gives the same amax as scanning every smoothed element exactly
    r = np.random.default_rng(11)
    x = O.round_to_bf16(r.standard_normal((40, 24)).astype(F32) * F32(3))
    s = np.exp(r.uniform(-2, 2, 24)).astype(F32)
    amax, _ = O.minmax_calibration(O.act_channel_absmax(x), s)
    xf = O.bf16_to_f32(x)
    want = max(abs(rn32(Fraction(float(v)) / Fraction(float(s[j]))))
               for row in xf for j, v in enumerate(row))
    assert Fraction(float(amax)) == want


def test_histogram_vs_exact_bins():
    # bin = floor(RN(|x'| / w)), w = RN(amax / bins), clamped; checked with
    # exact rationals, including values on bin edges and beyond amax
    r = np.random.default_rng(12)
    bins = 64
    x = O.round_to_bf16(r.standard_normal((6, 16)).astype(F32))
    xf = O.bf16_to_f32(x)
    xf[0, :4] = [0.0, -0.0, 0.25, -0.75]               # edges when w = 1/64 * amax
    s = np.exp(r.uniform(-1, 1, 16)).astype(F32)
    s[:4] = 1.0
    x = O.round_to_bf16(xf)
    amax = F32(2.0)                                      # some |x'| lie beyond it
    h = O.abs_histogram(x, s, amax, bins)
    w = rn32(Fraction(2) / bins)
    want = [0] * bins
    for row in O.bf16_to_f32(x):
        for j, v in enumerate(row):
            xs = rn32(Fraction(float(v)) / Fraction(float(s[j])))
            b = math.floor(rn32(abs(xs) / w))
            want[min(b, bins - 1)] += 1
    assert h.tolist() == want
    assert h[0] >= 2 and h[8] >= 1 and h[24] >= 1       # 0, 0.25 and 0.75 on their edges
    assert O.abs_histogram(x, None, F32(0.0), bins).tolist() == [x.size] + [0] * (bins - 1)


def test_entropy_hand_example():
    # four bins, two levels, h = [2, 1, 0, 1]:
    #   i = 2: P = [2, 2]/4, Q = [2, 1]/3          -> KL = 1/2 ln(9/8)
    #   i = 3: P = [2, 1, 1]/4, Q = [2, 1, 0]/3    -> P has mass where Q has none
    #   i = 4: P = [2, 1, 0, 1]/4, Q = [1.5, 1.5, 0, 1]/4
    #          -> KL = 1/2 ln(4/3) + 1/4 ln(2/3)
    hist = np.array([2, 1, 0, 1])
    kl = O.entropy_kl(hist, levels=2)
    assert math.isclose(kl[2], 0.5 * math.log(9 / 8), rel_tol=1e-12)
    assert math.isinf(kl[3])
    assert math.isclose(kl[4], 0.5 * math.log(4 / 3) + 0.25 * math.log(2 / 3), rel_tol=1e-12)
    i, T, S, _ = O.entropy_calibration(hist, F32(1.0), levels=2)
    assert i == 4 and T == F32(1.0) and Fraction(float(S)) == rn32(Fraction(1, 127))


def test_entropy_no_mass_beyond_first_levels():
    # all values below 128 bins: the first candidate keeps every bin as its own
    # code and clips nothing, so it loses nothing
    r = np.random.default_rng(13)
    bins = 512                                  # any bin count >= 128 behaves alike
    hist = np.zeros(bins, np.int64)
    hist[:128] = r.integers(1, 1000, 128)
    i, T, S, kl = O.entropy_calibration(hist, F32(16.0))
    assert i == 128 and kl[128] == 0.0
    assert T == F32(128 * 16.0 / bins)


def test_entropy_uniform_keeps_full_range():
    # a flat histogram is represented exactly by 128 flat groups at the full
    # range, while any clipping piles mass on one bin
    bins = 512
    hist = np.full(bins, 7, np.int64)
    i, T, S, kl = O.entropy_calibration(hist, F32(3.0))
    assert i == bins and kl[bins] == 0.0 and T == F32(3.0)
    assert np.all(kl[128:bins] > 0)


def test_entropy_clips_rare_outliers():
    # [PTQ] "2. Entropy Calibration": the threshold ignores rare outliers.
    # A normal bulk plus 0.01% of values near 25 sigma: T ends well below
    # the maximum but above the bulk's 99.9th percentile.
    r = np.random.default_rng(14)
    bulk = np.abs(r.standard_normal(200000))
    out = np.abs(r.normal(25.0, 1.0, 20))
    vals = np.concatenate([bulk, out])
    amax = F32(vals.max())
    bins = 1024
    w = float(amax) / bins
    hist = np.bincount(np.minimum((vals / w).astype(np.int64), bins - 1), minlength=bins)
    i, T, S, kl = O.entropy_calibration(hist, amax)
    assert np.quantile(bulk, 0.999) < float(T) < 0.5 * float(amax)


def test_quantize_act_static_page_example():
    # [HALF] "How SmoothQuant prevents outliers in activation tensors": at the
    # page's fixed scale 0.012 the smoothed activation quantizes to the printed
    # codes, with the exact ties 62.5 and 127.5 going to 63 and 127
    g = golden("half_smoothquant_gamma.json")
    act = np.array(g["activation_printed"], dtype=F32)
    q, s_tok = O.quantize_act_static_f32(act[None, :], np.array(g["smooth"], dtype=F32),
                                         F32(g["scale_printed"]))
    assert q[0].tolist() == g["q_printed_at_scale_printed"]
    assert s_tok.tolist() == [F32(g["scale_printed"])]


def test_quantize_act_static_clamp_binds_and_brute_force():
    r = np.random.default_rng(15)
    S = F32(0.0317)
    x = r.standard_normal((5, 32)).astype(F32) * F32(2)
    x[0, :6] = [200 * S, -200 * S, 127.4 * S, 127.6 * S, -1e6, 1e6]   # beyond the range
    s = np.exp(r.uniform(-1, 1, 32)).astype(F32)
    s[:6] = 1.0
    q, s_tok = O.quantize_act_static_f32(x, s, S)
    assert np.all(s_tok == S)
    assert q[0, :6].tolist() == [127, -127, 127, 127, -127, 127]
    for m in range(5):
        for j in range(32):
            xs = rn32(Fraction(float(x[m, j])) / Fraction(float(s[j])))
            want = max(-127, min(127, half_away(rn32(xs / Fraction(float(S))))))
            assert q[m, j] == want
    assert np.all(O.quantize_act_static_f32(x, s, F32(0))[0] == 0)


def test_static_reduces_to_dynamic_for_one_token():
    # with one token and S equal to its own per-token scale, the static and
    # the dynamic quantizers coincide
    r = np.random.default_rng(16)
    x = O.round_to_bf16(r.standard_normal((1, 300)).astype(F32) * F32(4))
    s = np.exp(r.uniform(-1, 1, 300)).astype(F32)
    q_dyn, S_dyn = O.quantize_act(x, s)
    q_st, S_st = O.quantize_act_static(x, s, S_dyn[0])
    assert np.array_equal(q_dyn, q_st) and np.array_equal(S_dyn, S_st)


def test_linear_static_composition():
    r = np.random.default_rng(17)
    x = O.round_to_bf16(r.standard_normal((3, 64)).astype(F32))
    wq = r.integers(-127, 128, (5, 64)).astype(np.int8)
    sw = np.exp(r.uniform(-6, -3, 5)).astype(F32)
    S = F32(0.021)
    out = O.linear_static(x, None, S, wq, sw)
    q, _ = O.quantize_act_static(x, None, S)
    for m in range(3):
        for n in range(5):
            acc = sum(int(q[m, k]) * int(wq[n, k]) for k in range(64))
            assert out["acc"][m, n] == acc
            y = rnbf16(Fraction(acc) * Fraction(float(S)) * Fraction(float(sw[n])))
            assert int(out["y"][m, n]) == bf16_bits_of(y)


def test_linear_static_smoothing_by_hand():
    # x' = x / s with power-of-two factors is exact; with S = 1/16 the codes
    # are x' * 16 clamped: x = [8, -4, 2, 1, 3], s = [2, 4, 1/2, 1, 1/4]
    # gives x' = [4, -1, 4, 1, 12] and codes [64, -16, 64, 16, 127 (192
    # clamped)]; against the unsmoothed x the codes would be [127, -64, 32,
    # 16, 48]. One weight row of ones adds the codes.
    x = O.round_to_bf16(np.array([[8, -4, 2, 1, 3]], F32))
    s = np.array([2, 4, 0.5, 1, 0.25], F32)
    S = F32(1 / 16)
    wq = np.ones((1, 5), np.int8)
    out = O.linear_static(x, s, S, wq, np.array([1.0], F32))
    assert out["xq"].tolist() == [[64, -16, 64, 16, 127]]
    assert out["acc"].tolist() == [[255]]
    # 255 / 16 = 15.9375 = 0b1111.1111 has 8 significant bits: exact in bf16
    assert float(O.bf16_to_f32(out["y"])[0, 0]) == 15.9375


# ---------------------------------------------------------------------------
# fused producers (RMSNorm + quantize, SiLU-gated product + quantize)
# ---------------------------------------------------------------------------

def _rms_inv_exact(row, eps):
    K = len(row)
    ms = rn32(sum(Fraction(float(v)) ** 2 for v in row) / K)
    d = rn32(ms + Fraction(float(F32(eps))))
    return rn32(Fraction(1) / _sqrt_rn32(d))


def test_rms_inverse_vs_fraction():
    r = np.random.default_rng(20)
    h = O.round_to_bf16(r.standard_normal((4, 96)).astype(F32) * F32(3))
    h32 = O.bf16_to_f32(h)
    h32[1, :5] = [1e-30, -2e-38, 400.0, 0.0, -0.0]
    h = O.round_to_bf16(h32)
    inv = O.rms_inverse(h, 1e-5)
    for m, row in enumerate(O.bf16_to_f32(h)):
        assert Fraction(float(inv[m])) == _rms_inv_exact(row, 1e-5)


def test_rms_inverse_rounds_the_mean_once():
    # 2.421875^2 + 0.05615234375^2 = 24614825 / 2^22 is exact in binary64, and
    # a sixteenth of it lies exactly halfway between two binary32 values. A
    # tiny entry (2^-60, square 2^-120; or bf16's least subnormal 2^-133,
    # square 2^-266) puts the exact mean just above that midpoint: one
    # rounding of the exact mean goes up, while rounding the sum to binary64
    # first loses the tiny square and the tie then goes to even (down).
    # Without a tiny entry the mean is the tie itself.
    K = 16
    tie = Fraction(24614825, 2 ** 22) / K
    assert rn32(tie) != rn32(tie + Fraction(1, 2 ** 300))
    rows = np.zeros((4, K), F32)
    rows[:, :2] = [2.421875, 0.05615234375]
    rows[0, 2] = 2.0 ** -60
    rows[2, 15] = -(2.0 ** -133)
    rows[3, 0] = -2.421875                     # signs do not matter
    rows[3, 9] = 2.0 ** -60
    h = O.round_to_bf16(rows)
    assert np.array_equal(O.bf16_to_f32(h), rows)
    for eps in (1e-5, 0.0):
        inv = O.rms_inverse(h, eps)
        for m in range(4):
            assert Fraction(float(inv[m])) == _rms_inv_exact(rows[m].tolist(), eps), (m, eps)
        assert inv[0] == inv[2] == inv[3]
    inv = O.rms_inverse(h, 1e-5)
    assert inv[0] < inv[1]                     # the larger mean, the smaller inverse


def test_rmsnorm_quantize_vs_fraction():
    r = np.random.default_rng(21)
    K = 48
    h = O.round_to_bf16(r.standard_normal((3, K)).astype(F32))
    res = O.round_to_bf16(r.standard_normal((3, K)).astype(F32) * F32(0.3))
    gamma = np.ones(K, F32)
    gamma[[3, 17]] = 20.0                       # the page's outlier mechanism
    s = np.exp(r.uniform(-1, 1, K)).astype(F32)
    g = O.fold_gamma(gamma, s)
    for k in range(K):
        assert Fraction(float(g[k])) == rn32(Fraction(float(gamma[k])) / Fraction(float(s[k])))
    q, S, h_out = O.rmsnorm_quantize(h, res, g, 1e-5)
    hf, rf = O.bf16_to_f32(h), O.bf16_to_f32(res)
    for m in range(3):
        summed = [rnbf16(rn32(Fraction(float(a)) + Fraction(float(b)))) for a, b in zip(hf[m], rf[m])]
        assert [bf16_bits_of(v) for v in summed] == h_out[m].tolist()
        inv = _rms_inv_exact([float(v) for v in summed], 1e-5)
        y = [rn32(rn32(v * inv) * Fraction(float(g[k]))) for k, v in enumerate(summed)]
        a = max(abs(v) for v in y)
        Sm = rn32(a / 127)
        assert Fraction(float(S[m])) == Sm
        assert q[m].tolist() == [max(-127, min(127, half_away(rn32(v / Sm)))) for v in y]


def test_rmsnorm_is_scale_invariant_without_eps():
    # RMSNorm(2^k h) = RMSNorm(h) exactly when eps = 0 (every step scales by a power of 2)
    r = np.random.default_rng(22)
    h32 = O.bf16_to_f32(O.round_to_bf16(r.standard_normal((5, 256)).astype(F32)))
    g = np.exp(r.uniform(-1, 1, 256)).astype(F32)
    q1, S1, _ = O.rmsnorm_quantize(O.round_to_bf16(h32), None, g, 0.0)
    q2, S2, _ = O.rmsnorm_quantize(O.round_to_bf16(h32 * F32(16)), None, g, 0.0)
    assert np.array_equal(q1, q2) and np.array_equal(S1, S2)
    # a row of +-1 has mean square 1: with g = 1 every code is +-127
    q, S, _ = O.rmsnorm_quantize(O.round_to_bf16(np.sign(h32[:1]) + F32(0) * h32[:1]),
                                 None, np.ones(256, F32), 0.0)
    assert np.all(np.abs(q) == 127) and Fraction(float(S[0])) == rn32(Fraction(1, 127))


def _silu_mul_exact(g, u):
    getcontext().prec = 80
    gd = Decimal(Fraction(float(g)).numerator) / Decimal(Fraction(float(g)).denominator)
    ud = Decimal(Fraction(float(u)).numerator) / Decimal(Fraction(float(u)).denominator)
    val = gd / (1 + (-gd).exp()) * ud
    bits = bf16_bits_of(rnbf16(Fraction(val)))
    return bits | 0x8000 if (bits == 0 and val.is_signed()) else bits


def test_silu_mul_vs_high_precision():
    r = np.random.default_rng(23)
    inter = 40
    gate = r.standard_normal((3, inter)).astype(F32) * F32(4)
    up = r.standard_normal((3, inter)).astype(F32)
    gate[0, :4] = [0.0, -200.0, 90.0, 0.5]
    up[0, :4] = [5.0, 3.0, -2.0, 1.0]
    gu = O.round_to_bf16(np.concatenate([gate, up], axis=1))
    m = O.silu_mul(gu)
    x = O.bf16_to_f32(gu)
    for i in range(3):
        for j in range(inter):
            assert int(m[i, j]) == _silu_mul_exact(x[i, j], x[i, inter + j])
    assert O.bf16_to_f32(m[0, :2]).tolist() == [0.0, 0.0]           # silu(0) = 0; underflow
    assert O.bf16_to_f32(m[0, 2:3]).tolist() == [-180.0]             # silu(90) * -2
    # gate and up are the two halves in that order: a zero gate zeroes the product
    gu2 = O.round_to_bf16(np.concatenate([np.zeros((1, 8), F32), np.full((1, 8), 7, F32)], 1))
    assert np.all(O.bf16_to_f32(O.silu_mul(gu2)) == 0)


def _bf16_float(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


def test_silu_mul_quantize_vs_high_precision():
    # the producer's codes from the SiLU product of 80-digit decimals, the
    # smoothing division and the per-token quantizer, all rounded exactly
    r = np.random.default_rng(25)
    inter = 24
    gate = r.standard_normal((2, inter)) * 3
    up = r.standard_normal((2, inter))
    gu = O.round_to_bf16(np.concatenate([gate, up], axis=1).astype(F32))
    s = np.exp(r.uniform(-1.5, 1.5, inter)).astype(F32)
    q, S = O.silu_mul_quantize(gu, s)
    x = O.bf16_to_f32(gu)
    for i in range(2):
        m = [_bf16_float(_silu_mul_exact(x[i, j], x[i, inter + j])) for j in range(inter)]
        qr, Sr = ref_quantize_row(m, s)
        assert q[i].tolist() == qr
        assert Fraction(float(S[i])) == Sr


def _ref_linear_row(q, S, wq, sw):
    """One token row through the integer GEMM and the binary32 epilogue,
    with Python integers and exact rationals."""
    out = []
    for n in range(wq.shape[0]):
        acc = sum(int(a) * int(b) for a, b in zip(q, wq[n]))
        out.append(rnbf16(rn32(rn32(rn32(Fraction(acc)) * S) * Fraction(float(sw[n])))))
    return out


def _ref_rmsnorm_row(h, res, g, eps):
    """(residual add,) RMSNorm and the per-token quantizer on one row of exact
    bf16 values; returns (codes, scale, new residual stream)."""
    if res is not None:
        h = [rnbf16(rn32(a + b)) for a, b in zip(h, res)]
    inv = _rms_inv_exact([float(v) for v in h], eps)
    y = [rn32(rn32(v * inv) * Fraction(float(gk))) for v, gk in zip(h, g)]
    a = max(abs(v) for v in y)
    S = rn32(a / 127)
    q = [0] * len(y) if S == 0 else [max(-127, min(127, half_away(rn32(v / S)))) for v in y]
    return q, S, h


def _ref_chain_row(x, layers, K, inter, eps=1e-5):
    """The block chain on one token, every step with exact arithmetic: pre-
    norm, qkv, the first K columns of qkv through o, residual + norm,
    gate_up, SiLU of the first half times the second, down, residual."""
    h = [Fraction(float(v)) for v in x]
    pending = None
    for L in layers:
        q, S, h = _ref_rmsnorm_row(h, pending, L["g_attn"], eps)
        y_qkv = _ref_linear_row(q, S, *L["qkv"])
        q, S = ref_quantize_row([float(v) for v in y_qkv[:K]], L["s_o"])
        y_o = _ref_linear_row(q, S, *L["o"])
        q, S, h = _ref_rmsnorm_row(h, y_o, L["g_mlp"], eps)
        y_gu = _ref_linear_row(q, S, *L["gate_up"])
        m = [_bf16_float(_silu_mul_exact(float(y_gu[j]), float(y_gu[inter + j])))
             for j in range(inter)]
        q, S = ref_quantize_row(m, L["s_down"])
        pending = _ref_linear_row(q, S, *L["down"])
    return [rnbf16(rn32(a + b)) for a, b in zip(h, pending)]


def test_chain_forward_vs_exact_arithmetic():
    # two small layers with smoothing factors and an outlier gamma, checked
    # row by row against the chain rebuilt from exact rationals
    r = np.random.default_rng(26)
    K, inter = 16, 24
    def lw(n, k):
        w = O.round_to_bf16(r.standard_normal((n, k)).astype(F32) * F32(0.2))
        return O.quantize_weight(w)
    layers = []
    for _ in range(2):
        gamma = np.ones(K, F32)
        gamma[[2, 11]] = 20.0
        layers.append({
            "g_attn": O.fold_gamma(gamma, np.exp(r.uniform(-1, 1, K)).astype(F32)),
            "g_mlp": np.exp(r.uniform(-0.5, 0.5, K)).astype(F32),
            "s_o": np.exp(r.uniform(-1, 1, K)).astype(F32),
            "s_down": np.exp(r.uniform(-1, 1, inter)).astype(F32),
            "qkv": lw(3 * K, K), "o": lw(K, K), "gate_up": lw(2 * inter, K),
            "down": lw(K, inter)})
    x = O.round_to_bf16(r.standard_normal((2, K)).astype(F32))
    out = O.chain_forward(x, layers)
    xf = O.bf16_to_f32(x)
    for m in range(2):
        ref = _ref_chain_row(xf[m], layers, K, inter)
        assert out[m].tolist() == [bf16_bits_of(v) for v in ref], m


def test_chain_rows_are_independent():
    # every op in the chain is row-local: running any subset of rows alone
    # gives those rows of the full run
    r = np.random.default_rng(24)
    K, I = 32, 48
    def lw(n, k):
        w = O.round_to_bf16(r.standard_normal((n, k)).astype(F32) * F32(0.05))
        return O.quantize_weight(w)
    layers = [{"g_attn": np.ones(K, F32), "g_mlp": np.ones(K, F32), "s_o": None, "s_down": None,
               "qkv": lw(3 * K, K), "o": lw(K, K), "gate_up": lw(2 * I, K), "down": lw(K, I)}
              for _ in range(2)]
    x = O.round_to_bf16(r.standard_normal((7, K)).astype(F32))
    full = O.chain_forward(x, layers)
    part = O.chain_forward(x[[1, 4, 6]], layers)
    assert np.array_equal(full[[1, 4, 6]], part)
    # one layer by hand
    one = O.chain_forward(x, layers[:1])
    L = layers[0]
    q, S, h = O.rmsnorm_quantize(x, None, L["g_attn"], 1e-5)
    yq = O.dequant_epilogue(O.gemm_i32(q, L["qkv"][0]), S, L["qkv"][1])[1]
    q, S = O.quantize_act(np.ascontiguousarray(yq[:, :K]), None)
    yo = O.dequant_epilogue(O.gemm_i32(q, L["o"][0]), S, L["o"][1])[1]
    q, S, h = O.rmsnorm_quantize(h, yo, L["g_mlp"], 1e-5)
    yg = O.dequant_epilogue(O.gemm_i32(q, L["gate_up"][0]), S, L["gate_up"][1])[1]
    q, S = O.silu_mul_quantize(yg, None)
    yd = O.dequant_epilogue(O.gemm_i32(q, L["down"][0]), S, L["down"][1])[1]
    assert np.array_equal(one, O.residual_add(h, yd))


# ---------------------------------------------------------------------------
# GPTQ
# ---------------------------------------------------------------------------

def test_gptq_diagonal_hessian_is_rtn():
    # with a diagonal Hessian no error is redistributed: GPTQ is RTN
    r = np.random.default_rng(30)
    w = O.round_to_bf16(r.standard_normal((9, 40)).astype(F32) * F32(0.02))
    s = np.exp(r.uniform(-1, 1, 40)).astype(F32)
    U = np.diag(np.exp(r.uniform(-2, 2, 40)))
    q, sw = O.gptq_quantize(w, s, U)
    q_rtn, sw_rtn = O.prepare_weight(w, s)
    assert np.array_equal(q, q_rtn) and np.array_equal(sw, sw_rtn)


def test_gptq_two_columns_by_hand():
    # the first column rounds as RTN; its error, divided by U00 and scaled by
    # U01, moves the second weight before it is rounded
    w32 = np.array([[0.31, -0.47], [0.05, 0.12]], dtype=F32)
    w = O.round_to_bf16(w32)
    U = np.array([[2.0, -0.75], [0.0, 1.5]])
    q, sw = O.gptq_quantize(w, None, U)
    wf = O.bf16_to_f32(w)
    for n in range(2):
        s = rn32(max(abs(Fraction(float(v))) for v in wf[n]) / 127)
        assert Fraction(float(sw[n])) == s
        a, b = Fraction(float(wf[n, 0])), Fraction(float(wf[n, 1]))
        q0 = max(-127, min(127, half_away(rn32(a / s))))
        assert q[n, 0] == q0
        err = float(Fraction(float(a)) - q0 * s) / 2.0          # binary64 steps
        b2 = float(b) - err * -0.75
        q1 = max(-127, min(127, half_away(rn32(Fraction(float(np.float32(b2))) / s))))
        assert q[n, 1] == q1


def test_gptq_factor_and_hessian():
    r = np.random.default_rng(31)
    x = O.round_to_bf16(r.standard_normal((50, 24)).astype(F32))
    H = O.gptq_hessian(x)
    xf = O.bf16_to_f32(x)
    for i, j in [(0, 0), (3, 7), (23, 11)]:
        exact = 2 * sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xf[:, i], xf[:, j]))
        assert abs(Fraction(float(H[i, j])) - exact) <= abs(exact) * Fraction(1, 2 ** 45)
    assert np.array_equal(H, H.T)
    U = O.gptq_factor(H)
    assert np.allclose(np.tril(U, -1), 0) and np.all(np.diag(U) > 0)
    Hd = H + 0.01 * np.mean(np.diag(H)) * np.eye(24)
    np.testing.assert_allclose(U.T @ U @ Hd, np.eye(24), atol=1e-9)
    # a never-excited column gets H_jj = 1 before damping
    H0 = H.copy(); H0[5, :] = 0; H0[:, 5] = 0
    U0 = O.gptq_factor(H0)
    assert np.all(np.isfinite(U0))


def test_gptq_hessian_of_smoothed_activations():
    # with power-of-two smoothing factors x / s is exact, so the Hessian of
    # the smoothed activations is the raw one scaled entry by entry by
    # 1 / (s_i s_j), exactly
    r = np.random.default_rng(32)
    x = O.round_to_bf16(r.standard_normal((40, 16)).astype(F32))
    s = (2.0 ** r.integers(-3, 4, 16)).astype(F32)
    H_raw = O.gptq_hessian(x)
    H_s = O.gptq_hessian(x, s)
    assert not np.array_equal(H_s, H_raw)
    np.testing.assert_array_equal(H_s, H_raw / np.outer(s, s).astype(np.float64))


def test_gptq_lowers_output_error_against_rtn():
    # the point of the method: the calibration output error of GPTQ codes is
    # below that of round-to-nearest; most so when input channels correlate
    r = np.random.default_rng(32)
    K, N = 128, 64
    w = O.round_to_bf16(r.standard_normal((N, K)).astype(F32) * F32(0.02))
    q_rtn, sw = O.prepare_weight(w, None)
    Wf = O.bf16_to_f32(w).astype(np.float64)
    mix = r.standard_normal((K, K)) * 0.3 + np.eye(K)
    for x, bound in ((O.round_to_bf16(r.standard_normal((512, K)).astype(F32)), 1.0),
                     (O.round_to_bf16((r.standard_normal((512, K)) @ mix).astype(F32)), 0.8)):
        q, sw_g = O.gptq_quantize(w, None, O.gptq_factor(O.gptq_hessian(x)))
        assert np.array_equal(sw_g, sw)
        X = O.bf16_to_f32(x).astype(np.float64)
        def out_err(qq):
            return np.linalg.norm((Wf - qq * sw[:, None].astype(np.float64)) @ X.T)
        assert out_err(q) < bound * out_err(q_rtn)
