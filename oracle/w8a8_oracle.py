"""Reference oracle for the W8A8 INT8 linear layer.

TEST INFRASTRUCTURE ONLY. This is the plain, slow, step-by-step CPU statement
of what the layer computes. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import it. The GPU library never calls it,
and it shares no code, table or constant with the GPU library.

Sources, cited by page title and section:

  [HALF]  "Understanding W8A8 INT8 LLM quantization: Half the size, better
          performance, same accuracy" (Red Hat, part 1 of the series)
  [PERF]  "Understanding W8A8 INT8 LLM quantization: Accuracy and performance
          results" (Red Hat, part 2)
  [PTQ]   "INT8 Post-Training Quantization for LLM Inference on NVIDIA GPUs"

What the layer computes (per linear, at inference):

  1. smooth:   x'[m,j] = x[m,j] / s[j]                        (SmoothQuant)
  2. scale:    S[m]    = max_j |x'[m,j]| / 127                (per token)
  3. quantize: q[m,j]  = clamp(round(x'[m,j] / S[m]), -127, 127)
  4. GEMM:     acc[m,n] = sum_j q[m,j] * Wq[n,j]               (exact integer)
  5. epilogue: y[m,n]  = bf16(acc[m,n] * S[m] * sw[n])

with offline weight preparation

  0. s[j] = sqrt(max_m |Xcal[m,j]| / max_n |W[n,j]|)            (alpha = 1/2)
     W'[n,j] = bf16(W[n,j] * s[j]);  sw[n] = max_j |W'[n,j]| / 127
     Wq[n,j] = clamp(round(W'[n,j] / sw[n]), -127, 127)

Precision and rounding (the readings taken where the pages leave it open):

  * Every floating-point step whose result decides an integer code (steps 0-3)
    is done in IEEE binary32, one correctly rounded operation at a time,
    in the order written above. Divisions are true divisions.
  * round() rounds half away from zero. [HALF] "How SmoothQuant prevents
    outliers in activation tensors" rounds 0.75/0.012 = 62.5 to 63, and its
    1.53/0.012 = 127.5 ends at 127, which is what half-away-then-clamp gives.
  * The clamp keeps codes in [-127, 127]; -128 is never produced.
  * A token (or weight channel) whose absmax is 0 gets scale 0 and all-zero
    codes (the pages do not say; this avoids 0/0).
  * Step 4 is exact: the float64 matmul below only ever holds integers of
    magnitude <= 128*128*K < 2**53, so every product and partial sum is exact
    whatever order the library uses.
  * Step 5 is a binary32 chain, float(acc) * S then * sw, each product
    rounded, then bf16 round-to-nearest-even (the "fp32, then rounded" value
    outputs are compared with); a binary64 value is kept for error reports.
  * bf16 values are handled as their uint16 bit patterns.

Parity pins: every function here is checked in tests/test_oracle_pins.py
against the pages' worked examples (tests/golden/), closed forms, brute force
with Python integers and fractions, and invariants of the method.
"""
from __future__ import annotations

import numpy as np

QMAX = 127  # largest code; [HALF] "How we compressed the model"
F32 = np.float32


# ---------------------------------------------------------------------------
# bf16 helpers
# ---------------------------------------------------------------------------

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32. Exact: bf16 is the top half of binary32."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(v) -> np.ndarray:
    """Round real values (float64 or float32 arrays) once to bf16,
    round-to-nearest-even. Returns uint16 bit patterns.

    bf16 keeps 8 significant bits and binary32's exponent range. A value is
    scaled by a power of two so that its rounding quantum becomes 1, rounded
    with rint (ties to even), and scaled back; all scalings are exact.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros(v.shape, dtype=np.float64)
    nz = v != 0
    _, e = np.frexp(v[nz])                       # |v| = f * 2**e, f in [0.5, 1)
    qexp = np.maximum(e - 8, -133)               # 8 significant bits; subnormal floor
    r = np.rint(np.ldexp(v[nz], -qexp))          # integer count of quanta
    out[nz] = np.ldexp(r, qexp)
    big = np.abs(out) > float(np.ldexp(255.0 / 128.0, 127))   # beyond bf16 max
    out[big] = np.copysign(np.inf, out[big])
    out = np.where(nz, out, v)                   # keep the sign of zero
    return (out.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------
# rounding to int8 codes
# ---------------------------------------------------------------------------

def round_half_away(v: np.ndarray) -> np.ndarray:
    """Nearest integer, ties away from zero, for float32 values (exact).

    trunc(v) and v - trunc(v) are both exact in binary32, so the comparison
    of the discarded fraction with 1/2 is exact.
    """
    v = np.asarray(v, dtype=F32)
    t = np.trunc(v)
    frac = v - t
    up = np.abs(frac) >= F32(0.5)
    return (t.astype(np.int64) + np.where(up, np.sign(v).astype(np.int64), 0))


def quantize_with_scale(xs: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """q = clamp(round(x / S), -127, 127) in binary32; S == 0 gives q = 0.

    [HALF] "The problem with naive quantization" (scale and round),
    [HALF] "How SmoothQuant prevents outliers in activation tensors" (ties),
    [PTQ] "1. Min-Max Calibration" (the symmetric [-127, 127] range).
    ``scale`` broadcasts against ``xs`` (one scale per row here).
    """
    xs = np.asarray(xs, dtype=F32)
    scale = np.asarray(scale, dtype=F32)
    safe = np.where(scale == 0, F32(1), scale)
    with np.errstate(over="ignore"):
        v = xs / safe
    # saturate before rounding (a fixed scale can send x/S past int range);
    # every |v| >= 127.5 ends at +-127 either way
    v = np.clip(v, F32(-2 * QMAX), F32(2 * QMAX))
    q = np.clip(round_half_away(v), -QMAX, QMAX)
    q = np.where(scale == 0, 0, q)
    return q.astype(np.int8)


def absmax_scale(xs: np.ndarray, axis: int = -1) -> np.ndarray:
    """S = max|x| / 127 along ``axis`` (binary32 division).

    [HALF] "How we compressed the model" (scale from the largest magnitude),
    [HALF] "Why activation quantization is hard" (one scale per token).
    """
    a = np.max(np.abs(np.asarray(xs, dtype=F32)), axis=axis)
    return (a / F32(QMAX)).astype(F32)


# ---------------------------------------------------------------------------
# steps 1-3: per-token dynamic activation quantization
# ---------------------------------------------------------------------------

def smooth_activations(x32: np.ndarray, smooth) -> np.ndarray:
    """x' = x / s (binary32 division per element). ``smooth`` None: x' = x.

    [HALF] "How the SmoothQuant smoothing factor is computed": each channel
    is divided by its factor (folded into RMSNorm's gamma there; applied to
    the activation here).
    """
    x32 = np.asarray(x32, dtype=F32)
    if smooth is None:
        return x32.copy()
    smooth = np.asarray(smooth, dtype=F32)
    assert np.all(smooth > 0) and np.all(np.isfinite(smooth)), "smooth must be > 0"
    return x32 / smooth[None, :]


def quantize_act_f32(x32: np.ndarray, smooth=None):
    """Per-token dynamic quantization of float32 activations [M, K].

    Returns (q int8 [M, K], S float32 [M]).
    [HALF] "Why activation quantization is hard, and how SmoothQuant fixes it";
    [PERF] "Inter-token latency (ITL)" (range, scale, convert, per token).
    """
    x32 = np.asarray(x32, dtype=F32)
    assert x32.ndim == 2 and np.all(np.isfinite(x32)), "finite [M, K] input"
    xs = smooth_activations(x32, smooth)
    s_tok = absmax_scale(xs, axis=1)
    q = quantize_with_scale(xs, s_tok[:, None])
    return q, s_tok


def quantize_act(x_bf16: np.ndarray, smooth=None):
    """quantize_act_f32 on bf16 activations given as uint16 bit patterns."""
    return quantize_act_f32(bf16_to_f32(x_bf16), smooth)


# ---------------------------------------------------------------------------
# step 0: offline preparation (smoothing factors, weight quantization)
# ---------------------------------------------------------------------------

def act_channel_absmax(x_bf16: np.ndarray) -> np.ndarray:
    """max over tokens of |X[m, j]| for every input channel j (float32 [K])."""
    return np.max(np.abs(bf16_to_f32(x_bf16)), axis=0).astype(F32)


def weight_channel_absmax(w_bf16: np.ndarray) -> np.ndarray:
    """max over output channels of |W[n, j]| for every input channel j.

    W is stored [N, K]; the page's K x N example calls this "row j of the
    receiving layer's weight" ([HALF] "How the SmoothQuant smoothing factor
    is computed").
    """
    return np.max(np.abs(bf16_to_f32(w_bf16)), axis=0).astype(F32)


def smoothing_factors(act_absmax: np.ndarray, w_absmax: np.ndarray) -> np.ndarray:
    """s[j] = sqrt(act_absmax[j] / w_absmax[j]) in binary32; 1 where either is 0.

    SmoothQuant's factor with migration strength alpha = 1/2; the page lists
    its terms ([HALF] "How the SmoothQuant smoothing factor is computed") and
    uses alpha = 0.8 there; the square root is the alpha = 1/2 member.
    """
    a = np.asarray(act_absmax, dtype=F32)
    w = np.asarray(w_absmax, dtype=F32)
    ok = (a > 0) & (w > 0)
    ratio = np.where(ok, a / np.where(ok, w, F32(1)), F32(1))
    return np.where(ok, np.sqrt(ratio.astype(F32)), F32(1)).astype(F32)


def smooth_weight(w_bf16: np.ndarray, smooth) -> np.ndarray:
    """W'[n, j] = bf16(W[n, j] * s[j]): binary32 product, then bf16 (RNE).

    The weights stay bf16 after smoothing ([HALF] "How the SmoothQuant
    smoothing factor is computed").
    """
    w32 = bf16_to_f32(w_bf16)
    if smooth is None:
        return np.asarray(w_bf16, dtype=np.uint16).copy()
    prod = w32 * np.asarray(smooth, dtype=F32)[None, :]
    return round_to_bf16(prod)


def quantize_weight_f32(w32: np.ndarray):
    """Per-output-channel symmetric RTN of float32 weights [N, K].

    Returns (Wq int8 [N, K], sw float32 [N]).
    [HALF] "The problem with naive quantization": one scale per weight
    channel (a column of its K x N example = a row of our [N, K] layout).
    """
    w32 = np.asarray(w32, dtype=F32)
    sw = absmax_scale(w32, axis=1)
    return quantize_with_scale(w32, sw[:, None]), sw


def quantize_weight(w_bf16: np.ndarray):
    return quantize_weight_f32(bf16_to_f32(w_bf16))


def prepare_weight(w_bf16: np.ndarray, smooth):
    """Smooth then quantize: (Wq int8 [N, K], sw float32 [N])."""
    return quantize_weight(smooth_weight(w_bf16, smooth))


# ---------------------------------------------------------------------------
# steps 4-5: integer GEMM and dequantizing epilogue
# ---------------------------------------------------------------------------

def gemm_i32(xq: np.ndarray, wq: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k xq[m, k] * wq[n, k], exact; returned as int32.

    [HALF] "How we compressed the model" (both operands int8 in the matmul).
    """
    xq = np.asarray(xq, dtype=np.int8)
    wq = np.asarray(wq, dtype=np.int8)
    assert xq.ndim == 2 and wq.ndim == 2 and xq.shape[1] == wq.shape[1]
    K = xq.shape[1]
    assert 128 * 128 * max(K, 1) < 2 ** 53
    acc = xq.astype(np.float64) @ wq.astype(np.float64).T
    acc_i = acc.astype(np.int64)
    assert np.all(acc_i == acc)
    assert np.all(np.abs(acc_i) < 2 ** 31), "accumulator leaves int32"
    return acc_i.astype(np.int32)


def dequant_epilogue(acc: np.ndarray, s_tok: np.ndarray, s_chan: np.ndarray):
    """y[m, n] = bf16(RN32(RN32(RN32(acc[m, n]) * S[m]) * sw[n])).

    The per-token and per-channel scales factor out of the K-sum, so they are
    applied after accumulation ([HALF] "Why activation quantization is hard";
    [PERF] "Inter-token latency (ITL)": convert back to BF16). The chain is
    binary32, one rounding per step in the order written (the accumulator
    converted, times the token scale, times the channel scale), then bf16
    round-to-nearest-even: the "fp32, then rounded" value the outputs are
    compared with. Returns (y64 float64 [M, N], y bf16 bits uint16 [M, N]),
    y64 = acc * S * sw in binary64 for reporting the error of y.
    """
    acc = np.asarray(acc)
    st = np.asarray(s_tok, dtype=F32)
    sc = np.asarray(s_chan, dtype=F32)
    t = acc.astype(F32)                       # int32 -> binary32, nearest even
    v = (t * st[:, None]) * sc[None, :]       # binary32 products, in this order
    y64 = (acc.astype(np.float64) * st.astype(np.float64)[:, None]
           * sc.astype(np.float64)[None, :])
    return y64, round_to_bf16(v)


def linear(x_bf16: np.ndarray, smooth, wq: np.ndarray, s_chan: np.ndarray):
    """Steps 1-5 for one linear. Returns a dict of every intermediate."""
    xq, s_tok = quantize_act(x_bf16, smooth)
    acc = gemm_i32(xq, wq)
    y64, y = dequant_epilogue(acc, s_tok, s_chan)
    return {"xq": xq, "s_tok": s_tok, "acc": acc, "y64": y64, "y": y}


# ---------------------------------------------------------------------------
# static per-tensor activation scale, calibrated offline ([PTQ])
# ---------------------------------------------------------------------------
#
# [PTQ] "The Heart of PTQ: Entropy-Based Calibration" fixes one scale per
# activation tensor ahead of time instead of one per token at run time:
# min-max calibration maps the largest magnitude seen to 127; entropy
# calibration clips at the threshold T that loses the least information
# (smallest KL divergence between the clipped histogram and its quantized
# version) and uses S = T / 127. The run-time step then needs no reduction,
# and the clamp to [-127, 127] binds for values beyond the threshold.
#
# Readings where the page leaves the procedure open (it is partly garbled):
#   * magnitudes |x'| are histogrammed (the int8 grid is symmetric), in
#     HIST_BINS equal bins over [0, amax]: bin = floor(|x'| / w) with
#     w = amax / HIST_BINS, both binary32 divisions, clamped to the last bin;
#   * candidate thresholds are bin edges T_i = i * w, i = QUANT_LEVELS ..
#     HIST_BINS (the page moves T inward from the maximum);
#   * reference distribution P_i: bins 0 .. i-1 of the histogram h, the mass
#     beyond T_i folded into bin i-1 (saturated values land on the top code);
#   * quantized distribution Q_i: the values inside [0, T_i) only, i.e. h[0..i)
#     split into QUANT_LEVELS groups [g*i // L, (g+1)*i // L) (the 128 code
#     magnitudes 0..127), each group's count spread evenly over its bins
#     with h > 0;
#   * KL(P_i || Q_i) = sum over p > 0 of p log(p / q), P_i and Q_i each
#     normalized to sum 1, in binary64; a bin with p > 0 and q = 0 makes the
#     candidate infinitely bad; the smallest i with the minimal value wins;
#   * T = i * w and S = T / 127 in binary32.

HIST_BINS = 2048
QUANT_LEVELS = 128


def minmax_calibration(act_absmax: np.ndarray, smooth=None):
    """amax = max_j |x'[., j]| and S = amax / 127 from per-channel maxima.

    [PTQ] "1. Min-Max Calibration". ``act_absmax[j]`` = max over calibration
    tokens of |x[m, j]| (bf16 values, as act_channel_absmax returns). Since
    RN(a / s) is monotone in a for s > 0, max_m |RN(x / s)| = RN(max_m|x| / s),
    so the smoothed maximum is one division per channel. Returns float32
    (amax, S).
    """
    a = np.asarray(act_absmax, dtype=F32)
    if smooth is not None:
        a = smooth_activations(a[None, :], smooth)[0]
    amax = F32(np.max(a)) if a.size else F32(0)
    return amax, F32(amax / F32(QMAX))


def abs_histogram(x_bf16: np.ndarray, smooth, amax, bins: int = HIST_BINS) -> np.ndarray:
    """Counts of |x'| in ``bins`` equal bins over [0, amax] (int64 [bins]).

    bin = floor(min(RN(|x'| / w), bins - 1)), w = RN(amax / bins): values at
    or beyond amax land in the last bin. When w is 0 (amax 0, or so small
    that amax / bins underflows) every value goes to bin 0.
    """
    xs = smooth_activations(bf16_to_f32(x_bf16), smooth)
    a = np.abs(xs).ravel()
    w = F32(F32(amax) / F32(bins))
    if w == 0:
        idx = np.zeros(a.shape, np.int64)
    else:
        with np.errstate(over="ignore"):
            ratio = (a / w).astype(F32)
        idx = np.floor(np.minimum(ratio, F32(bins - 1))).astype(np.int64)
    return np.bincount(idx, minlength=bins).astype(np.int64)


def entropy_kl(hist: np.ndarray, levels: int = QUANT_LEVELS) -> np.ndarray:
    """KL(P_i || Q_i) for every candidate i (float64 [bins + 1], NaN below
    ``levels``, +inf where Q_i misses mass of P_i), following the readings
    above. An empty histogram gives 0 everywhere."""
    h = np.asarray(hist, dtype=np.float64)
    bins = h.size
    kl = np.full(bins + 1, np.nan)
    if h.sum() == 0:
        kl[levels:] = 0.0
        return kl
    for i in range(levels, bins + 1):
        p = h[:i].copy()
        p[i - 1] += h[i:].sum()                      # saturated mass
        q = np.zeros(i)
        for g in range(levels):
            lo, hi = g * i // levels, (g + 1) * i // levels
            seg = h[lo:hi]
            used = seg > 0
            if used.any():
                q[lo:hi][used] = seg.sum() / used.sum()
        if q.sum() == 0:                             # nothing below T_i
            kl[i] = np.inf
            continue
        pn, qn = p / p.sum(), q / q.sum()
        m = pn > 0
        if np.any(qn[m] == 0):
            kl[i] = np.inf
            continue
        kl[i] = float(np.sum(pn[m] * np.log(pn[m] / qn[m])))
    return kl


def entropy_calibration(hist: np.ndarray, amax, levels: int = QUANT_LEVELS):
    """The KL-minimizing threshold. Returns (i, T, S, kl) with T = i * w and
    S = T / 127 in binary32 (w = amax / bins). [PTQ] "2. Entropy Calibration:
    Minimizing Information Loss"."""
    kl = entropy_kl(hist, levels)
    bins = len(hist)
    i_best = levels + int(np.argmin(kl[levels:]))   # first minimum
    w = F32(F32(amax) / F32(bins))
    T = F32(F32(i_best) * w)
    return i_best, T, F32(T / F32(QMAX)), kl


def quantize_act_static_f32(x32: np.ndarray, smooth, scale):
    """q = clamp(round(x' / S), -127, 127) with one fixed scale S for every
    token; returns (q int8 [M, K], S repeated as float32 [M]). S == 0 gives
    zero codes. [PTQ] "1. Min-Max Calibration" (S = T / 127, symmetric
    range); [HALF] "How SmoothQuant prevents outliers in activation tensors"
    (a fixed scale: its codes at S = 0.012 saturate at 127)."""
    x32 = np.asarray(x32, dtype=F32)
    assert x32.ndim == 2 and np.all(np.isfinite(x32)), "finite [M, K] input"
    xs = smooth_activations(x32, smooth)
    S = F32(scale)
    s_tok = np.full(x32.shape[0], S, dtype=F32)
    return quantize_with_scale(xs, s_tok[:, None]), s_tok


def quantize_act_static(x_bf16: np.ndarray, smooth, scale):
    """quantize_act_static_f32 on bf16 activations given as uint16 bit patterns."""
    return quantize_act_static_f32(bf16_to_f32(x_bf16), smooth, scale)


def linear_static(x_bf16: np.ndarray, smooth, scale, wq: np.ndarray, s_chan: np.ndarray):
    """Steps 1-5 with a static activation scale. Returns every intermediate."""
    xq, s_tok = quantize_act_static(x_bf16, smooth, scale)
    acc = gemm_i32(xq, wq)
    y64, y = dequant_epilogue(acc, s_tok, s_chan)
    return {"xq": xq, "s_tok": s_tok, "acc": acc, "y64": y64, "y": y}


# ---------------------------------------------------------------------------
# fused producers: the ops that feed the linears in a Llama block
# ---------------------------------------------------------------------------
#
# [HALF] "How SmoothQuant prevents outliers in activation tensors" places the
# outliers in the RMSNorm weight gamma, and "How the SmoothQuant smoothing
# factor is computed" folds the smoothing division into that weight. A
# producer that ends in the quantizer therefore emits int8 codes and per-token
# scales directly. Readings where the pages say nothing:
#   * RMSNorm: ms = mean of h^2 over the row: the exact sum divided by K
#     and rounded once to binary32; inv = 1 / sqrt(ms + eps), each step one
#     binary32 rounding (sum, square root, division); y = (h * inv) * g with
#     g = gamma / s folded once per channel (binary32); then per-token
#     quantization of y;
#   * residual add: h = bf16(h + r), the binary32 sum of two bf16 values
#     rounded to bf16 (it becomes the new residual stream);
#   * SiLU-gated product: m = bf16((g / (1 + exp(-g))) * u) evaluated in
#     binary64 from the bf16 gate and up values and rounded once (binary32
#     exp is not correctly rounded on either side; in binary64 both sides
#     round to the same bf16 except within 2^-52 of a rounding boundary);
#     then x' = m / s and per-token quantization.

def fold_gamma(gamma, smooth) -> np.ndarray:
    """g = gamma / s (binary32): the smoothing division moved into RMSNorm's
    weight ([HALF] "How the SmoothQuant smoothing factor is computed")."""
    gamma = np.asarray(gamma, dtype=F32)
    if smooth is None:
        return gamma.copy()
    return (gamma / np.asarray(smooth, dtype=F32)).astype(F32)


def residual_add(h_bf16: np.ndarray, r_bf16: np.ndarray) -> np.ndarray:
    """bf16(h + r): binary32 sum of two bf16 values, rounded to bf16."""
    return round_to_bf16(bf16_to_f32(h_bf16) + bf16_to_f32(r_bf16))


def _bf16_square_sum_scaled(row_bits) -> int:
    """The exact sum of the squares of a row of bf16 values, times 2^266,
    as a Python integer.

    A bf16 value with biased exponent E and fraction f is m 2^(e) with the
    integer significand m = f (E = 0) or 128 + f, and e = max(E, 1) - 134,
    so e >= -133 and its square m^2 2^(2e) is an integer multiple of 2^-266.
    """
    b = np.asarray(row_bits, dtype=np.uint16).astype(np.int64)
    E = (b >> 7) & 0xFF
    f = b & 0x7F
    m = np.where(E == 0, f, f | 0x80)
    k = np.maximum(E, 1) - 1                     # e + 133, 0 .. 253
    total = 0
    for kk, mm in zip(k.tolist(), m.tolist()):
        total += (mm * mm) << (2 * kk)
    return total


def _round_ratio_f32(num: int, den: int) -> np.float32:
    """num / den (integers, num >= 0, den > 0) rounded once to binary32,
    nearest with ties to even, with subnormals and overflow to +inf."""
    if num == 0:
        return F32(0)
    e = num.bit_length() - den.bit_length()      # 2^(e-1) < num/den < 2^(e+1)
    if (num << max(-e, 0)) < (den << max(e, 0)):
        e -= 1                                   # now 2^e <= num/den < 2^(e+1)
    qe = max(e - 23, -149)                       # exponent of the last kept bit
    if qe >= 0:
        n, r = divmod(num, den << qe)
        half = den << qe
    else:
        n, r = divmod(num << -qe, den)
        half = den
    if 2 * r > half or (2 * r == half and n % 2 == 1):
        n += 1
    if e >= 128 or n * 2.0 ** qe >= 2.0 ** 128:
        return F32(np.inf)
    return F32(np.ldexp(float(n), qe))           # n < 2^25: exact in both formats


def rms_inverse(h_bf16: np.ndarray, eps) -> np.ndarray:
    """inv[m] = RN32(1 / RN32(sqrt(RN32(ms[m] + eps)))) with ms[m] the mean of
    the squares of row m: the exact sum divided by K, rounded once to
    binary32 (no intermediate rounding of the sum or of the quotient)."""
    h = np.asarray(h_bf16, dtype=np.uint16)
    K = h.shape[1]
    ms = np.array([_round_ratio_f32(_bf16_square_sum_scaled(row), K << 266) for row in h],
                  dtype=F32)
    d = (ms + F32(eps)).astype(F32)
    return (F32(1) / np.sqrt(d).astype(F32)).astype(F32)


def rmsnorm_quantize(h_bf16: np.ndarray, residual, g, eps):
    """RMSNorm with the folded weight g, then per-token quantization.

    With ``residual`` the row first becomes bf16(h + residual). Returns
    (q int8 [M, K], S float32 [M], h_out bf16 [M, K] (the residual stream)).
    """
    h = np.asarray(h_bf16, dtype=np.uint16)
    if residual is not None:
        h = residual_add(h, residual)
    inv = rms_inverse(h, eps)
    y = (bf16_to_f32(h) * inv[:, None]).astype(F32) * np.asarray(g, dtype=F32)[None, :]
    q, S = quantize_act_f32(y.astype(F32))
    return q, S, h


def silu_mul(gu_bf16: np.ndarray) -> np.ndarray:
    """m = bf16(silu(gate) * up) for gu = [gate | up] (bf16 [M, 2I] -> [M, I])."""
    x = bf16_to_f32(gu_bf16).astype(np.float64)
    inter = x.shape[1] // 2
    g, u = x[:, :inter], x[:, inter:2 * inter]
    with np.errstate(over="ignore"):
        m = (g / (1.0 + np.exp(-g))) * u
    return round_to_bf16(m)


def silu_mul_quantize(gu_bf16: np.ndarray, smooth):
    """silu_mul, then the per-token quantizer (x' = m / s). Returns (q, S)."""
    return quantize_act(silu_mul(gu_bf16), smooth)


def chain_forward(x_bf16: np.ndarray, layers, eps=1e-5):
    """A stack of Llama-shaped blocks built from the W8A8 linears (one row
    per token; every step is row-local, so any subset of rows can be run on
    its own). Per layer:

      q, S, h = rmsnorm_quantize(h, pending, g_attn)      pre-attention norm
      y_qkv   = linear(q, S; qkv)
      y_o     = linear(quantize_act(y_qkv[:, :K], s_o); o)  attention stand-in:
                                                             the q slice
      q, S, h = rmsnorm_quantize(h, y_o, g_mlp)           residual + norm
      y_gu    = linear(q, S; gate_up)
      pending = linear(silu_mul_quantize(y_gu, s_down); down)

    and at the end h = residual_add(h, pending). ``layers`` holds per-layer
    dicts with keys g_attn, g_mlp (folded norm weights), s_o, s_down
    (smoothing factors) and (wq, sw) pairs qkv, o, gate_up, down.
    Returns the final residual stream (bf16 [M, K]).
    """
    h = np.asarray(x_bf16, dtype=np.uint16)
    K = h.shape[1]
    pending = None

    def lin(q, S, w):
        return dequant_epilogue(gemm_i32(q, w[0]), S, w[1])[1]

    for L in layers:
        q, S, h = rmsnorm_quantize(h, pending, L["g_attn"], eps)
        y_qkv = lin(q, S, L["qkv"])
        q, S = quantize_act(np.ascontiguousarray(y_qkv[:, :K]), L["s_o"])
        y_o = lin(q, S, L["o"])
        q, S, h = rmsnorm_quantize(h, y_o, L["g_mlp"], eps)
        y_gu = lin(q, S, L["gate_up"])
        q, S = silu_mul_quantize(y_gu, L["s_down"])
        pending = lin(q, S, L["down"])
    return residual_add(h, pending) if pending is not None else h


# ---------------------------------------------------------------------------
# GPTQ: weight quantization with error compensation ([HALF])
# ---------------------------------------------------------------------------
#
# [HALF] "The solution: How GPTQ improves on naive quantization" quantizes a
# layer's weights one input column at a time and, after each, pushes the
# rounding error onto the columns not yet quantized, weighted by the inverse
# of the Hessian H = 2 X^T X of the calibration activations (the paper the
# page cites, Frantar et al. 2022, gives the update through the upper
# Cholesky factor U of H^-1). Readings:
#   * X are the smoothed calibration activations x' = x / s (binary32, then
#     binary64); H = 2 X^T X in binary64;
#   * damping: H + lambda I with lambda = 0.01 * mean(diag H); a column never
#     excited (H_jj = 0) gets H_jj = 1 first;
#   * columns in their natural order; one scale per output channel, the RTN
#     scale max|W'| / 127 of the smoothed bf16 weights, fixed beforehand;
#   * the code of column j is the RTN rule applied to the binary32 value of
#     the updated weight: clamp(round(RN32(w) / s)) in binary32, round half
#     away; then err = (w - q s) / U_jj and w_k -= err * U_jk for k > j, in
#     binary64, a product then a difference (no fused multiply-add).

GPTQ_DAMP = 0.01


def gptq_hessian(x_bf16: np.ndarray, smooth=None) -> np.ndarray:
    """H = 2 X'^T X' (float64 [K, K]) of smoothed calibration activations."""
    xs = smooth_activations(bf16_to_f32(x_bf16), smooth).astype(np.float64)
    return 2.0 * (xs.T @ xs)


def gptq_factor(H: np.ndarray, damp: float = GPTQ_DAMP) -> np.ndarray:
    """U, upper triangular with H_damped^-1 = U^T U (float64 [K, K])."""
    H = np.array(H, dtype=np.float64, copy=True)
    d = np.diag(H).copy()
    d[d == 0] = 1.0
    np.fill_diagonal(H, d)
    H[np.diag_indices_from(H)] += damp * float(np.mean(d))
    Hinv = np.linalg.inv(H)
    Hinv = 0.5 * (Hinv + Hinv.T)
    return np.linalg.cholesky(Hinv).T


def gptq_quantize(w_bf16: np.ndarray, smooth, U: np.ndarray):
    """GPTQ codes of a weight [N, K] given the factor U. Returns
    (Wq int8 [N, K], sw float32 [N]); the scales are RTN's."""
    wb = smooth_weight(w_bf16, smooth)
    w32 = bf16_to_f32(wb)
    sw = absmax_scale(w32, axis=1)
    W = w32.astype(np.float64)
    N, K = W.shape
    q = np.zeros((N, K), np.int8)
    s64 = sw.astype(np.float64)
    for j in range(K):
        qj = quantize_with_scale(W[:, j].astype(F32)[:, None], sw[:, None])[:, 0]
        q[:, j] = qj
        err = (W[:, j] - qj.astype(np.float64) * s64) / U[j, j]
        if j + 1 < K:
            W[:, j + 1:] -= np.outer(err, U[j, j + 1:])
    return q, sw
