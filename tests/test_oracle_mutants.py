"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in the oracle (on the CPU, by monkeypatching a
function of oracle.w8a8_oracle) and runs the pin tests; at least one pin must
fail. The oracle itself is restored after every case.
"""
import numpy as np
import pytest

import test_oracle_pins as P
from oracle import w8a8_oracle as O

F32 = np.float32


def _rint_round(v):                           # ties to even instead of away
    return np.rint(np.asarray(v, dtype=F32)).astype(np.int64)


def _ceil_ties(v):                            # ties toward +inf (sign slip)
    return np.floor(np.asarray(v, dtype=np.float64) + 0.5).astype(np.int64)


def _no_clamp(xs, scale):
    xs = np.asarray(xs, dtype=F32)
    scale = np.asarray(scale, dtype=F32)
    safe = np.where(scale == 0, F32(1), scale)
    v = np.clip(xs / safe, F32(-1e6), F32(1e6))
    q = O.round_half_away(v)
    q = np.where(scale == 0, 0, q)
    return q.astype(np.int64).astype(np.int8)      # wraps 128 to -128


def _recip_mul(xs, scale):                    # x * (1/S) instead of x / S
    xs = np.asarray(xs, dtype=F32)
    scale = np.asarray(scale, dtype=F32)
    safe = np.where(scale == 0, F32(1), scale)
    v = np.clip(xs * (F32(1) / safe), F32(-254), F32(254))
    q = np.clip(O.round_half_away(v), -127, 127)
    return np.where(scale == 0, 0, q).astype(np.int8)


def _signed_max_scale(xs, axis=-1):           # max instead of max |x|
    return (np.max(np.asarray(xs, dtype=F32), axis=axis) / F32(127)).astype(F32)


def _scale_128(xs, axis=-1):
    return (np.max(np.abs(np.asarray(xs, dtype=F32)), axis=axis) / F32(128)).astype(F32)


def _smooth_mul(x32, smooth):                 # multiply instead of divide
    x32 = np.asarray(x32, dtype=F32)
    return x32.copy() if smooth is None else x32 * np.asarray(smooth, dtype=F32)[None, :]


def _gemm_no_transpose(xq, wq):
    return (np.asarray(xq, np.int64) @ np.asarray(wq, np.int64)).astype(np.int32)


def _gemm_wrong_operand(xq, wq):              # W^T X^T: transposed result
    return (np.asarray(wq, np.int64) @ np.asarray(xq, np.int64).T).T.copy().astype(np.int32)[:, ::-1]


def _epilogue_swapped(acc, s_tok, s_chan):
    M, N = np.asarray(acc).shape
    st = np.resize(np.asarray(s_chan, F32), M)
    sc = np.resize(np.asarray(s_tok, F32), N)
    y = np.asarray(acc, np.float64) * st.astype(np.float64)[:, None] * sc.astype(np.float64)[None, :]
    return y, O.round_to_bf16(y)


def _bf16_truncate(v):
    v = np.asarray(v, dtype=np.float64).astype(F32)
    return (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _smoothing_alpha1(a, w):
    a = np.asarray(a, F32)
    w = np.asarray(w, F32)
    ok = (a > 0) & (w > 0)
    return np.where(ok, a / np.where(ok, w, F32(1)), F32(1)).astype(F32)


def _smoothing_inverted(a, w):
    return O.smoothing_factors(w, a)


def _smooth_weight_div(w_bf16, smooth):
    return O.round_to_bf16(O.bf16_to_f32(w_bf16) / np.asarray(smooth, F32)[None, :])


def _quantize_weight_per_input(w32):
    w32 = np.asarray(w32, dtype=F32)
    sw = O.absmax_scale(w32, axis=0)
    return O.quantize_with_scale(w32, sw[None, :]), sw


def _entropy_variant(fold=True, q_from_p=False, spread_all=False):
    def kl_fn(hist, levels=O.QUANT_LEVELS):
        h = np.asarray(hist, dtype=np.float64)
        bins = h.size
        kl = np.full(bins + 1, np.nan)
        for i in range(levels, bins + 1):
            p = h[:i].copy()
            if fold:
                p[i - 1] += h[i:].sum()
            src = p if q_from_p else h[:i]
            q = np.zeros(i)
            for g in range(levels):
                lo, hi = g * i // levels, (g + 1) * i // levels
                seg = src[lo:hi]
                used = np.ones_like(seg, bool) if spread_all else seg > 0
                if used.any():
                    q[lo:hi][used] = seg.sum() / used.sum()
            pn, qn = p / p.sum(), q / max(q.sum(), 1e-300)
            m = pn > 0
            kl[i] = np.inf if np.any(qn[m] == 0) else float(np.sum(pn[m] * np.log(pn[m] / qn[m])))
        return kl
    return kl_fn


def _histogram_rounds(x_bf16, smooth, amax, bins=O.HIST_BINS):   # nearest bin, not floor
    xs = O.smooth_activations(O.bf16_to_f32(x_bf16), smooth)
    a = np.abs(xs).ravel()
    if F32(amax) == 0:
        return np.bincount(np.zeros(a.shape, np.int64), minlength=bins)
    w = F32(F32(amax) / F32(bins))
    idx = np.clip(np.rint(a / w).astype(np.int64), 0, bins - 1)
    return np.bincount(idx, minlength=bins)


def _minmax_no_smoothing(act_absmax, smooth=None):
    a = np.asarray(act_absmax, dtype=F32)
    amax = F32(np.max(a))
    return amax, F32(amax / F32(127))


def _static_uses_token_scale(x32, smooth, scale):
    return O.quantize_act_f32(x32, smooth)


def _epilogue_binary64(acc, s_tok, s_chan):
    y = (np.asarray(acc, dtype=np.float64) * np.asarray(s_tok, F32).astype(np.float64)[:, None]
         * np.asarray(s_chan, F32).astype(np.float64)[None, :])
    return y, O.round_to_bf16(y)


def _rms_sum_not_mean(h_bf16, eps):
    import math
    h = O.bf16_to_f32(h_bf16).astype(np.float64)
    ss = np.array([math.fsum((row * row).tolist()) for row in h]).astype(F32)
    return (F32(1) / np.sqrt((ss + F32(eps)).astype(F32)).astype(F32)).astype(F32)


def _rms_eps_outside(h_bf16, eps):
    import math
    h = O.bf16_to_f32(h_bf16).astype(np.float64)
    ms = np.array([math.fsum((row * row).tolist()) / h.shape[1] for row in h]).astype(F32)
    return (F32(1) / (np.sqrt(ms).astype(F32) + F32(eps))).astype(F32)


def _fold_gamma_multiplies(gamma, smooth):
    g = np.asarray(gamma, F32)
    return g.copy() if smooth is None else (g * np.asarray(smooth, F32)).astype(F32)


def _rms_double_rounding(h_bf16, eps):          # sum rounded to binary64, then /K, then binary32
    import math
    h = O.bf16_to_f32(h_bf16).astype(np.float64)
    ms = np.array([math.fsum((row * row).tolist()) / h.shape[1] for row in h]).astype(F32)
    return (F32(1) / np.sqrt((ms + F32(eps)).astype(F32)).astype(F32)).astype(F32)


def _silu_quantize_drops_smooth(gu_bf16, smooth):
    return O.quantize_act(O.silu_mul(gu_bf16), None)


def _chain_variant(qkv_slice=0, final_residual=True):
    # the block chain with one wiring mistake: o reads another K-column slice
    # of the qkv output, or the last residual add is left out
    def chain(x_bf16, layers, eps=1e-5):
        h = np.asarray(x_bf16, dtype=np.uint16)
        K = h.shape[1]
        pending = None

        def lin(q, S, w):
            return O.dequant_epilogue(O.gemm_i32(q, w[0]), S, w[1])[1]

        for L in layers:
            q, S, h = O.rmsnorm_quantize(h, pending, L["g_attn"], eps)
            y_qkv = lin(q, S, L["qkv"])
            c0 = qkv_slice * K
            q, S = O.quantize_act(np.ascontiguousarray(y_qkv[:, c0:c0 + K]), L["s_o"])
            y_o = lin(q, S, L["o"])
            q, S, h = O.rmsnorm_quantize(h, y_o, L["g_mlp"], eps)
            y_gu = lin(q, S, L["gate_up"])
            q, S = O.silu_mul_quantize(y_gu, L["s_down"])
            pending = lin(q, S, L["down"])
        if pending is None:
            return h
        return O.residual_add(h, pending) if final_residual else pending
    return chain


_real_rmsnorm_quantize = O.rmsnorm_quantize


def _rmsnorm_drops_residual(h_bf16, residual, g, eps):
    return _real_rmsnorm_quantize(h_bf16, None, g, eps)


def _silu_halves_swapped(gu_bf16):
    inter = gu_bf16.shape[1] // 2
    return _real_silu_mul(
        np.concatenate([gu_bf16[:, inter:], gu_bf16[:, :inter]], axis=1))


_real_silu_mul = O.silu_mul


def _gptq_no_feedback(w_bf16, smooth, U):                 # plain RTN
    return O.prepare_weight(w_bf16, smooth)


def _gptq_error_sign(w_bf16, smooth, U):
    wb = O.smooth_weight(w_bf16, smooth)
    w32 = O.bf16_to_f32(wb)
    sw = O.absmax_scale(w32, axis=1)
    W = w32.astype(np.float64)
    q = np.zeros(W.shape, np.int8)
    for j in range(W.shape[1]):
        qj = O.quantize_with_scale(W[:, j].astype(F32)[:, None], sw[:, None])[:, 0]
        q[:, j] = qj
        err = (W[:, j] - qj * sw.astype(np.float64)) / U[j, j]
        W[:, j + 1:] += np.outer(err, U[j, j + 1:])
    return q, sw


def _gptq_factor_lower(H, damp=O.GPTQ_DAMP):                # H^-1 = L L^T, L used as U
    return _real_gptq_factor(H, damp).T


_real_gptq_factor = O.gptq_factor


MUTANTS = {
    "ties_to_even": ("round_half_away", _rint_round),
    "ties_toward_plus_inf": ("round_half_away", _ceil_ties),
    "no_clamp": ("quantize_with_scale", _no_clamp),
    "reciprocal_multiply": ("quantize_with_scale", _recip_mul),
    "signed_max_scale": ("absmax_scale", _signed_max_scale),
    "scale_over_128": ("absmax_scale", _scale_128),
    "smooth_multiplies": ("smooth_activations", _smooth_mul),
    "gemm_no_transpose": ("gemm_i32", _gemm_no_transpose),
    "gemm_wrong_orientation": ("gemm_i32", _gemm_wrong_operand),
    "epilogue_scales_swapped": ("dequant_epilogue", _epilogue_swapped),
    "epilogue_binary64": ("dequant_epilogue", _epilogue_binary64),
    "bf16_truncates": ("round_to_bf16", _bf16_truncate),
    "smoothing_alpha_one": ("smoothing_factors", _smoothing_alpha1),
    "smoothing_inverted": ("smoothing_factors", _smoothing_inverted),
    "smooth_weight_divides": ("smooth_weight", _smooth_weight_div),
    "weight_scale_per_input_channel": ("quantize_weight_f32", _quantize_weight_per_input),
    "entropy_no_saturation_fold": ("entropy_kl", _entropy_variant(fold=False)),
    "entropy_q_from_clipped_p": ("entropy_kl", _entropy_variant(q_from_p=True)),
    "entropy_spread_over_empty_bins": ("entropy_kl", _entropy_variant(spread_all=True)),
    "histogram_nearest_bin": ("abs_histogram", _histogram_rounds),
    "minmax_ignores_smoothing": ("minmax_calibration", _minmax_no_smoothing),
    "static_uses_token_scale": ("quantize_act_static_f32", _static_uses_token_scale),
    "rms_sum_not_mean": ("rms_inverse", _rms_sum_not_mean),
    "rms_eps_outside_sqrt": ("rms_inverse", _rms_eps_outside),
    "rms_mean_rounded_twice": ("rms_inverse", _rms_double_rounding),
    "silu_quantize_drops_smoothing": ("silu_mul_quantize", _silu_quantize_drops_smooth),
    "chain_o_reads_k_slice": ("chain_forward", _chain_variant(qkv_slice=1)),
    "chain_o_reads_v_slice": ("chain_forward", _chain_variant(qkv_slice=2)),
    "chain_drops_last_residual": ("chain_forward", _chain_variant(final_residual=False)),
    "fold_gamma_multiplies": ("fold_gamma", _fold_gamma_multiplies),
    "rmsnorm_drops_residual": ("rmsnorm_quantize", _rmsnorm_drops_residual),
    "silu_halves_swapped": ("silu_mul", _silu_halves_swapped),
    "gptq_no_feedback": ("gptq_quantize", _gptq_no_feedback),
    "gptq_error_sign": ("gptq_quantize", _gptq_error_sign),
    "gptq_factor_lower": ("gptq_factor", _gptq_factor_lower),
}

# --- further plausible mistakes -------------------------------------------

def _residual_subtracts(h_bf16, r_bf16):               # h - r instead of h + r
    return O.round_to_bf16(O.bf16_to_f32(h_bf16) - O.bf16_to_f32(r_bf16))


def _linear_drops_smoothing(x_bf16, smooth, wq, s_chan):
    xq, s_tok = O.quantize_act(x_bf16, None)
    acc = O.gemm_i32(xq, wq)
    y64, y = O.dequant_epilogue(acc, s_tok, s_chan)
    return {"xq": xq, "s_tok": s_tok, "acc": acc, "y64": y64, "y": y}


def _linear_static_drops_smoothing(x_bf16, smooth, scale, wq, s_chan):
    xq, s_tok = O.quantize_act_static(x_bf16, None, scale)
    acc = O.gemm_i32(xq, wq)
    y64, y = O.dequant_epilogue(acc, s_tok, s_chan)
    return {"xq": xq, "s_tok": s_tok, "acc": acc, "y64": y64, "y": y}


def _entropy_last_minimum(hist, amax, levels=O.QUANT_LEVELS):   # ties go to the largest i
    kl = O.entropy_kl(hist, levels)
    bins = len(hist)
    sub = kl[levels:]
    i_best = levels + int(len(sub) - 1 - np.argmin(sub[::-1]))
    w = F32(F32(amax) / F32(bins))
    T = F32(F32(i_best) * w)
    return i_best, T, F32(T / F32(O.QMAX)), kl


def _hessian_not_doubled(x_bf16, smooth=None):          # X'^T X' without the 2
    xs = O.smooth_activations(O.bf16_to_f32(x_bf16), smooth).astype(np.float64)
    return xs.T @ xs


def _hessian_unsmoothed(x_bf16, smooth=None):           # raw activations
    xs = O.bf16_to_f32(x_bf16).astype(np.float64)
    return 2.0 * (xs.T @ xs)


def _act_absmax_signed(x_bf16):                         # max x instead of max |x|
    return np.max(O.bf16_to_f32(x_bf16), axis=0).astype(F32)


def _silu_sign_slip(gu_bf16):                           # g / (1 + e^g)
    x = O.bf16_to_f32(gu_bf16).astype(np.float64)
    inter = x.shape[1] // 2
    g, u = x[:, :inter], x[:, inter:2 * inter]
    with np.errstate(over="ignore"):
        m = (g / (1.0 + np.exp(g))) * u
    return O.round_to_bf16(m)


def _ratio_truncates(num, den):                         # toward zero, not nearest
    q = O._round_ratio_f32(num, den)
    exact = num / den
    if float(q) > exact and q > 0:
        return np.nextafter(q, F32(0))
    return q


MUTANTS.update({
    "residual_add_subtracts": ("residual_add", _residual_subtracts),
    "linear_drops_smoothing": ("linear", _linear_drops_smoothing),
    "linear_static_drops_smoothing": ("linear_static", _linear_static_drops_smoothing),
    "entropy_last_minimum": ("entropy_calibration", _entropy_last_minimum),
    "hessian_not_doubled": ("gptq_hessian", _hessian_not_doubled),
    "hessian_unsmoothed": ("gptq_hessian", _hessian_unsmoothed),
    "act_absmax_signed": ("act_channel_absmax", _act_absmax_signed),
    "silu_sign_slip": ("silu_mul", _silu_sign_slip),
    "mean_square_truncates": ("_round_ratio_f32", _ratio_truncates),
})


PINS = [getattr(P, n) for n in dir(P)
        if n.startswith("test_") and callable(getattr(P, n))]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception:                         # assertion or shape error
            caught.append(pin.__name__)
    assert caught, f"mutant {name} survived every pin"

