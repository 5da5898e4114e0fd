"""GPU parity of the fused producers and of the Llama-shaped block chain.

The producers (residual add + RMSNorm + quantize, SiLU-gated product +
quantize) and the small helpers must match the oracle bit for bit. The chain
(32 layers x 4 W8A8 linears on a ragged batch of 3000 tokens) runs in full on
the GPU; every step is row-local, so the oracle follows sampled token rows
through all 32 layers on its own and the final residual stream of those rows
must match bit for bit.
"""
import numpy as np
import pytest

import int8_w8a8_quantized_token_amd as W
from int8_w8a8_quantized_token_amd import workloads as WL
from oracle import w8a8_oracle as O
from gpu_util import dev, dev_bf16, host, torch

pytestmark = pytest.mark.gpu

F32 = np.float32
EPS = 1e-5


def act(M, K, tag, frac=0.01, mult=20.0):
    return WL.activations(M, K, "producers", tag, frac=frac, mult=mult)


def gamma_with_outliers(K, tag):
    g = np.ones(K, F32)
    g[WL.outlier_channels(K, 0.01, tag)] = 20.0
    return g


@pytest.mark.parametrize("M,K", [(1, 4096), (16, 4096), (64, 14336), (513, 4096),
                                 (1100, 4096 + 16), (3, 65536)])
@pytest.mark.parametrize("add", [False, True], ids=["norm", "add+norm"])
def test_rmsnorm_quantize_bit_exact(M, K, add):
    h = act(M, K, "rms-h")
    res = WL.activations(M, K, "producers", "rms-r", frac=0.0, mult=1.0) if add else None
    s = np.exp(WL.rng("rms-s", K).uniform(-1, 1, K)).astype(F32)
    g = O.fold_gamma(gamma_with_outliers(K, "rms"), s)
    q_ref, s_ref, h_ref = O.rmsnorm_quantize(h, res, g, EPS)
    d_h = dev_bf16(h)
    xq, st = W.w8a8_rmsnorm_quantize(d_h, dev(g), EPS,
                                     residual=dev_bf16(res) if add else None)
    torch().cuda.synchronize()
    np.testing.assert_array_equal(host(d_h), h_ref)
    np.testing.assert_array_equal(host(st).view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(host(xq), q_ref)


def test_rmsnorm_quantize_edge_rows():
    K = 256
    rows = np.zeros((6, K), F32)
    rows[1, :] = 1.0                                     # mean square 1
    rows[2, ::3] = 3e38                                  # squares overflow binary32, not binary64
    rows[3, :] = 2.0 ** -130                             # subnormal values
    rows[4, 5] = -7.0                                    # one nonzero value
    rows[5, :] = np.linspace(-1000, 1000, K)
    h = O.round_to_bf16(rows)
    g = np.exp(WL.rng("rms-edge", K).uniform(-2, 2, K)).astype(F32)
    # eps = 0 only where the mean square is a positive binary32 value
    for eps, sel in ((EPS, [0, 1, 2, 3, 4, 5]), (0.0, [1, 4, 5])):
        q_ref, s_ref, _ = O.rmsnorm_quantize(h[sel], None, g, eps)
        xq, st = W.w8a8_rmsnorm_quantize(dev_bf16(h[sel]), dev(g), eps)
        torch().cuda.synchronize()
        np.testing.assert_array_equal(host(st).view(np.uint32), s_ref.view(np.uint32))
        np.testing.assert_array_equal(host(xq), q_ref)


# Pairs of bf16 values whose mean square over K lies exactly halfway between
# two binary32 values (checked below with exact rationals). For K = 16 and
# 4096 the tie goes down to the even neighbour, so a tiny extra square (which
# lifts the mean) changes the rounding and, at eps = 1e-5, the scale; for
# 14336 = 7 * 2^11 the tie itself goes up.
MIDPOINT_PAIRS = {16: (2.421875, 0.05615234375), 4096: (129.0, 4.40625),
                  14336: (175.0, 2.078125)}


@pytest.mark.parametrize("K", sorted(MIDPOINT_PAIRS))
@pytest.mark.parametrize("M", [4, 600])
@pytest.mark.parametrize("add", [False, True], ids=["norm", "add+norm"])
def test_rmsnorm_mean_rounded_once_near_midpoints(K, M, add):
    # A tiny square anywhere in the row (in another thread's vector too) puts
    # the exact mean just above the midpoint, so its one rounding goes up;
    # without it the mean is the tie and goes to even. Both take the exact
    # comparison in the kernel. Random rows fill the rest (600 rows take the
    # 256/512-thread kernels).
    from fractions import Fraction
    a, b = MIDPOINT_PAIRS[K]
    mean = (Fraction(a) ** 2 + Fraction(b) ** 2) / K
    assert mean.denominator & (mean.denominator - 1) == 0
    assert mean.numerator % 2 == 1 and mean.numerator.bit_length() == 25   # a binary32 midpoint
    tie_goes_down = mean.numerator % 4 == 1
    rows = O.bf16_to_f32(act(M, K, "rms-mid")).copy()
    rows[:4] = 0.0
    rows[:4, :2] = [a, b]
    rows[0, 2] = 2.0 ** -60
    rows[2, K - 1] = -(2.0 ** -133)
    rows[3, 0] = -a
    rows[3, K // 2 + 3] = 2.0 ** -60
    h = O.round_to_bf16(rows)
    assert np.array_equal(O.bf16_to_f32(h[:4]), rows[:4])
    res = np.zeros_like(h) if add else None
    g = np.ones(K, F32)
    for eps in (EPS, 0.0):
        q_ref, s_ref, _ = O.rmsnorm_quantize(h, res, g, eps)
        if eps == EPS and tie_goes_down:
            assert s_ref[0] != s_ref[1]          # the tiny square decides the scale
        xq, st = W.w8a8_rmsnorm_quantize(dev_bf16(h), dev(g), eps,
                                         residual=dev_bf16(res) if add else None)
        torch().cuda.synchronize()
        np.testing.assert_array_equal(host(st).view(np.uint32), s_ref.view(np.uint32))
        np.testing.assert_array_equal(host(xq), q_ref)


@pytest.mark.parametrize("M,I", [(1, 14336), (16, 14336), (64, 2048), (600, 14336 + 16),
                                 (700, 512)])
@pytest.mark.parametrize("use_smooth", [False, True], ids=["plain", "smooth"])
def test_silu_mul_quantize_bit_exact(M, I, use_smooth):
    gu = WL.activations(M, 2 * I, "producers", "silu", frac=0.01, mult=20.0)
    smooth = np.exp(WL.rng("silu-s", I).uniform(-1, 1, I)).astype(F32) if use_smooth else None
    q_ref, s_ref = O.silu_mul_quantize(gu, smooth)
    xq, st = W.w8a8_silu_mul_quantize(dev_bf16(gu), dev(smooth) if use_smooth else None)
    torch().cuda.synchronize()
    np.testing.assert_array_equal(host(st).view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(host(xq), q_ref)


def test_silu_mul_extremes():
    inter = 64
    gate = np.linspace(-120, 120, inter).astype(F32)
    gate[:6] = [0.0, -0.0, 1e37, -1e37, 1e-38, -88.0]
    up = np.linspace(-4, 4, inter).astype(F32)
    gu = O.round_to_bf16(np.stack([np.concatenate([gate, up]), np.concatenate([up, gate])]))
    q_ref, s_ref = O.silu_mul_quantize(gu, None)
    xq, st = W.w8a8_silu_mul_quantize(dev_bf16(gu))
    torch().cuda.synchronize()
    np.testing.assert_array_equal(host(st).view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(host(xq), q_ref)


def test_fold_gamma_and_residual_add():
    K = 4096 + 16
    gamma = gamma_with_outliers(K, "fold")
    s = np.exp(WL.rng("fold-s", K).uniform(-3, 3, K)).astype(F32)
    g = W.w8a8_fold_gamma(dev(gamma), dev(s))
    a, b = act(33, K, "add-a"), act(33, K, "add-b", frac=0.0, mult=1.0)
    d_a = dev_bf16(a)
    W.w8a8_residual_add(d_a, dev_bf16(b))
    torch().cuda.synchronize()
    np.testing.assert_array_equal(host(g).view(np.uint32), O.fold_gamma(gamma, s).view(np.uint32))
    np.testing.assert_array_equal(host(d_a), O.residual_add(a, b))


# ---------------------------------------------------------------------------
# the Llama-shaped block chain
# ---------------------------------------------------------------------------

HIDDEN, INTER = 4096, 14336
SHAPES = {"qkv": (6144, HIDDEN), "o": (HIDDEN, HIDDEN), "gate_up": (2 * INTER, HIDDEN),
          "down": (HIDDEN, INTER)}
NAME = "llama8b_chain"


@pytest.fixture(scope="module")
def chain_params():
    """One seeded weight set and smoothing vector per projection, shared by
    every layer; each side prepares its own copy (oracle on the host, the
    library's prep kernels on the GPU)."""
    wl = WL.WORKLOADS[NAME]
    gamma = gamma_with_outliers(HIDDEN, NAME)
    host_p, dev_p = {}, {}
    for proj, (N, K) in SHAPES.items():
        w = WL.weights(N, K, wl.w_std, NAME, proj, 0)
        # the qkv and gate_up inputs carry the norm's outlier channels
        outl = WL.outlier_channels(K, 0.01, NAME) if proj in ("qkv", "gate_up") else []
        xcal = WL.activations(256, K, NAME, "cal", proj, outliers=np.asarray(outl, np.int64))
        s = O.smoothing_factors(O.act_channel_absmax(xcal), O.weight_channel_absmax(w))
        host_p[proj] = (O.prepare_weight(w, s), s)
        d_w = dev_bf16(w)
        d_s = W.w8a8_smoothing_factors(W.w8a8_channel_absmax(dev_bf16(xcal)),
                                       W.w8a8_channel_absmax(d_w))
        dev_p[proj] = (W.w8a8_quantize_weight(d_w, d_s), d_s)
        del d_w
    torch().cuda.synchronize()
    for proj in SHAPES:                        # the two preparations agree
        np.testing.assert_array_equal(host(dev_p[proj][1]), host_p[proj][1])
        np.testing.assert_array_equal(host(dev_p[proj][0][1]), host_p[proj][0][1])
    layer = {"g_attn": O.fold_gamma(gamma, host_p["qkv"][1]),
             "g_mlp": O.fold_gamma(gamma, host_p["gate_up"][1]),
             "s_o": host_p["o"][1], "s_down": host_p["down"][1],
             **{p: host_p[p][0] for p in SHAPES}}
    d_gamma = dev(gamma)
    d_layer = {"g_attn": W.w8a8_fold_gamma(d_gamma, dev_p["qkv"][1]),
               "g_mlp": W.w8a8_fold_gamma(d_gamma, dev_p["gate_up"][1]),
               "s_o": dev_p["o"][1], "s_down": dev_p["down"][1],
               **{p: dev_p[p][0] for p in SHAPES}}
    return layer, d_layer


def gpu_chain(x, L, layers):
    """The chain on the GPU through the C ABI (all rows)."""
    t = torch()
    M = x.shape[0]
    h = x.clone()
    y_qkv = t.empty((M, SHAPES["qkv"][0]), dtype=t.bfloat16, device="cuda")
    y_o = t.empty((M, HIDDEN), dtype=t.bfloat16, device="cuda")
    y_gu = t.empty((M, 2 * INTER), dtype=t.bfloat16, device="cuda")
    y_d = t.empty((M, HIDDEN), dtype=t.bfloat16, device="cuda")
    pending = None
    for _ in range(layers):
        xq, st = W.w8a8_rmsnorm_quantize(h, L["g_attn"], EPS, residual=pending)
        W.w8a8_gemm(xq, st, *L["qkv"], y=y_qkv)
        xq, st = W.w8a8_quantize_act(y_qkv[:, :HIDDEN], L["s_o"])
        W.w8a8_gemm(xq, st, *L["o"], y=y_o)
        xq, st = W.w8a8_rmsnorm_quantize(h, L["g_mlp"], EPS, residual=y_o)
        W.w8a8_gemm(xq, st, *L["gate_up"], y=y_gu)
        xq, st = W.w8a8_silu_mul_quantize(y_gu, L["s_down"])
        W.w8a8_gemm(xq, st, *L["down"], y=y_d)
        pending = y_d
    W.w8a8_residual_add(h, pending)
    return h


def test_chain_two_layers_all_rows(chain_params):
    layer, d_layer = chain_params
    x = WL.activations(64, HIDDEN, NAME, "x-small", outliers=WL.outlier_channels(HIDDEN, 0.01, NAME))
    want = O.chain_forward(x, [layer] * 2, EPS)
    got = host(gpu_chain(dev_bf16(x), d_layer, 2))
    torch().cuda.synchronize()
    np.testing.assert_array_equal(got, want)


def test_chain_config_full_size_sampled_rows(chain_params):
    # 8 sequences, 3000 tokens, 32 layers; the oracle follows the first and
    # last token of every sequence
    layer, d_layer = chain_params
    wl = WL.WORKLOADS[NAME]
    lengths = WL.ragged_lengths(wl.ms[0], 8, NAME)
    assert sum(lengths) == 3000 and min(lengths) >= 1
    x = WL.activations(3000, HIDDEN, NAME, "x", outliers=WL.outlier_channels(HIDDEN, 0.01, NAME))
    out = host(gpu_chain(dev_bf16(x), d_layer, 32))
    torch().cuda.synchronize()
    ends = np.cumsum(lengths)
    rows = sorted(set(np.concatenate([ends - np.array(lengths), ends - 1]).tolist()))
    want = O.chain_forward(x[rows], [layer] * 32, EPS)
    np.testing.assert_array_equal(out[rows], want)
    h = O.bf16_to_f32(out)
    assert np.all(np.isfinite(h))


# Shapes that reach every (threads, vectors per thread) instance of the two
# producers that the launch rule can pick (256 threads with 1, 2 or 4
# vectors of 8 per thread, 512 with 4 or 8, 1024 with 1, 2, 4 or 8; the
# fixed shapes here and in the tests above), plus seeded random shapes. Every code and scale is compared with the oracle's.
_FIXED_SHAPES = [(700, 6144), (520, 16384), (530, 30000), (520, 40000), (600, 1024),
                 (2, 160), (511, 12000), (300, 20000)]
_r = np.random.default_rng(20240)
PRODUCER_SHAPES = _FIXED_SHAPES + [(int(_r.integers(1, 700)), 16 * int(_r.integers(1, 1300)))
                                   for _ in range(4)]


def _threads_and_vectors(M, K):
    """The producers' launch rule, restated for the test ids."""
    bs = 1024 if M <= 512 else (512 if K > 8192 else 256)
    while bs < 1024 and -(-(K // 8) // bs) > 8:
        bs *= 2
    per = -(-(K // 8) // bs)
    return bs, 1 if per <= 1 else 2 if per <= 2 else 4 if per <= 4 else 8


@pytest.mark.parametrize("M,K", PRODUCER_SHAPES,
                         ids=[f"M{m}-K{k}-bs{_threads_and_vectors(m, k)[0]}"
                              f"-nv{_threads_and_vectors(m, k)[1]}" for m, k in PRODUCER_SHAPES])
def test_producers_every_launch_shape(M, K):
    print(f"\n[producers] M={M} K={K} {_threads_and_vectors(M, K)}", flush=True)
    h = act(M, K, f"shape-h-{M}-{K}")
    res = WL.activations(M, K, "producers", f"shape-r-{M}-{K}", frac=0.0, mult=1.0)
    s = np.exp(WL.rng("shape-s", K).uniform(-1, 1, K)).astype(F32)
    g = O.fold_gamma(gamma_with_outliers(K, "shape"), s)
    for add in (False, True):
        q_ref, s_ref, h_ref = O.rmsnorm_quantize(h, res if add else None, g, EPS)
        d_h = dev_bf16(h)
        xq, st = W.w8a8_rmsnorm_quantize(d_h, dev(g), EPS,
                                         residual=dev_bf16(res) if add else None)
        torch().cuda.synchronize()
        np.testing.assert_array_equal(host(d_h), h_ref)
        np.testing.assert_array_equal(host(st).view(np.uint32), s_ref.view(np.uint32))
        np.testing.assert_array_equal(host(xq), q_ref)
    gu = WL.activations(M, 2 * K, "producers", f"shape-gu-{M}-{K}", frac=0.01, mult=20.0)
    for smooth in (None, s):
        q_ref, s_ref = O.silu_mul_quantize(gu, smooth)
        xq, st = W.w8a8_silu_mul_quantize(dev_bf16(gu), dev(smooth) if smooth is not None else None)
        torch().cuda.synchronize()
        np.testing.assert_array_equal(host(st).view(np.uint32), s_ref.view(np.uint32))
        np.testing.assert_array_equal(host(xq), q_ref)
