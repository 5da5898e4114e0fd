"""Parity at the full benchmark sizes, in the launch configuration the
benchmark times (w8a8_linear on the whole [M, K] x [N, K] problem).

Both sides start from the same seeded bf16 X and W and each prepares its own
smoothing factors and int8 weights. The oracle then recomputes a sample: all
K smoothing factors, a sample of weight rows (their int8 codes and scales),
a sample of token rows (codes and scales), and the int32 accumulators (of
w8a8_gemm_i32 on the whole problem) and bf16 outputs on the sampled rows x
sampled columns. Rows of both quantizations are independent of each other,
so a sampled row is checked exactly. Properties that hold at any size are
checked on the whole output. The tests further below compare every element
of every one of those launches: the Llama-3.1-8B decode, prefill and chain
projections and the Llama-3-70B projections.
"""
import numpy as np
import pytest

import int8_w8a8_quantized_token_amd as W
from int8_w8a8_quantized_token_amd import workloads as WL
from oracle import w8a8_oracle as O
from gpu_util import check_bf16, dev_bf16, host, torch

pytestmark = pytest.mark.gpu

CASES = []
for wl_name in ("llama8b_decode", "llama8b_prefill", "llama70b", "llama8b_chain"):
    wl = WL.WORKLOADS[wl_name]
    for proj, N, K in wl.shapes:
        for M in wl.ms:
            CASES.append((wl_name, proj, N, K, M))

_cache = {}


def weight_case(wl, proj, N, K):
    """(w_bf16 host, w device, oracle weight absmax) for one projection, cached
    for the M values of the same workload (one entry kept at a time)."""
    key = (wl.name, proj)
    if key not in _cache:
        _cache.clear()
        w = WL.weights(N, K, wl.w_std, wl.name, proj, 0)
        aw = np.zeros(K, np.float32)
        for r0 in range(0, N, 4096):                # max over row chunks = max over rows
            aw = np.maximum(aw, O.weight_channel_absmax(w[r0:r0 + 4096]))
        _cache[key] = (w, dev_bf16(w), aw)
    return _cache[key]


@pytest.mark.parametrize("wl_name,proj,N,K,M", CASES,
                         ids=[f"{c[0]}-{c[1]}-M{c[4]}" for c in CASES])
def test_full_size_linear_sampled(wl_name, proj, N, K, M):
    wl = WL.WORKLOADS[wl_name]
    print(f"\n[full-size] {wl_name} {proj} M={M} N={N} K={K}", flush=True)
    w, wd, aw_ref = weight_case(wl, proj, N, K)
    out = WL.outlier_channels(K, wl.outlier_frac, wl.name)
    x = WL.activations(M, K, wl.name, proj, 0, outliers=out, mult=wl.outlier_mult)
    xd = dev_bf16(x)

    # GPU: calibrate on this X, prepare the weight, run the layer
    s = W.w8a8_smoothing_factors(W.w8a8_channel_absmax(xd), W.w8a8_channel_absmax(wd))
    wq, sw = W.w8a8_quantize_weight(wd, s)
    y = W.w8a8_linear(xd, s, wq, sw)
    xq, st = W.w8a8_quantize_act(xd, s)
    r = WL.rng("sample", wl_name, proj, M)
    ms = np.unique(np.concatenate([[0, M - 1], r.choice(M, size=min(M, 12), replace=False)]))
    ns = np.unique(np.concatenate([[0, N - 1], r.choice(N, size=min(N, 64), replace=False)]))
    ms_d = torch().from_numpy(ms).cuda()
    ns_d = torch().from_numpy(ns).cuda()
    # int32 from the whole problem (the kernel route of the timed launch),
    # then the sampled rows and columns
    acc = W.w8a8_gemm_i32(xq, wq).index_select(0, ms_d).index_select(1, ns_d)
    torch().cuda.synchronize()

    # oracle on the sample
    s_ref = O.smoothing_factors(O.act_channel_absmax(x), aw_ref)
    np.testing.assert_array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    wq_ref, sw_ref = O.prepare_weight(w[ns], s_ref)
    np.testing.assert_array_equal(host(sw)[ns].view(np.uint32), sw_ref.view(np.uint32))
    np.testing.assert_array_equal(host(wq.index_select(0, ns_d)), wq_ref)
    xq_ref, st_ref = O.quantize_act(x[ms], s_ref)
    xq_h = host(xq)
    np.testing.assert_array_equal(host(st)[ms].view(np.uint32), st_ref.view(np.uint32))
    np.testing.assert_array_equal(xq_h[ms], xq_ref)
    acc_ref = O.gemm_i32(xq_ref, wq_ref)
    np.testing.assert_array_equal(host(acc), acc_ref)
    y_h = host(y)
    y64, y_ref = O.dequant_epilogue(acc_ref, st_ref, sw_ref)
    check_bf16(y_h[np.ix_(ms, ns)], y64, y_ref)

    # properties of the whole output
    assert xq_h.min() >= -127
    rowmax = np.abs(xq_h.astype(np.int16)).max(axis=1)
    assert np.all((rowmax == 127) | (host(st) == 0))
    yf = (y_h.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isfinite(yf))


# ---------------------------------------------------------------------------
# every element of the full problem
# ---------------------------------------------------------------------------
#
# The launches the benchmark times, compared in full: all 16 Llama-3.1-8B
# decode (projection, M) pairs, the four projections at M = 4096 (the prefill
# kernel's 256 x 256 tile, and 192 x 256 for qkv) and at the chain's 3000
# tokens (256 x 192 tiles for o and down). The int32 accumulators come
# from w8a8_gemm_i32 on the whole problem (the same kernel route as
# w8a8_gemm at that shape) and every one is compared with the oracle's
# integer GEMM; every code, scale and bf16 output of w8a8_linear is compared
# with the oracle's. The oracle prepares the whole weight (row blocks are
# independent). Smoothing factors are calibrated on the projection's
# activations at the largest M of the workload and shared by its smaller M.

EVERY_CASES = ([("llama8b_decode", p, N, K, M) for p, N, K in WL.LLAMA31_8B for M in (1, 4, 16, 64)]
               + [("llama8b_prefill", p, N, K, 4096) for p, N, K in WL.LLAMA31_8B]
               + [("llama8b_chain", p, N, K, 3000) for p, N, K in WL.LLAMA31_8B])

_prep = {}


def prepared(wl, proj, N, K):
    """Both sides' smoothing factors and int8 weights for one projection,
    checked against each other in full once (one entry kept at a time)."""
    key = (wl.name, proj)
    if key in _prep:
        return _prep[key]
    _prep.clear()
    out = WL.outlier_channels(K, wl.outlier_frac, wl.name)
    xcal = WL.activations(max(wl.ms), K, wl.name, proj, 0, outliers=out, mult=wl.outlier_mult)
    w = WL.weights(N, K, wl.w_std, wl.name, proj, 0)
    wd = dev_bf16(w)
    s = W.w8a8_smoothing_factors(W.w8a8_channel_absmax(dev_bf16(xcal)), W.w8a8_channel_absmax(wd))
    wq, sw = W.w8a8_quantize_weight(wd, s)
    del wd
    aw = np.zeros(K, np.float32)
    for r0 in range(0, N, 4096):
        aw = np.maximum(aw, O.weight_channel_absmax(w[r0:r0 + 4096]))
    s_ref = O.smoothing_factors(O.act_channel_absmax(xcal), aw)
    wq_ref = np.empty((N, K), np.int8)
    sw_ref = np.empty(N, np.float32)
    for r0 in range(0, N, 2048):
        wq_ref[r0:r0 + 2048], sw_ref[r0:r0 + 2048] = O.prepare_weight(w[r0:r0 + 2048], s_ref)
    torch().cuda.synchronize()
    np.testing.assert_array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(host(sw).view(np.uint32), sw_ref.view(np.uint32))
    np.testing.assert_array_equal(host(wq), wq_ref)
    _prep[key] = (s, wq, sw, s_ref, wq_ref, sw_ref)
    return _prep[key]


@pytest.mark.parametrize("wl_name,proj,N,K,M", EVERY_CASES,
                         ids=[f"{c[0]}-{c[1]}-M{c[4]}" for c in EVERY_CASES])
def test_full_size_every_element(wl_name, proj, N, K, M):
    wl = WL.WORKLOADS[wl_name]
    print(f"\n[every element] {wl_name} {proj} M={M} N={N} K={K}", flush=True)
    s, wq, sw, s_ref, wq_ref, sw_ref = prepared(wl, proj, N, K)
    out = WL.outlier_channels(K, wl.outlier_frac, wl.name)
    x = WL.activations(M, K, wl.name, proj, 0, outliers=out, mult=wl.outlier_mult)
    xd = dev_bf16(x)
    y = W.w8a8_linear(xd, s, wq, sw)
    xq, st = W.w8a8_quantize_act(xd, s)
    acc = W.w8a8_gemm_i32(xq, wq)
    torch().cuda.synchronize()

    xq_ref, st_ref = O.quantize_act(x, s_ref)
    np.testing.assert_array_equal(host(st).view(np.uint32), st_ref.view(np.uint32))
    np.testing.assert_array_equal(host(xq), xq_ref)
    acc_ref = O.gemm_i32(xq_ref, wq_ref)
    np.testing.assert_array_equal(host(acc), acc_ref)
    del acc
    y64, y_ref = O.dequant_epilogue(acc_ref, st_ref, sw_ref)
    check_bf16(host(y), y64, y_ref)


# The static-scale linear (one activation scale for every token) on every
# decode launch the benchmark's static line times, and the Llama-3-70B decode
# projections o and down at 32 tokens, each compared in full. The static
# scale is the oracle's min-max calibration on the calibration activations,
# handed to both sides.

STATIC_CASES = [("llama8b_decode", p, N, K, M) for p, N, K in WL.LLAMA31_8B for M in (1, 4, 16, 64)]


@pytest.mark.parametrize("wl_name,proj,N,K,M", STATIC_CASES,
                         ids=[f"{c[0]}-{c[1]}-M{c[4]}" for c in STATIC_CASES])
def test_full_size_static_linear_every_element(wl_name, proj, N, K, M):
    wl = WL.WORKLOADS[wl_name]
    print(f"\n[static, every element] {wl_name} {proj} M={M} N={N} K={K}", flush=True)
    s, wq, sw, s_ref, wq_ref, sw_ref = prepared(wl, proj, N, K)
    out = WL.outlier_channels(K, wl.outlier_frac, wl.name)
    xcal = WL.activations(max(wl.ms), K, wl.name, proj, 0, outliers=out, mult=wl.outlier_mult)
    _, S = O.minmax_calibration(O.act_channel_absmax(xcal), s_ref)
    x = WL.activations(M, K, wl.name, proj, 0, outliers=out, mult=wl.outlier_mult)
    xd = dev_bf16(x)
    Sd = torch().tensor([float(S)], dtype=torch().float32, device="cuda")
    y = W.w8a8_linear_static(xd, s, Sd, wq, sw)
    xq, st = W.w8a8_quantize_act_static(xd, s, Sd)
    torch().cuda.synchronize()
    ref = O.linear_static(x, s_ref, S, wq_ref, sw_ref)
    np.testing.assert_array_equal(host(st).view(np.uint32), ref["s_tok"].view(np.uint32))
    np.testing.assert_array_equal(host(xq), ref["xq"])
    check_bf16(host(y), ref["y64"], ref["y"])


# The four Llama-3-70B projections at both of the workload's token counts:
# 32 (mid kernel) and 2048 (prefill kernel), every element.
B70_CASES = [("llama70b", p, N, K, M) for p, N, K in WL.LLAMA3_70B for M in (32, 2048)]


@pytest.mark.parametrize("wl_name,proj,N,K,M", B70_CASES,
                         ids=[f"{c[0]}-{c[1]}-M{c[4]}" for c in B70_CASES])
def test_full_size_70b_every_element(wl_name, proj, N, K, M):
    test_full_size_every_element(wl_name, proj, N, K, M)
