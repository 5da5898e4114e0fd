"""The layer under HIP graph capture, the way the benchmark times it: one
captured w8a8_linear replayed several times, with new inputs written eagerly
between replays; every replay must equal an eager call on the same inputs
bit for bit, and the first also the oracle."""
import numpy as np
import pytest

import int8_w8a8_quantized_token_amd as W
from int8_w8a8_quantized_token_amd import workloads as WL
from oracle import w8a8_oracle as O
from gpu_util import check_bf16, dev, dev_bf16, host, torch

pytestmark = pytest.mark.gpu

# one token on a short, narrow weight (one-launch kernel); decode sizes on the
# LDS-staged GEMM at short and deep K; enough tokens for the prefill kernel
GRAPH_SHAPES = [(1, 4096, 4096), (4, 6144, 4096), (64, 1024, 14336), (600, 512, 4096)]


def act(M, K, tag, replay):
    outl = WL.outlier_channels(K, 0.01, "graph", tag)
    return WL.activations(M, K, "graph", tag, replay, outliers=outl, mult=20.0)


@pytest.mark.parametrize("M,N,K", GRAPH_SHAPES, ids=[f"M{m}_N{n}_K{k}" for m, n, k in GRAPH_SHAPES])
def test_linear_graph_replays(M, N, K):
    t = torch()
    tag = f"{M}x{N}x{K}"
    x0 = act(M, K, tag, 0)
    w = WL.weights(N, K, 0.02, "graph", tag)
    s = O.smoothing_factors(O.act_channel_absmax(x0), O.weight_channel_absmax(w))
    wq, sw = O.prepare_weight(w, s)
    s_d, wq_d, sw_d = dev(s), dev(wq), dev(sw)
    x_d = dev_bf16(x0)
    y = t.empty((M, N), dtype=t.bfloat16, device="cuda")
    ws = t.empty((W.w8a8_linear_workspace_bytes(M, K),), dtype=t.uint8, device="cuda")

    def call():
        W.w8a8_linear(x_d, s_d, wq_d, sw_d, y=y, workspace=ws)

    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        call()
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        call()
    t.cuda.synchronize()

    for replay in range(4):
        x = x0 if replay == 0 else act(M, K, tag, replay)
        x_d.copy_(dev_bf16(x))                  # eager write between replays
        y.fill_(7.0)
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        got = host(y).copy()
        want = host(W.w8a8_linear(x_d, s_d, wq_d, sw_d))
        t.cuda.synchronize()
        np.testing.assert_array_equal(got, want, err_msg=f"replay {replay}")
        if replay == 0:
            ref = O.linear(x, s, wq, sw)
            check_bf16(got, ref["y64"], ref["y"], what=f"replay {replay}")


STATIC_SHAPES = [(1, 4096, 4096), (16, 6144, 4096), (600, 512, 4096)]


@pytest.mark.parametrize("M,N,K", STATIC_SHAPES, ids=[f"M{m}_N{n}_K{k}" for m, n, k in STATIC_SHAPES])
def test_linear_static_graph_replays(M, N, K):
    t = torch()
    tag = f"static{M}x{N}x{K}"
    x0 = act(M, K, tag, 0)
    w = WL.weights(N, K, 0.02, "graph", tag)
    s = O.smoothing_factors(O.act_channel_absmax(x0), O.weight_channel_absmax(w))
    wq, sw = O.prepare_weight(w, s)
    _, scale = O.minmax_calibration(O.act_channel_absmax(x0), s)
    scale = np.asarray([scale], np.float32).reshape(1)
    s_d, sc_d, wq_d, sw_d = dev(s), dev(scale), dev(wq), dev(sw)
    x_d = dev_bf16(x0)
    y = t.empty((M, N), dtype=t.bfloat16, device="cuda")
    ws = t.empty((W.w8a8_linear_workspace_bytes(M, K),), dtype=t.uint8, device="cuda")
    g = capture(lambda: W.w8a8_linear_static(x_d, s_d, sc_d, wq_d, sw_d, y=y, workspace=ws))
    for replay in range(4):
        x = x0 if replay == 0 else act(M, K, tag, replay)
        x_d.copy_(dev_bf16(x))
        y.fill_(7.0)
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        got = host(y).copy()
        want = host(W.w8a8_linear_static(x_d, s_d, sc_d, wq_d, sw_d))
        t.cuda.synchronize()
        np.testing.assert_array_equal(got, want, err_msg=f"replay {replay}")
        if replay == 0:
            ref = O.linear_static(x, s, scale[0], wq, sw)
            check_bf16(got, ref["y64"], ref["y"], what="static replay 0")


def test_producers_graph_replays():
    # the chain's producers as one captured sequence: residual add + RMSNorm
    # (h updated in place), then the SiLU-gated product, both quantized
    t = torch()
    M, K, I = 300, 4096, 14336
    gamma = (WL.rng("graph", "gamma", K).random(K, dtype=np.float32) + 0.5).astype(np.float32)
    sm = (WL.rng("graph", "smooth", I).random(I, dtype=np.float32) + 0.5).astype(np.float32)
    g_d, sm_d = dev(gamma), dev(sm)
    h_d = t.empty((M, K), dtype=t.bfloat16, device="cuda")
    r_d = t.empty((M, K), dtype=t.bfloat16, device="cuda")
    gu_d = t.empty((M, 2 * I), dtype=t.bfloat16, device="cuda")
    q1 = t.empty((M, K), dtype=t.int8, device="cuda")
    s1 = t.empty((M,), dtype=t.float32, device="cuda")
    q2 = t.empty((M, I), dtype=t.int8, device="cuda")
    s2 = t.empty((M,), dtype=t.float32, device="cuda")

    def step():
        W.w8a8_rmsnorm_quantize(h_d, g_d, 1e-5, residual=r_d, xq=q1, s_tok=s1)
        W.w8a8_silu_mul_quantize(gu_d, sm_d, xq=q2, s_tok=s2)

    def inputs(replay):
        return (act(M, K, "prod_h", replay), act(M, K, "prod_r", replay),
                act(M, 2 * I, "prod_gu", replay))

    h0, r0, gu0 = inputs(0)
    h_d.copy_(dev_bf16(h0)); r_d.copy_(dev_bf16(r0)); gu_d.copy_(dev_bf16(gu0))
    g = capture(step)
    for replay in range(3):
        h, r, gu = inputs(replay)
        h_d.copy_(dev_bf16(h)); r_d.copy_(dev_bf16(r)); gu_d.copy_(dev_bf16(gu))
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        got = [host(v).copy() for v in (q1, s1, h_d, q2, s2)]
        h_d.copy_(dev_bf16(h))                      # the same inputs, eagerly
        t.cuda.synchronize()
        step()
        t.cuda.synchronize()
        want = [host(v) for v in (q1, s1, h_d, q2, s2)]
        for a, b in zip(got, want):
            np.testing.assert_array_equal(a.view(np.uint8), b.view(np.uint8), err_msg=f"replay {replay}")
        if replay == 0:
            q_ref, s_ref, h_ref = O.rmsnorm_quantize(h, r, gamma, 1e-5)
            np.testing.assert_array_equal(got[0], q_ref)
            np.testing.assert_array_equal(got[1].view(np.uint32), s_ref.view(np.uint32))
            np.testing.assert_array_equal(got[2], h_ref)
            q2_ref, s2_ref = O.silu_mul_quantize(gu, sm)
            np.testing.assert_array_equal(got[3], q2_ref)
            np.testing.assert_array_equal(got[4].view(np.uint32), s2_ref.view(np.uint32))


def capture(fn):
    t = torch()
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        fn()
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        fn()
    t.cuda.synchronize()
    return g
