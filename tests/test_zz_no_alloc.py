"""w8a8_linear_noalloc (the linear with the library's fixed workspace) gives
the same bits as w8a8_linear with a caller workspace, on consecutive calls
through the one array, the second with a smaller input, and on the fused
one-launch path; oversized problems are refused before anything is
enqueued."""
import numpy as np
import pytest

import int8_w8a8_quantized_token_amd as W
from int8_w8a8_quantized_token_amd import binding as B
from int8_w8a8_quantized_token_amd import workloads as WL
from gpu_util import dev, dev_bf16, host, torch

pytestmark = pytest.mark.gpu

F32 = np.float32


def _prep(N, K, tag):
    w = WL.weights(N, K, 0.02, "noalloc", tag)
    x_cal = WL.activations(64, K, "noalloc", tag, "cal")
    wd = dev_bf16(w)
    s = W.w8a8_smoothing_factors(W.w8a8_channel_absmax(dev_bf16(x_cal)), W.w8a8_channel_absmax(wd))
    wq, sw = W.w8a8_quantize_weight(wd, s)
    return s, wq, sw


@pytest.mark.parametrize("N,K,Ms", [(4096, 4096, (64, 16)), (6144, 4096, (1536, 1)),
                                    (4096, 14336, (64, 4)), (512, 1024 + 16, (300, 7))])
def test_noalloc_linear_matches_linear(N, K, Ms):
    print(f"\n[noalloc] N={N} K={K} M={Ms}", flush=True)
    s, wq, sw = _prep(N, K, f"{N}x{K}")
    for M in Ms:                                 # the second call is smaller
        x = dev_bf16(WL.activations(M, K, "noalloc", N, K, M))
        y_ref = W.w8a8_linear(x, s, wq, sw)
        y = torch().full((M, N), -1, dtype=torch().int16, device="cuda").view(torch().bfloat16)
        B.w8a8_linear_noalloc(x, s, wq, sw, y=y)
        torch().cuda.synchronize()
        np.testing.assert_array_equal(host(y), host(y_ref))


def test_noalloc_refuses_oversized_problems():
    K = 4096
    M = B.NOALLOC_MAX_BYTES // K                 # codes alone fill the array; scales do not fit
    assert W.w8a8_linear_workspace_bytes(M, K) > B.NOALLOC_MAX_BYTES
    s, wq, sw = _prep(256, K, "big")
    x = torch().zeros((M, K), dtype=torch().bfloat16, device="cuda")
    y = torch().empty((M, 256), dtype=torch().bfloat16, device="cuda")
    with pytest.raises(W.W8A8Error, match="WORKSPACE"):
        B.w8a8_linear_noalloc(x, s, wq, sw, y=y)
    # the largest M that fits still runs
    M2 = M - 1
    while W.w8a8_linear_workspace_bytes(M2, K) > B.NOALLOC_MAX_BYTES:
        M2 -= 1
    x2 = dev_bf16(WL.activations(M2, K, "noalloc", "edge"))
    y2 = B.w8a8_linear_noalloc(x2, s, wq, sw)
    y_ref = W.w8a8_linear(x2, s, wq, sw)
    torch().cuda.synchronize()
    np.testing.assert_array_equal(host(y2), host(y_ref))


@pytest.mark.parametrize("M,N,K", [(16, 4096, 4096), (64, 1024, 14336)])
def test_noalloc_linear_under_graph_capture(M, N, K):
    # the callers it is for: a captured graph replayed with new inputs
    # written between replays; every replay equals w8a8_linear
    t = torch()
    s, wq, sw = _prep(N, K, f"graph{N}x{K}")
    x = dev_bf16(WL.activations(M, K, "noalloc", "graph", 0))
    y = t.empty((M, N), dtype=t.bfloat16, device="cuda")
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        B.w8a8_linear_noalloc(x, s, wq, sw, y=y)          # eager call first
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        B.w8a8_linear_noalloc(x, s, wq, sw, y=y)
    t.cuda.synchronize()
    for replay in range(3):
        x.copy_(dev_bf16(WL.activations(M, K, "noalloc", "graph", replay + 1)))
        y.fill_(7.0)
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        got = host(y).copy()
        want = host(W.w8a8_linear(x, s, wq, sw))
        t.cuda.synchronize()
        np.testing.assert_array_equal(got, want, err_msg=f"replay {replay}")
