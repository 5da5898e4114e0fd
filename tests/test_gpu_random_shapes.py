"""Seeded random shapes across every GEMM route and configuration the
dispatch rules can pick (token counts 1..700, ragged N, K a multiple of 16
with and without 128 | K), int32 accumulators bit-exact against the oracle,
and the bf16 output of the whole linear on a subset."""
import numpy as np
import pytest

import int8_w8a8_quantized_token_amd as W
from int8_w8a8_quantized_token_amd import workloads as WL
from oracle import w8a8_oracle as O
from gpu_util import check_bf16, dev, dev_bf16, host, torch

pytestmark = pytest.mark.gpu


def _shapes(n=32):
    r = WL.rng("random_shapes")
    out = []
    for i in range(n):
        M = int(r.integers(1, 65)) if i % 4 else int(r.integers(65, 701))
        N = int(r.integers(1, 9001))
        K = 128 * int(r.integers(1, 33)) if i % 2 else 16 * int(r.integers(1, 257))
        out.append((M, N, K))
    return out


SHAPES = _shapes()


@pytest.mark.parametrize("M,N,K", SHAPES, ids=[f"M{m}_N{n}_K{k}" for m, n, k in SHAPES])
def test_gemm_i32_random_shape(M, N, K):
    a = WL.rng("rs_a", M, N, K).integers(-127, 128, size=(M, K), dtype=np.int64).astype(np.int8)
    b = WL.rng("rs_b", M, N, K).integers(-127, 128, size=(N, K), dtype=np.int64).astype(np.int8)
    acc = W.w8a8_gemm_i32(dev(a), dev(b))
    torch().cuda.synchronize()
    np.testing.assert_array_equal(host(acc), O.gemm_i32(a, b))


@pytest.mark.parametrize("M,N,K", SHAPES[::4], ids=[f"M{m}_N{n}_K{k}" for m, n, k in SHAPES[::4]])
def test_linear_random_shape(M, N, K):
    outl = WL.outlier_channels(K, 0.01, "rs", M, N, K)
    x = WL.activations(M, K, "rs", M, N, K, outliers=outl, mult=20.0)
    w = WL.weights(N, K, 0.02, "rs", M, N, K)
    s = O.smoothing_factors(O.act_channel_absmax(x), O.weight_channel_absmax(w))
    wq, sw = O.prepare_weight(w, s)
    y = W.w8a8_linear(dev_bf16(x), dev(s), dev(wq), dev(sw))
    torch().cuda.synchronize()
    ref = O.linear(x, s, wq, sw)
    check_bf16(host(y), ref["y64"], ref["y"])
