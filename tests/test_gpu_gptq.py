"""GPU parity of the GPTQ entry points against the oracle.

* w8a8_gptq_hessian: binary64 sums of exact products; against the oracle's
  binary64 matmul within n * 2^-52 of the sum of magnitudes.
* w8a8_gptq_factor: a different factorization route than the oracle's
  (reversal + Cholesky + triangular inverse against inverse + Cholesky);
  U within 1e-9 of the oracle's, relative to max |U|, and U^T U (H + lambda I)
  within 1e-9 of the identity.
* w8a8_gptq_quantize: given the same U, every weight receives the same
  updates in the same order and rounding, so codes and scales are bit-exact.
* End to end on the GPU: codes agree with the oracle's end-to-end codes
  except where the factor's last-bit differences move a weight across a
  rounding boundary (bounded below), and the output error on the calibration
  set is below round-to-nearest's.
"""
import numpy as np
import pytest

import int8_w8a8_quantized_token_amd as W
from int8_w8a8_quantized_token_amd import workloads as WL
from oracle import w8a8_oracle as O
from gpu_util import dev, dev_bf16, host, torch

pytestmark = pytest.mark.gpu

F32 = np.float32


def calib(n, K, tag, correlated=True):
    """Calibration activations whose channels correlate (as real ones do)."""
    r = WL.rng("gptq-x", tag, n, K)
    z = r.standard_normal((n, K)).astype(np.float64)
    if correlated:
        mix = r.standard_normal((K, K)) * (0.3 / np.sqrt(K / 128)) + np.eye(K)
        z = z @ mix
    return O.round_to_bf16(z.astype(F32))


@pytest.mark.parametrize("n,K,use_smooth", [(300, 512, False), (257, 528, True), (64, 1024, True)])
def test_hessian(n, K, use_smooth):
    x = calib(n, K, "h")
    smooth = np.exp(WL.rng("gptq-s", K).uniform(-1, 1, K)).astype(F32) if use_smooth else None
    H = W.w8a8_gptq_hessian(dev_bf16(x), dev(smooth) if use_smooth else None)
    W.w8a8_gptq_hessian(dev_bf16(x), dev(smooth) if use_smooth else None, H=H)   # accumulates
    torch().cuda.synchronize()
    want = 2 * O.gptq_hessian(x, smooth)
    xs = np.abs(O.smooth_activations(O.bf16_to_f32(x), smooth).astype(np.float64))
    bound = 4 * (2 * n + 4) * 2.0 ** -52 * (xs.T @ xs)            # sum of |terms|
    got = host(H)
    assert np.all(np.abs(got - want) <= bound + 1e-300)


@pytest.mark.parametrize("K", [128, 512, 528])
def test_factor(K):
    x = calib(400, K, "f")
    H = O.gptq_hessian(x)
    H[7, :] = 0.0
    H[:, 7] = 0.0                                   # a channel never excited
    U = W.w8a8_gptq_factor(dev(H))
    torch().cuda.synchronize()
    got = host(U)
    want = O.gptq_factor(H)
    assert np.allclose(np.tril(got, -1), 0) and np.all(np.diag(got) > 0)
    assert np.max(np.abs(got - want)) <= 1e-9 * np.max(np.abs(want))
    d = np.diag(H).copy()
    d[d == 0] = 1.0
    Hd = H.copy()
    np.fill_diagonal(Hd, d + 0.01 * np.mean(d))
    np.testing.assert_allclose(got.T @ got @ Hd, np.eye(K), atol=1e-9)


@pytest.mark.parametrize("N,K,use_smooth", [(200, 512, False), (65, 528, True), (130, 1040, True)])
def test_quantize_bit_exact_given_factor(N, K, use_smooth):
    x = calib(300, K, "q")
    w = WL.weights(N, K, 0.02, "gptq", "w", N, K)
    smooth = np.exp(WL.rng("gptq-s", K).uniform(-1, 1, K)).astype(F32) if use_smooth else None
    U = O.gptq_factor(O.gptq_hessian(x, smooth))
    q_ref, s_ref = O.gptq_quantize(w, smooth, U)
    wq, sc = W.w8a8_gptq_quantize(dev_bf16(w), dev(smooth) if use_smooth else None, dev(U))
    torch().cuda.synchronize()
    np.testing.assert_array_equal(host(sc).view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(host(wq), q_ref)
    # the scales are the round-to-nearest ones; the codes are not
    q_rtn, s_rtn = O.prepare_weight(w, smooth)
    assert np.array_equal(s_ref, s_rtn) and not np.array_equal(q_ref, q_rtn)


def test_end_to_end_on_gpu():
    N, K = 256, 512
    x = calib(512, K, "e2e")
    w = WL.weights(N, K, 0.02, "gptq", "e2e")
    d_x = dev_bf16(x)
    H = W.w8a8_gptq_hessian(d_x)
    U = W.w8a8_gptq_factor(H)
    wq, sc = W.w8a8_gptq_quantize(dev_bf16(w), None, U)
    torch().cuda.synchronize()
    q_ref, s_ref = O.gptq_quantize(w, None, O.gptq_factor(O.gptq_hessian(x)))
    got = host(wq)
    np.testing.assert_array_equal(host(sc), s_ref)
    assert np.mean(got != q_ref) <= 1e-3          # only near-boundary flips may differ
    X = O.bf16_to_f32(x).astype(np.float64)
    Wf = O.bf16_to_f32(w).astype(np.float64)
    q_rtn, _ = O.prepare_weight(w, None)
    def out_err(q):
        return np.linalg.norm((Wf - q * s_ref[:, None].astype(np.float64)) @ X.T)
    assert out_err(got) < 0.8 * out_err(q_rtn)


def test_llama_shaped_projection():
    # o_proj-sized weight (4096 x 4096) with 512 calibration tokens: the GPU
    # path runs at this size and lowers the calibration output error
    N = K = 4096
    t = torch()
    x = calib(512, K, "llama", correlated=False)
    w = WL.weights(N, K, 0.02, "gptq", "llama")
    d_x, d_w = dev_bf16(x), dev_bf16(w)
    U = W.w8a8_gptq_factor(W.w8a8_gptq_hessian(d_x))
    wq, sc = W.w8a8_gptq_quantize(d_w, None, U)
    wq_rtn, sc_rtn = W.w8a8_quantize_weight(d_w)
    t.cuda.synchronize()
    assert t.equal(sc, sc_rtn)
    assert bool(t.isfinite(U).all())
    X = d_x.to(t.float64)
    Wf = d_w.to(t.float64)
    def out_err(q):
        return float(t.linalg.norm((Wf - q.to(t.float64) * sc.to(t.float64)[:, None]) @ X.T))
    assert out_err(wq) < out_err(wq_rtn)
