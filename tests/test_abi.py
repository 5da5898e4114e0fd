"""C-ABI checks that need no GPU: the library loads, exports every function
include/w8a8.h declares, and rejects bad arguments on the host before any
HIP call. Every call below with fake pointers either fails validation or is
an empty (M == 0 / N == 0) no-op, so nothing is ever launched, even on a
machine with a GPU."""
import ctypes
import re
import subprocess

import pytest

import int8_w8a8_quantized_token_amd as W
from int8_w8a8_quantized_token_amd import binding as B

OK, INVALID, MISALIGNED, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3, 4
A = 0x10000          # a fake, 256-byte aligned "device" address
MIS = A + 8          # 8-byte aligned only


@pytest.fixture(scope="module")
def lib():
    return W.lib()


def test_exports_every_header_function(lib):
    names = W.header_functions()
    assert len(names) == 25
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported


def test_version_and_status_strings(lib):
    assert W.w8a8_abi_version() == 1
    for s in range(6):
        assert isinstance(W.w8a8_status_string(s), str) and W.w8a8_status_string(s)
    assert W.w8a8_status_string(99) == "unknown status"


def test_workspace_bytes(lib):
    def al(v):
        return (v + 255) // 256 * 256
    for M, K in [(1, 16), (16, 4096), (3000, 14336), (7, 48)]:
        assert W.w8a8_linear_workspace_bytes(M, K) == al(M * K) + al(4 * M)
    assert W.w8a8_linear_workspace_bytes(0, 4096) == 0
    assert W.w8a8_linear_workspace_bytes(16, 0) == 0


def q(lib, x=A, ldx=4096, smooth=None, M=16, K=4096, xq=A, ldq=4096, s=A):
    return lib.w8a8_quantize_act(x, ldx, smooth, M, K, xq, ldq, s, None)


def test_quantize_act_validation(lib):
    assert q(lib, x=None) == INVALID
    assert q(lib, M=-1) == INVALID
    assert q(lib, K=0) == INVALID
    assert q(lib, K=24, ldx=24, ldq=24) == UNSUPPORTED
    assert q(lib, K=131072 + 16, ldx=131088, ldq=131088) == UNSUPPORTED
    assert q(lib, M=0, x=None, xq=None, s=None) == OK            # empty call, nothing launched
    assert q(lib, x=MIS) == MISALIGNED
    assert q(lib, ldx=4100) == MISALIGNED                         # 8200-byte rows
    assert q(lib, ldx=4000) == INVALID                            # ld < K
    assert q(lib, ldq=4104) == MISALIGNED
    assert q(lib, s=None) == INVALID
    assert q(lib, smooth=A + 2) == MISALIGNED


def g(lib, xq=A, ldq=4096, st=A, wq=A, ldw=4096, sc=A, M=16, N=4096, K=4096, y=A, ldy=4096):
    return lib.w8a8_gemm(xq, ldq, st, wq, ldw, sc, M, N, K, y, ldy, None)


def test_gemm_validation(lib):
    assert g(lib, N=0, xq=None, wq=None, y=None) == OK
    assert g(lib, M=0, xq=None, wq=None, y=None) == OK
    assert g(lib, N=-5) == INVALID
    assert g(lib, y=None) == INVALID
    assert g(lib, wq=None) == INVALID
    assert g(lib, sc=None) == INVALID
    assert g(lib, y=A + 1) == MISALIGNED                         # bf16 needs 2-byte alignment
    assert g(lib, wq=MIS) == MISALIGNED
    assert g(lib, K=40, ldq=40, ldw=40) == UNSUPPORTED
    assert g(lib, ldw=4000) == INVALID


def test_gemm_i32_validation(lib):
    f = lib.w8a8_gemm_i32
    assert f(A, 64, A, 64, 4, 8, 64, None, 8, None) == INVALID
    assert f(A, 64, A, 64, 4, 8, 64, A, 6, None) == INVALID     # ldc < N
    assert f(A, 64, A, 64, 4, 10, 64, A + 2, 10, None) == MISALIGNED  # int32 needs 4 bytes
    assert f(A, 64, A, 64, 0, 10, 64, None, 10, None) == OK


def lin(lib, ws=A, wsb=None, M=16, N=4096, K=4096, x=A):
    if wsb is None:
        wsb = W.w8a8_linear_workspace_bytes(M, K)
    return lib.w8a8_linear(x, K, None, A, K, A, M, N, K, A, N, ws, wsb, None)


def test_linear_validation(lib):
    assert lin(lib, ws=None) == WORKSPACE
    assert lin(lib, wsb=W.w8a8_linear_workspace_bytes(16, 4096) - 1) == WORKSPACE
    assert lin(lib, ws=A + 16) == MISALIGNED
    assert lin(lib, x=None) == INVALID
    assert lin(lib, M=0, ws=None, x=None) == OK
    assert lin(lib, K=4104) == UNSUPPORTED


def test_linear_noalloc_validation(lib):
    f = lib.w8a8_linear_noalloc
    def call(M=16, N=4096, K=4096, x=A, y=A):
        return f(x, K, None, A, K, A, M, N, K, y, N, None)
    assert call(M=2048) == WORKSPACE             # workspace past the fixed 8 MiB
    assert call(M=1 << 20, K=16) == WORKSPACE
    assert call(x=None) == INVALID
    assert call(y=None) == INVALID
    assert call(K=4104) == UNSUPPORTED
    assert call(x=MIS) == MISALIGNED
    assert call(M=0, x=None, y=None) == OK        # empty call, nothing launched
    assert W.w8a8_linear_workspace_bytes(2046, 4096) <= B.NOALLOC_MAX_BYTES
    assert W.w8a8_linear_workspace_bytes(2047, 4096) > B.NOALLOC_MAX_BYTES


def test_prep_validation(lib):
    ca = lib.w8a8_channel_absmax
    assert ca(A, 4096, 16, 4096, None, None) == INVALID
    assert ca(A, 12, 16, 12, A, None) == UNSUPPORTED           # K % 8
    assert ca(A, 4096, 0, 4096, None, None) == OK
    assert ca(MIS, 4096, 16, 4096, A, None) == MISALIGNED
    sf = lib.w8a8_smoothing_factors
    assert sf(A, A, -1, A, None) == INVALID
    assert sf(None, None, 0, None, None) == OK
    assert sf(A, None, 16, A, None) == INVALID
    qw = lib.w8a8_quantize_weight
    assert qw(A, 4096, None, 16, 4096, A, 4096, None, None) == INVALID
    assert qw(A, 4096, None, 16, 4104, A, 4104, A, None) == UNSUPPORTED
    assert qw(A, 4096, None, 0, 4096, None, 4096, None, None) == OK


def test_static_scale_validation(lib):
    qs = lib.w8a8_quantize_act_static
    assert qs(A, 4096, None, None, 16, 4096, A, 4096, A, None) == INVALID       # no scale
    assert qs(A, 4096, None, A + 2, 16, 4096, A, 4096, A, None) == MISALIGNED
    assert qs(A, 4096, None, A, 16, 24, A, 24, A, None) == UNSUPPORTED         # K % 16
    assert qs(MIS, 4096, None, A, 16, 4096, A, 4096, A, None) == MISALIGNED
    assert qs(None, 4096, None, None, 0, 4096, None, 4096, None, None) == OK   # empty
    ls = lib.w8a8_linear_static
    assert ls(A, 4096, None, A, A, 4096, A, 16, 4096, 4096, A, 4096, None, 0, None) == WORKSPACE
    assert ls(A, 4096, None, None, A, 4096, A, 16, 4096, 4096, A, 4096, A, 1 << 30, None) == INVALID
    assert ls(None, 4096, None, None, None, 4096, None, 0, 4096, 4096, None, 4096, None, 0,
              None) == OK
    cm = lib.w8a8_calibrate_minmax
    assert cm(A, None, 0, A, A, None) == INVALID
    assert cm(None, None, 16, A, A, None) == INVALID
    assert cm(A, None, 16, A, A + 1, None) == MISALIGNED
    ah = lib.w8a8_activation_histogram
    assert ah(A, 4096, None, 16, 4096, A, 127, A, None) == UNSUPPORTED          # bins
    assert ah(A, 4096, None, 16, 4096, A, 8193, A, None) == UNSUPPORTED
    assert ah(A, 12, None, 16, 12, A, 2048, A, None) == UNSUPPORTED             # K % 8
    assert ah(A, 4096, None, 16, 4096, None, 2048, A, None) == INVALID          # no amax
    assert ah(A, 4096, None, 16, 4096, A, 2048, None, None) == INVALID          # no hist
    assert ah(None, 4096, None, 0, 4096, None, 2048, None, None) == OK          # no rows
    ce = lib.w8a8_calibrate_entropy
    assert ce(A, 100, A, A, None, None) == UNSUPPORTED
    assert ce(None, 2048, A, A, None, None) == INVALID
    assert ce(A, 2048, A, None, None, None) == INVALID
    assert ce(A, 2048, A, A, A + 4, None) == MISALIGNED                         # kl alignment


def test_producer_validation(lib):
    rq = lib.w8a8_rmsnorm_quantize
    assert rq(A, 4096, None, 4096, A, 1e-5, 16, 4096, A, 4096, None, None) == INVALID   # s_tok
    assert rq(A, 4096, None, 4096, A, -1.0, 16, 4096, A, 4096, A, None) == INVALID      # eps
    assert rq(A, 4096, None, 4096, A, float("nan"), 16, 4096, A, 4096, A, None) == INVALID
    assert rq(A, 4096, None, 4096, A, 1e-5, 16, 4104, A, 4104, A, None) == UNSUPPORTED
    assert rq(A, 65552, None, 65552, A, 1e-5, 1, 65552, A, 65552, A, None) == UNSUPPORTED
    assert rq(A, 4096, MIS, 4096, A, 1e-5, 16, 4096, A, 4096, A, None) == MISALIGNED
    assert rq(None, 4096, None, 4096, None, 1e-5, 0, 4096, None, 4096, None, None) == OK
    sq = lib.w8a8_silu_mul_quantize
    assert sq(A, 8192, None, 16, 4096, A, 4096, None, None) == INVALID
    assert sq(A, 8000, None, 16, 4096, A, 4096, A, None) == INVALID                 # ld < 2I
    assert sq(A, 8192, None, 16, 4104, A, 4104, A, None) == UNSUPPORTED
    assert sq(None, 8192, None, 0, 4096, None, 4096, None, None) == OK
    fg = lib.w8a8_fold_gamma
    assert fg(None, None, 16, A, None) == INVALID
    assert fg(None, None, 0, None, None) == OK
    ra = lib.w8a8_residual_add
    assert ra(A, 4096, None, 4096, 16, 4096, None) == INVALID
    assert ra(A, 12, A, 12, 16, 12, None) == UNSUPPORTED
    assert ra(None, 4096, None, 4096, 0, 4096, None) == OK


def test_gptq_validation(lib):
    gh = lib.w8a8_gptq_hessian
    assert gh(A, 4096, None, 16, 4096, None, None) == INVALID                 # no H
    assert gh(A, 4096, None, 16, 4096, A + 4, None) == MISALIGNED
    assert gh(A, 40000, None, 16, 40000, A, None) == UNSUPPORTED            # K > 32768
    assert gh(None, 4096, None, 0, 4096, None, None) == OK
    assert lib.w8a8_gptq_factor_workspace_bytes(0) == 0
    assert lib.w8a8_gptq_factor_workspace_bytes(64) == (64 * 64 + 1) * 8 + (256 - (64 * 64 + 1) * 8 % 256)
    gf = lib.w8a8_gptq_factor
    assert gf(A, 64, 0.01, A, None, 0, None) == WORKSPACE
    assert gf(A, 64, -1.0, A, A, 1 << 20, None) == INVALID
    assert gf(A, 0, 0.01, A, A, 1 << 20, None) == INVALID
    assert gf(A, 64, 0.01, A, A + 16, 1 << 20, None) == MISALIGNED
    gq = lib.w8a8_gptq_quantize
    wsb = lib.w8a8_gptq_quantize_workspace_bytes(16, 64)
    assert wsb == 16 * 64 * 8 + 16 * 64 * 8
    assert gq(A, 64, None, A, 16, 64, A, 64, A, A, wsb - 1, None) == WORKSPACE
    assert gq(A, 64, None, None, 16, 64, A, 64, A, A, wsb, None) == INVALID
    assert gq(A, 64, None, A, 16, 72, A, 72, A, A, 1 << 20, None) == UNSUPPORTED  # K % 16
    assert gq(None, 64, None, None, 0, 64, None, 64, None, None, 0, None) == OK


def test_python_binding_raises_typed_error(lib):
    torch = pytest.importorskip("torch")
    with pytest.raises((TypeError, ValueError)):
        W.w8a8_quantize_act(torch.zeros((4, 16), dtype=torch.float32))


def test_binding_checks_every_extent(lib):
    # The ABI sees bare pointers, so the binding must refuse buffers that do
    # not match the sizes it passes. These are host tensors: the extent checks
    # come before the device check, so each call stops at the size it names.
    torch = pytest.importorskip("torch")
    bf, i8, f32 = torch.bfloat16, torch.int8, torch.float32
    e = lambda *s, dt=f32: torch.empty(s, dtype=dt)      # noqa: E731
    M, N, K = 4, 32, 64
    x, wq, xq = e(M, K, dt=bf), e(N, K, dt=i8), e(M, K, dt=i8)
    cases = [
        (lambda: W.w8a8_quantize_act(x, smooth=e(K - 1)), "smooth"),
        (lambda: W.w8a8_quantize_act(x, xq=e(M - 1, K, dt=i8)), "xq"),
        (lambda: W.w8a8_quantize_act(x, s_tok=e(M - 1)), "s_tok"),
        (lambda: W.w8a8_gemm(xq, e(M - 1), wq, e(N)), "s_tok"),
        (lambda: W.w8a8_gemm(xq, e(M), wq, e(N - 1)), "s_chan"),
        (lambda: W.w8a8_gemm(xq, e(M), e(N, K + 16, dt=i8), e(N)), "disagree on K"),
        (lambda: W.w8a8_gemm(xq, e(M), wq, e(N), y=e(M - 1, N, dt=bf)), "y"),
        (lambda: W.w8a8_gemm_i32(xq, wq, acc=e(M, N - 1, dt=torch.int32)), "acc"),
        (lambda: W.w8a8_linear(x, e(K - 1), wq, e(N)), "smooth"),
        (lambda: W.w8a8_linear(x, None, wq, e(N - 1)), "s_chan"),
        (lambda: W.w8a8_linear(x, None, e(N, 2 * K, dt=i8), e(N)), "disagree on K"),
        (lambda: W.w8a8_linear(x, None, wq, e(N), y=e(M - 1, N, dt=bf)), "y"),
        (lambda: W.w8a8_channel_absmax(x, absmax=e(K - 1)), "absmax"),
        (lambda: W.w8a8_smoothing_factors(e(K), e(K - 1)), "w_absmax"),
        (lambda: W.w8a8_quantize_weight(e(N, K, dt=bf), e(K - 1)), "smooth"),
        (lambda: W.w8a8_quantize_weight(e(N, K, dt=bf), wq=e(N, K - 16, dt=i8)), "wq"),
        (lambda: W.w8a8_quantize_weight(e(N, K, dt=bf), s_chan=e(N - 1)), "s_chan"),
        (lambda: W.w8a8_quantize_act_static(x, None, e(0)), "scale"),
        (lambda: W.w8a8_linear_static(x, None, e(1), wq, e(N - 1)), "s_chan"),
        (lambda: W.w8a8_calibrate_minmax(e(K), e(K - 1)), "smooth"),
        (lambda: W.w8a8_activation_histogram(x, None, e(1), hist=e(2047, dt=torch.int32)), "hist"),
        (lambda: W.w8a8_calibrate_entropy(e(2048, dt=torch.int32), e(1),
                                          kl=e(2048, dt=torch.float64)), "kl"),
        (lambda: W.w8a8_rmsnorm_quantize(x, e(K - 1)), "gamma"),
        (lambda: W.w8a8_rmsnorm_quantize(x, e(K), residual=e(M, K - 16, dt=bf)), "residual"),
        (lambda: W.w8a8_silu_mul_quantize(e(M, 2 * K + 1, dt=bf)), "gate | up"),
        (lambda: W.w8a8_silu_mul_quantize(e(M, 2 * K, dt=bf), e(K - 1)), "smooth"),
        (lambda: W.w8a8_silu_mul_quantize(e(M, 2 * K, dt=bf), xq=e(M, 2 * K, dt=i8)), "xq"),
        (lambda: W.w8a8_fold_gamma(e(K), e(K - 1)), "smooth"),
        (lambda: W.w8a8_residual_add(x, e(M, K - 16, dt=bf)), "r"),
        (lambda: W.w8a8_gptq_hessian(x, H=e(K, K - 1, dt=torch.float64)), "H"),
        (lambda: W.w8a8_gptq_factor(e(K, K - 1, dt=torch.float64)), "H"),
        (lambda: W.w8a8_gptq_quantize(e(N, K, dt=bf), None, e(K - 1, K, dt=torch.float64)), "U"),
    ]
    for call, what in cases:
        pattern = f"^{what}: " if what.isidentifier() else re.escape(what)
        with pytest.raises(ValueError, match=pattern):
            call()
    # with every extent right, a host tensor stops at the device check
    with pytest.raises(ValueError, match="device tensor"):
        W.w8a8_gemm(xq, e(M), wq, e(N), y=e(M, N, dt=bf))
