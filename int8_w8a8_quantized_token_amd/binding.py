"""ctypes binding of libw8a8.so: one Python function per C entry point, same
names, argument marshalling only.

torch is used for device memory (outputs and workspaces are allocated with
torch.empty when the caller does not pass them) and for the current HIP
stream. Every step of the layer runs in the library's kernels. If the
library is missing the first call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libw8a8.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "w8a8.h")

STATUS = {0: "W8A8_SUCCESS", 1: "W8A8_ERROR_INVALID_VALUE", 2: "W8A8_ERROR_MISALIGNED",
          3: "W8A8_ERROR_UNSUPPORTED", 4: "W8A8_ERROR_WORKSPACE", 5: "W8A8_ERROR_HIP"}


class W8A8Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} "
                         f"({lib().w8a8_status_string(status).decode()})")


_p, _i64, _sz, _i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int

_SIGNATURES = {
    "w8a8_status_string": (ctypes.c_char_p, [_i]),
    "w8a8_abi_version": (_i, []),
    "w8a8_quantize_act": (_i, [_p, _i64, _p, _i64, _i64, _p, _i64, _p, _p]),
    "w8a8_gemm": (_i, [_p, _i64, _p, _p, _i64, _p, _i64, _i64, _i64, _p, _i64, _p]),
    "w8a8_gemm_i32": (_i, [_p, _i64, _p, _i64, _i64, _i64, _i64, _p, _i64, _p]),
    "w8a8_linear_workspace_bytes": (_sz, [_i64, _i64]),
    "w8a8_linear": (_i, [_p, _i64, _p, _p, _i64, _p, _i64, _i64, _i64, _p, _i64, _p, _sz, _p]),
    "w8a8_linear_noalloc": (_i, [_p, _i64, _p, _p, _i64, _p, _i64, _i64, _i64, _p, _i64, _p]),
    "w8a8_channel_absmax": (_i, [_p, _i64, _i64, _i64, _p, _p]),
    "w8a8_smoothing_factors": (_i, [_p, _p, _i64, _p, _p]),
    "w8a8_quantize_weight": (_i, [_p, _i64, _p, _i64, _i64, _p, _i64, _p, _p]),
    "w8a8_quantize_act_static": (_i, [_p, _i64, _p, _p, _i64, _i64, _p, _i64, _p, _p]),
    "w8a8_linear_static": (_i, [_p, _i64, _p, _p, _p, _i64, _p, _i64, _i64, _i64, _p, _i64,
                                _p, _sz, _p]),
    "w8a8_calibrate_minmax": (_i, [_p, _p, _i64, _p, _p, _p]),
    "w8a8_activation_histogram": (_i, [_p, _i64, _p, _i64, _i64, _p, _i64, _p, _p]),
    "w8a8_calibrate_entropy": (_i, [_p, _i64, _p, _p, _p, _p]),
    "w8a8_rmsnorm_quantize": (_i, [_p, _i64, _p, _i64, _p, ctypes.c_float, _i64, _i64, _p, _i64,
                                   _p, _p]),
    "w8a8_silu_mul_quantize": (_i, [_p, _i64, _p, _i64, _i64, _p, _i64, _p, _p]),
    "w8a8_fold_gamma": (_i, [_p, _p, _i64, _p, _p]),
    "w8a8_residual_add": (_i, [_p, _i64, _p, _i64, _i64, _i64, _p]),
    "w8a8_gptq_hessian": (_i, [_p, _i64, _p, _i64, _i64, _p, _p]),
    "w8a8_gptq_factor_workspace_bytes": (_sz, [_i64]),
    "w8a8_gptq_factor": (_i, [_p, _i64, ctypes.c_double, _p, _p, _sz, _p]),
    "w8a8_gptq_quantize_workspace_bytes": (_sz, [_i64, _i64]),
    "w8a8_gptq_quantize": (_i, [_p, _i64, _p, _p, _i64, _i64, _p, _i64, _p, _p, _sz, _p]),
}

HIST_BINS = 2048       # W8A8_HIST_BINS
QUANT_LEVELS = 128     # W8A8_QUANT_LEVELS

_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m int8_w8a8_quantized_token_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _LIB = handle
    return _LIB


def header_functions() -> list:
    """Names of the functions include/w8a8.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w8a8_[a-z0-9_]+)\s*\(", text)))


# ---------------------------------------------------------------------------
# torch-facing marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _mat(t, dtypes, name):
    torch = _torch()
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name}: need a 2-D tensor with a contiguous last dim")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor")
    return t.data_ptr(), (t.stride(0) if t.shape[0] > 1 else max(t.shape[1], t.stride(0)))


def _vec(t, name, dtype=None):
    if t is None:
        return None
    torch = _torch()
    dtype = dtype or torch.float32
    if t.dtype != dtype or t.dim() != 1 or (t.numel() > 1 and t.stride(0) != 1):
        raise TypeError(f"{name}: need a contiguous 1-D {dtype} tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor")
    return t.data_ptr()


# The C ABI takes bare pointers and cannot see how long a buffer is, so the
# binding checks every tensor's extent against the sizes it passes before
# anything reaches the library: a short output would be written past its
# end, a short input read past it.

def _shape(t, name, rows, cols):
    if t is None:
        return
    if t.dim() != 2 or tuple(t.shape) != (rows, cols):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected ({rows}, {cols})")


def _dims(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name}: need a 2-D tensor, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _length(t, name, n):
    if t is None:
        return
    if t.dim() != 1 or t.numel() < n:
        raise ValueError(f"{name}: {tuple(t.shape)} holds fewer than the {n} elements needed")


def _one_device(*tensors):
    devs = {t.device for t in tensors if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors on different devices: {sorted(str(d) for d in devs)}")


def _nbytes(t):
    return t.numel() * t.element_size()


def _check(status, where):
    if status != 0:
        raise W8A8Error(status, where)


def _bf16_types():
    torch = _torch()
    return (torch.bfloat16, torch.int16)


def w8a8_status_string(status: int) -> str:
    return lib().w8a8_status_string(status).decode()


def w8a8_abi_version() -> int:
    return lib().w8a8_abi_version()


def w8a8_quantize_act(x, smooth=None, xq=None, s_tok=None, stream=None):
    """x bf16 [M, K] -> (xq int8 [M, K], s_tok fp32 [M])."""
    torch = _torch()
    M, K = _dims(x, "x")
    _length(smooth, "smooth", K)
    _shape(xq, "xq", M, K)
    _length(s_tok, "s_tok", M)
    _one_device(x, smooth, xq, s_tok)
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if s_tok is None:
        s_tok = torch.empty((M,), dtype=torch.float32, device=x.device)
    px, ldx = _mat(x, _bf16_types(), "x")
    pq, ldq = _mat(xq, (torch.int8,), "xq")
    _check(lib().w8a8_quantize_act(px, ldx, _vec(smooth, "smooth"), M, K, pq, ldq,
                                   _vec(s_tok, "s_tok"), _stream(stream)), "w8a8_quantize_act")
    return xq, s_tok


def w8a8_gemm(xq, s_tok, wq, s_chan, y=None, stream=None):
    """(xq [M, K], s_tok [M]) x (wq [N, K], s_chan [N]) -> y bf16 [M, N]."""
    torch = _torch()
    M, K = _dims(xq, "xq")
    N, Kw = _dims(wq, "wq")
    if Kw != K:
        raise ValueError(f"xq and wq disagree on K ({K} vs {Kw})")
    _length(s_tok, "s_tok", M)
    _length(s_chan, "s_chan", N)
    _shape(y, "y", M, N)
    _one_device(xq, s_tok, wq, s_chan, y)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    pq, ldq = _mat(xq, (torch.int8,), "xq")
    pw, ldw = _mat(wq, (torch.int8,), "wq")
    py, ldy = _mat(y, _bf16_types(), "y")
    _check(lib().w8a8_gemm(pq, ldq, _vec(s_tok, "s_tok"), pw, ldw, _vec(s_chan, "s_chan"),
                           M, N, K, py, ldy, _stream(stream)), "w8a8_gemm")
    return y


def w8a8_gemm_i32(xq, wq, acc=None, stream=None):
    """Exact int32 accumulators acc [M, N] = xq @ wq.T."""
    torch = _torch()
    M, K = _dims(xq, "xq")
    N, Kw = _dims(wq, "wq")
    if Kw != K:
        raise ValueError(f"xq and wq disagree on K ({K} vs {Kw})")
    _shape(acc, "acc", M, N)
    _one_device(xq, wq, acc)
    if acc is None:
        acc = torch.empty((M, N), dtype=torch.int32, device=xq.device)
    pq, ldq = _mat(xq, (torch.int8,), "xq")
    pw, ldw = _mat(wq, (torch.int8,), "wq")
    pc, ldc = _mat(acc, (torch.int32,), "acc")
    _check(lib().w8a8_gemm_i32(pq, ldq, pw, ldw, M, N, K, pc, ldc, _stream(stream)),
           "w8a8_gemm_i32")
    return acc


def w8a8_linear_workspace_bytes(M: int, K: int) -> int:
    return lib().w8a8_linear_workspace_bytes(M, K)


def w8a8_linear(x, smooth, wq, s_chan, y=None, workspace=None, stream=None):
    """x bf16 [M, K] -> y bf16 [M, N] (quantize + GEMM + epilogue)."""
    torch = _torch()
    M, K = _dims(x, "x")
    N, Kw = _dims(wq, "wq")
    if Kw != K:
        raise ValueError(f"x and wq disagree on K ({K} vs {Kw})")
    _length(smooth, "smooth", K)
    _length(s_chan, "s_chan", N)
    _shape(y, "y", M, N)
    _one_device(x, smooth, wq, s_chan, y, workspace)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    nbytes = w8a8_linear_workspace_bytes(M, K)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=x.device)
    px, ldx = _mat(x, _bf16_types(), "x")
    pw, ldw = _mat(wq, (torch.int8,), "wq")
    py, ldy = _mat(y, _bf16_types(), "y")
    _check(lib().w8a8_linear(px, ldx, _vec(smooth, "smooth"), pw, ldw, _vec(s_chan, "s_chan"),
                             M, N, K, py, ldy, workspace.data_ptr(), _nbytes(workspace),
                             _stream(stream)),
           "w8a8_linear")
    return y


NOALLOC_MAX_BYTES = 8 << 20   # W8A8_NOALLOC_MAX_BYTES


def w8a8_linear_noalloc(x, smooth, wq, s_chan, y=None, stream=None):
    """w8a8_linear with the library's fixed workspace (no workspace argument;
    the library call allocates nothing). Pass y to allocate nothing here
    either."""
    torch = _torch()
    M, K = _dims(x, "x")
    N, Kw = _dims(wq, "wq")
    if Kw != K:
        raise ValueError(f"x and wq disagree on K ({K} vs {Kw})")
    _length(smooth, "smooth", K)
    _length(s_chan, "s_chan", N)
    _shape(y, "y", M, N)
    _one_device(x, smooth, wq, s_chan, y)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    px, ldx = _mat(x, _bf16_types(), "x")
    pw, ldw = _mat(wq, (torch.int8,), "wq")
    py, ldy = _mat(y, _bf16_types(), "y")
    _check(lib().w8a8_linear_noalloc(px, ldx, _vec(smooth, "smooth"), pw, ldw,
                                     _vec(s_chan, "s_chan"), M, N, K, py, ldy, _stream(stream)),
           "w8a8_linear_noalloc")
    return y


def w8a8_channel_absmax(a, absmax=None, stream=None):
    """absmax [K] = max(absmax, max over rows |a|); zero-initialized if not given."""
    torch = _torch()
    rows, K = _dims(a, "a")
    _length(absmax, "absmax", K)
    _one_device(a, absmax)
    if absmax is None:
        absmax = torch.zeros((K,), dtype=torch.float32, device=a.device)
    pa, lda = _mat(a, _bf16_types(), "a")
    _check(lib().w8a8_channel_absmax(pa, lda, rows, K, _vec(absmax, "absmax"), _stream(stream)),
           "w8a8_channel_absmax")
    return absmax


def w8a8_smoothing_factors(act_absmax, w_absmax, smooth=None, stream=None):
    torch = _torch()
    K = act_absmax.shape[0]
    _length(w_absmax, "w_absmax", K)
    _length(smooth, "smooth", K)
    _one_device(act_absmax, w_absmax, smooth)
    if smooth is None:
        smooth = torch.empty((K,), dtype=torch.float32, device=act_absmax.device)
    _check(lib().w8a8_smoothing_factors(_vec(act_absmax, "act_absmax"), _vec(w_absmax, "w_absmax"),
                                        K, _vec(smooth, "smooth"), _stream(stream)),
           "w8a8_smoothing_factors")
    return smooth


def w8a8_quantize_weight(w, smooth=None, wq=None, s_chan=None, stream=None):
    """w bf16 [N, K] -> (wq int8 [N, K], s_chan fp32 [N])."""
    torch = _torch()
    N, K = _dims(w, "w")
    _length(smooth, "smooth", K)
    _shape(wq, "wq", N, K)
    _length(s_chan, "s_chan", N)
    _one_device(w, smooth, wq, s_chan)
    if wq is None:
        wq = torch.empty((N, K), dtype=torch.int8, device=w.device)
    if s_chan is None:
        s_chan = torch.empty((N,), dtype=torch.float32, device=w.device)
    pw, ldw = _mat(w, _bf16_types(), "w")
    pq, ldq = _mat(wq, (torch.int8,), "wq")
    _check(lib().w8a8_quantize_weight(pw, ldw, _vec(smooth, "smooth"), N, K, pq, ldq,
                                      _vec(s_chan, "s_chan"), _stream(stream)),
           "w8a8_quantize_weight")
    return wq, s_chan


# ---------------------------------------------------------------------------
# static per-tensor activation scale
# ---------------------------------------------------------------------------

def w8a8_quantize_act_static(x, smooth, scale, xq=None, s_tok=None, stream=None):
    """x bf16 [M, K], scale fp32 [1] (device) -> (xq int8 [M, K], s_tok fp32 [M] = scale)."""
    torch = _torch()
    M, K = _dims(x, "x")
    _length(smooth, "smooth", K)
    _length(scale, "scale", 1)
    _shape(xq, "xq", M, K)
    _length(s_tok, "s_tok", M)
    _one_device(x, smooth, scale, xq, s_tok)
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if s_tok is None:
        s_tok = torch.empty((M,), dtype=torch.float32, device=x.device)
    px, ldx = _mat(x, _bf16_types(), "x")
    pq, ldq = _mat(xq, (torch.int8,), "xq")
    _check(lib().w8a8_quantize_act_static(px, ldx, _vec(smooth, "smooth"), _vec(scale, "scale"),
                                          M, K, pq, ldq, _vec(s_tok, "s_tok"), _stream(stream)),
           "w8a8_quantize_act_static")
    return xq, s_tok


def w8a8_linear_static(x, smooth, scale, wq, s_chan, y=None, workspace=None, stream=None):
    """x bf16 [M, K] -> y bf16 [M, N] with the fixed activation scale scale[0]."""
    torch = _torch()
    M, K = _dims(x, "x")
    N, Kw = _dims(wq, "wq")
    if Kw != K:
        raise ValueError(f"x and wq disagree on K ({K} vs {Kw})")
    _length(smooth, "smooth", K)
    _length(scale, "scale", 1)
    _length(s_chan, "s_chan", N)
    _shape(y, "y", M, N)
    _one_device(x, smooth, scale, wq, s_chan, y, workspace)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    nbytes = w8a8_linear_workspace_bytes(M, K)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=x.device)
    px, ldx = _mat(x, _bf16_types(), "x")
    pw, ldw = _mat(wq, (torch.int8,), "wq")
    py, ldy = _mat(y, _bf16_types(), "y")
    _check(lib().w8a8_linear_static(px, ldx, _vec(smooth, "smooth"), _vec(scale, "scale"), pw, ldw,
                                    _vec(s_chan, "s_chan"), M, N, K, py, ldy, workspace.data_ptr(),
                                    _nbytes(workspace), _stream(stream)),
           "w8a8_linear_static")
    return y


def w8a8_calibrate_minmax(act_absmax, smooth=None, amax=None, scale=None, stream=None):
    """Per-channel maxima [K] -> (amax fp32 [1], scale fp32 [1]) on the device."""
    torch = _torch()
    K = act_absmax.shape[0]
    _length(smooth, "smooth", K)
    _length(amax, "amax", 1)
    _length(scale, "scale", 1)
    _one_device(act_absmax, smooth, amax, scale)
    dev = act_absmax.device
    amax = torch.empty((1,), dtype=torch.float32, device=dev) if amax is None else amax
    scale = torch.empty((1,), dtype=torch.float32, device=dev) if scale is None else scale
    _check(lib().w8a8_calibrate_minmax(_vec(act_absmax, "act_absmax"), _vec(smooth, "smooth"), K,
                                       _vec(amax, "amax"), _vec(scale, "scale"), _stream(stream)),
           "w8a8_calibrate_minmax")
    return amax, scale


def w8a8_activation_histogram(x, smooth, amax, bins=HIST_BINS, hist=None, stream=None):
    """Adds the |x'| counts of x bf16 [rows, K] to hist (uint32 [bins], kept in
    an int32 tensor; zero-initialized when not given) and returns it."""
    torch = _torch()
    rows, K = _dims(x, "x")
    _length(smooth, "smooth", K)
    _length(amax, "amax", 1)
    _length(hist, "hist", bins)
    _one_device(x, smooth, amax, hist)
    if hist is None:
        hist = torch.zeros((bins,), dtype=torch.int32, device=x.device)
    px, ldx = _mat(x, _bf16_types(), "x")
    _check(lib().w8a8_activation_histogram(px, ldx, _vec(smooth, "smooth"), rows, K,
                                           _vec(amax, "amax"), bins,
                                           _vec(hist, "hist", torch.int32), _stream(stream)),
           "w8a8_activation_histogram")
    return hist


def w8a8_calibrate_entropy(hist, amax, scale=None, kl=None, want_kl=False, stream=None):
    """hist [bins] (int32 tensor holding uint32 counts), amax [1] -> (scale fp32 [1],
    kl fp64 [bins + 1] or None)."""
    torch = _torch()
    bins = hist.shape[0]
    _length(amax, "amax", 1)
    _length(scale, "scale", 1)
    _length(kl, "kl", bins + 1)
    _one_device(hist, amax, scale, kl)
    dev = hist.device
    scale = torch.empty((1,), dtype=torch.float32, device=dev) if scale is None else scale
    if kl is None and want_kl:
        kl = torch.empty((bins + 1,), dtype=torch.float64, device=dev)
    _check(lib().w8a8_calibrate_entropy(_vec(hist, "hist", torch.int32), bins, _vec(amax, "amax"),
                                        _vec(scale, "scale"),
                                        _vec(kl, "kl", torch.float64) if kl is not None else None,
                                        _stream(stream)),
           "w8a8_calibrate_entropy")
    return scale, kl


# ---------------------------------------------------------------------------
# fused producers
# ---------------------------------------------------------------------------

def w8a8_rmsnorm_quantize(h, gamma, eps=1e-5, residual=None, xq=None, s_tok=None, stream=None):
    """(residual add into h,) RMSNorm with the folded weight, per-token codes.
    h bf16 [M, K] (updated in place when residual is given) -> (xq, s_tok)."""
    torch = _torch()
    M, K = _dims(h, "h")
    _length(gamma, "gamma", K)
    _shape(residual, "residual", M, K)
    _shape(xq, "xq", M, K)
    _length(s_tok, "s_tok", M)
    _one_device(h, gamma, residual, xq, s_tok)
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=h.device)
    if s_tok is None:
        s_tok = torch.empty((M,), dtype=torch.float32, device=h.device)
    ph, ldh = _mat(h, _bf16_types(), "h")
    pr, ldr = (None, K) if residual is None else _mat(residual, _bf16_types(), "residual")
    pq, ldq = _mat(xq, (torch.int8,), "xq")
    _check(lib().w8a8_rmsnorm_quantize(ph, ldh, pr, ldr, _vec(gamma, "gamma"), float(eps), M, K,
                                       pq, ldq, _vec(s_tok, "s_tok"), _stream(stream)),
           "w8a8_rmsnorm_quantize")
    return xq, s_tok


def w8a8_silu_mul_quantize(gu, smooth=None, xq=None, s_tok=None, stream=None):
    """gu bf16 [M, 2I] (gate | up) -> (xq int8 [M, I], s_tok fp32 [M])."""
    torch = _torch()
    M, two_i = _dims(gu, "gu")
    if two_i % 2:
        raise ValueError(f"gu: width {two_i} is not gate | up of equal halves")
    inter = two_i // 2
    _length(smooth, "smooth", inter)
    _shape(xq, "xq", M, inter)
    _length(s_tok, "s_tok", M)
    _one_device(gu, smooth, xq, s_tok)
    if xq is None:
        xq = torch.empty((M, inter), dtype=torch.int8, device=gu.device)
    if s_tok is None:
        s_tok = torch.empty((M,), dtype=torch.float32, device=gu.device)
    pg, ldg = _mat(gu, _bf16_types(), "gu")
    pq, ldq = _mat(xq, (torch.int8,), "xq")
    _check(lib().w8a8_silu_mul_quantize(pg, ldg, _vec(smooth, "smooth"), M, inter, pq, ldq,
                                        _vec(s_tok, "s_tok"), _stream(stream)),
           "w8a8_silu_mul_quantize")
    return xq, s_tok


def w8a8_fold_gamma(gamma, smooth=None, g=None, stream=None):
    torch = _torch()
    K = gamma.shape[0]
    _length(smooth, "smooth", K)
    _length(g, "g", K)
    _one_device(gamma, smooth, g)
    if g is None:
        g = torch.empty((K,), dtype=torch.float32, device=gamma.device)
    _check(lib().w8a8_fold_gamma(_vec(gamma, "gamma"), _vec(smooth, "smooth"), K, _vec(g, "g"),
                                 _stream(stream)), "w8a8_fold_gamma")
    return g


def w8a8_residual_add(h, r, stream=None):
    """h = bf16(h + r) in place."""
    M, K = _dims(h, "h")
    _shape(r, "r", M, K)
    _one_device(h, r)
    ph, ldh = _mat(h, _bf16_types(), "h")
    pr, ldr = _mat(r, _bf16_types(), "r")
    _check(lib().w8a8_residual_add(ph, ldh, pr, ldr, M, K, _stream(stream)), "w8a8_residual_add")
    return h


# ---------------------------------------------------------------------------
# GPTQ
# ---------------------------------------------------------------------------

def _dense_f64(t, name):
    torch = _torch()
    if t.dtype != torch.float64 or not t.is_contiguous() or t.device.type != "cuda":
        raise TypeError(f"{name}: need a contiguous float64 device tensor")
    return t.data_ptr()


def w8a8_gptq_hessian(x, smooth=None, H=None, stream=None):
    """H [K, K] float64 += 2 x'^T x' (zero-initialized when not given)."""
    torch = _torch()
    n, K = _dims(x, "x")
    _length(smooth, "smooth", K)
    _shape(H, "H", K, K)
    _one_device(x, smooth, H)
    if H is None:
        H = torch.zeros((K, K), dtype=torch.float64, device=x.device)
    px, ldx = _mat(x, _bf16_types(), "x")
    _check(lib().w8a8_gptq_hessian(px, ldx, _vec(smooth, "smooth"), n, K, _dense_f64(H, "H"),
                                   _stream(stream)), "w8a8_gptq_hessian")
    return H


def w8a8_gptq_factor_workspace_bytes(K: int) -> int:
    return lib().w8a8_gptq_factor_workspace_bytes(K)


def w8a8_gptq_factor(H, damp=0.01, U=None, workspace=None, stream=None):
    """U [K, K] float64, upper, U^T U = (H + lambda I)^-1."""
    torch = _torch()
    K = H.shape[0]
    _shape(H, "H", K, K)
    _shape(U, "U", K, K)
    _one_device(H, U, workspace)
    if U is None:
        U = torch.empty((K, K), dtype=torch.float64, device=H.device)
    nbytes = w8a8_gptq_factor_workspace_bytes(K)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=H.device)
    _check(lib().w8a8_gptq_factor(_dense_f64(H, "H"), K, float(damp), _dense_f64(U, "U"),
                                  workspace.data_ptr(), _nbytes(workspace), _stream(stream)),
           "w8a8_gptq_factor")
    return U


def w8a8_gptq_quantize_workspace_bytes(N: int, K: int) -> int:
    return lib().w8a8_gptq_quantize_workspace_bytes(N, K)


def w8a8_gptq_quantize(w, smooth, U, wq=None, s_chan=None, workspace=None, stream=None):
    """w bf16 [N, K] -> (wq int8 [N, K], s_chan fp32 [N]) with GPTQ error feedback."""
    torch = _torch()
    N, K = _dims(w, "w")
    _length(smooth, "smooth", K)
    _shape(U, "U", K, K)
    _shape(wq, "wq", N, K)
    _length(s_chan, "s_chan", N)
    _one_device(w, smooth, U, wq, s_chan, workspace)
    if wq is None:
        wq = torch.empty((N, K), dtype=torch.int8, device=w.device)
    if s_chan is None:
        s_chan = torch.empty((N,), dtype=torch.float32, device=w.device)
    nbytes = w8a8_gptq_quantize_workspace_bytes(N, K)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=w.device)
    pw, ldw = _mat(w, _bf16_types(), "w")
    pq, ldq = _mat(wq, (torch.int8,), "wq")
    _check(lib().w8a8_gptq_quantize(pw, ldw, _vec(smooth, "smooth"), _dense_f64(U, "U"), N, K,
                                    pq, ldq, _vec(s_chan, "s_chan"), workspace.data_ptr(),
                                    _nbytes(workspace), _stream(stream)), "w8a8_gptq_quantize")
    return wq, s_chan
