"""Helpers for the GPU parity tests: host <-> device marshalling and the
comparison rules (bit-exact for integers, <= 1 bf16 ulp for bf16 outputs).

The bf16 criterion is one ulp of the oracle's fp32-then-rounded value. The
kernels evaluate the same binary32 chain in the same order, so the tests
also assert what that gives: no distance at all (EXACT_BF16)."""
import numpy as np

REL_TOL = 2.0 ** -8      # relative error bound for bf16 outputs
ULP_TOL = 1              # ordered bf16 distance bound (the criterion)
EXACT_BF16 = True        # the kernels' epilogue is the oracle's binary32 chain


def torch():
    import torch as t
    return t


def dev_bf16(u16: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(u16).view(np.int16)).cuda().view(t.bfloat16)


def dev(a: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    tt = torch()
    t = t.detach()
    if t.dtype == tt.bfloat16:
        return t.view(tt.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_ordered(u16: np.ndarray) -> np.ndarray:
    b = u16.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def check_bf16(y_gpu: np.ndarray, y64: np.ndarray, y_oracle: np.ndarray, what: str = "y"):
    """GPU bf16 vs the oracle: within 1 bf16 ulp of the oracle's bf16 (its
    binary32 chain, rounded), relative error <= 2**-8 against the binary64
    value, exact 0. Returns (worst ulp distance, worst relative error)."""
    assert y_gpu.shape == y64.shape == y_oracle.shape
    dist = np.abs(bf16_ordered(y_gpu) - bf16_ordered(y_oracle))
    worst = int(dist.max()) if dist.size else 0
    assert worst <= ULP_TOL, f"{what}: bf16 distance {worst} at {np.unravel_index(dist.argmax(), dist.shape)}"
    if EXACT_BF16:
        assert worst == 0, f"{what}: bf16 differs from the binary32 chain by {worst} ulp"
    g = (y_gpu.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    zero = y64 == 0
    assert np.all(g[zero] == 0), f"{what}: nonzero where the exact value is 0"
    rel = np.abs(g[~zero] - y64[~zero]) / np.abs(y64[~zero])
    assert rel.size == 0 or rel.max() <= REL_TOL, f"{what}: relative error {rel.max()}"
    return worst, float(rel.max()) if rel.size else 0.0
