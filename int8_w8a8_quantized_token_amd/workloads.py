"""Seeded synthetic inputs for the W8A8 INT8 linear layer.

This module only draws random numbers and names shapes. It holds none of the
layer's arithmetic (no scales, no rounding to int8, no GEMM), so both the HIP
path and the CPU oracle may take their inputs from it.

Shapes are the projection shapes of the Llama-3.1-8B and Llama-3-70B
transformer layers that the Red Hat article "Understanding W8A8 INT8 LLM
quantization: Half the size, better performance, same accuracy" compresses
(section "The experiment: What we built and why"). Value distributions stand
in for the activations that article describes in "Why activation quantization
is hard, and how SmoothQuant fixes it": roughly unit-scale token activations
with a few persistent outlier channels that are much larger than the rest.

Every array is drawn from numpy's PCG64 seeded through SeedSequence with a
spawn key that names (workload, layer, role), drawn in float32, and rounded to
bf16 by torch's CPU cast (round-to-nearest-even). bf16 tensors are handed out
as their raw uint16 bit patterns.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass

import numpy as np

ROOT_SEED = 0

# (name, N, K): output channels N, input channels K.
LLAMA31_8B = (("qkv", 6144, 4096), ("o", 4096, 4096),
              ("gate_up", 28672, 4096), ("down", 4096, 14336))
LLAMA3_70B = (("qkv", 10240, 8192), ("o", 8192, 8192),
              ("gate_up", 57344, 8192), ("down", 8192, 28672))


@dataclass(frozen=True)
class Workload:
    name: str
    shapes: tuple          # ((proj, N, K), ...)
    ms: tuple              # token counts M
    w_std: float           # weight ~ N(0, w_std)
    outlier_frac: float    # fraction of input channels that carry outliers
    outlier_mult: float    # outlier channels are multiplied by this


WORKLOADS = {
    # one 4096x4096 linear at 16 tokens; small enough for the oracle in full
    "single": Workload("single", (("o", 4096, 4096),), (16,), 0.02, 0.01, 20.0),
    # Llama-3.1-8B decode projections
    "llama8b_decode": Workload("llama8b_decode", LLAMA31_8B, (1, 4, 16, 64),
                               0.02, 0.01, 20.0),
    # Llama-3.1-8B prefill projections
    "llama8b_prefill": Workload("llama8b_prefill", LLAMA31_8B, (4096,),
                                0.02, 0.01, 20.0),
    # Llama-3-70B per-layer projections on one GPU
    "llama70b": Workload("llama70b", LLAMA3_70B, (32, 2048), 0.015, 0.005, 30.0),
    # 32-layer chain of config-1 shapes, ragged batch of 8 sequences (3000 tokens)
    "llama8b_chain": Workload("llama8b_chain", LLAMA31_8B, (3000,), 0.02, 0.01, 20.0),
}


def _key(*parts) -> tuple:
    out = []
    for p in parts:
        if isinstance(p, str):
            out.append(zlib.crc32(p.encode()) & 0x7FFFFFFF)
        else:
            out.append(int(p))
    return tuple(out)


def rng(*parts) -> np.random.Generator:
    """Generator for the stream named by ``parts`` (strings or ints)."""
    ss = np.random.SeedSequence(ROOT_SEED, spawn_key=_key(*parts))
    return np.random.Generator(np.random.PCG64(ss))


def to_bf16_bits(a32: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16) via torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def outlier_channels(K: int, frac: float, *key) -> np.ndarray:
    """round(frac*K) distinct channel indices, seeded, sorted."""
    n = int(round(frac * K))
    return np.sort(rng("outliers", K, *key).choice(K, size=n, replace=False))


def activations(M: int, K: int, *key, frac: float = 0.01, mult: float = 20.0,
                outliers: np.ndarray | None = None) -> np.ndarray:
    """bf16 [M, K]: N(0,1) with the outlier channels scaled by ``mult``."""
    a = rng("act", M, K, *key).standard_normal((M, K), dtype=np.float32)
    if outliers is None:
        outliers = outlier_channels(K, frac, *key)
    if len(outliers):
        a[:, outliers] *= np.float32(mult)
    return to_bf16_bits(a)


def weights(N: int, K: int, std: float, *key) -> np.ndarray:
    """bf16 [N, K]: N(0, std)."""
    w = rng("w", N, K, *key).standard_normal((N, K), dtype=np.float32)
    w *= np.float32(std)
    return to_bf16_bits(w)


def ragged_lengths(total: int, parts: int, *key) -> np.ndarray:
    """``parts`` sequence lengths >= 1 summing to ``total`` (seeded multinomial)."""
    r = rng("lens", total, parts, *key)
    extra = r.multinomial(total - parts, np.full(parts, 1.0 / parts))
    return extra + 1


def layer_inputs(wl: Workload, proj: str, N: int, K: int, M: int, layer: int = 0):
    """(x_bf16 [M,K], w_bf16 [N,K]) for one projection of one layer of ``wl``.

    Outlier channels depend only on (workload, K), so every projection that
    reads the same hidden size sees the same persistent outlier channels.
    """
    out = outlier_channels(K, wl.outlier_frac, wl.name)
    x = activations(M, K, wl.name, proj, layer, outliers=out, mult=wl.outlier_mult)
    w = weights(N, K, wl.w_std, wl.name, proj, layer)
    return x, w
