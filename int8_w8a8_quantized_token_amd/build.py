"""Builds libw8a8.so (the gfx950 kernels and the C ABI) in-tree with hipcc.

    python -m int8_w8a8_quantized_token_amd.build
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libw8a8.so")
SOURCES = ["api.hip", "quantize.hip", "gemm.hip", "static_scale.hip", "producers.hip", "gptq.hip", "linear_fused.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-mcode-object-version=5", "-O3", "-std=c++17", "-fPIC", "-shared",
    # every floating-point step is one IEEE operation in the written order
    "-ffp-contract=off", "-fno-fast-math",
    # packed fp32 ops are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(out: str = LIB, extra=(), verbose: bool = False) -> str:
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-o", out + ".tmp",
           *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    print("built", LIB)
