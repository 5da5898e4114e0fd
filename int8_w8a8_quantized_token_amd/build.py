"""Builds libw8a8.so (the gfx950 kernels and the C ABI) in-tree with hipcc.

    python -m int8_w8a8_quantized_token_amd.build

Each source compiles to its own object (in parallel), then one link makes
the shared library. The sources share no device code across files, so no
relocatable device code is needed.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libw8a8.so")
OBJ_DIR = os.path.join(os.path.dirname(HERE), "_build")
SOURCES = ["api.hip", "quantize.hip", "gemm.hip", "static_scale.hip", "producers.hip", "gptq.hip",
           "linear_fused.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-mcode-object-version=5", "-O3", "-std=c++17", "-fPIC",
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


def _jobs() -> int:
    env = os.environ.get("MAX_JOBS")
    n = int(env) if env and env.isdigit() else (os.cpu_count() or 1)
    return max(1, min(n, len(SOURCES), 16))


def build(out: str = LIB, extra=(), verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = [os.path.join(OBJ_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[hipcc(), *HIPCC_FLAGS, *extra, "-c", "-o", o, os.path.join(CSRC, s)]
            for s, o in zip(SOURCES, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    with ThreadPoolExecutor(_jobs()) as pool:
        results = list(pool.map(lambda c: subprocess.run(c, capture_output=True, text=True), cmds))
    failed = False
    for c, r in zip(cmds, results):
        if r.stderr and (verbose or r.returncode):
            sys.stderr.write(r.stderr)
        failed |= r.returncode != 0
    if failed:
        raise subprocess.CalledProcessError(1, "hipcc")
    link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out + ".tmp", *objs]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    print("built", LIB)
