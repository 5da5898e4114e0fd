"""The LDS-DMA helper (dma16 in csrc/gemm_common.h) sets m0 inside inline
assembly and names it as clobbered; the compiler does not promise to keep
its own uses of a reserved register intact across such a statement. This
CPU test compiles every source that uses the helper for gfx950, with the
library's flags, and checks the generated code for what makes that safe:
every m0 write is the helper's own, directly followed by its DMA
instruction, and nothing else in any kernel reads or writes m0. It runs on
whatever compiler builds the library, so a compiler that starts using m0
in these kernels fails here instead of corrupting LDS on the GPU."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from int8_w8a8_quantized_token_amd import build as B

SOURCES = ["gemm.hip", "linear_fused.hip"]


def _asm(src, out):
    cmd = [B.hipcc(), *[f for f in B.HIPCC_FLAGS if f != "-fPIC"], "--cuda-device-only", "-S",
           "-o", out, os.path.join(B.CSRC, src)]
    subprocess.run(cmd, check=True, capture_output=True)
    with open(out) as f:
        return f.read()


@pytest.fixture(scope="module")
def listings(tmp_path_factory):
    if not os.path.exists(B.hipcc()) and B.hipcc() != "hipcc":
        pytest.skip("no hipcc")
    d = tmp_path_factory.mktemp("isa")
    with ThreadPoolExecutor(len(SOURCES)) as pool:
        texts = list(pool.map(lambda s: _asm(s, str(d / (s + ".s"))), SOURCES))
    return dict(zip(SOURCES, texts))


def kernels(text):
    """(name, instruction lines) of every function in an assembly listing."""
    out = []
    for m in re.finditer(r"^(_Z\S+):", text, re.M):
        end = text.index(".Lfunc_end", m.end())
        body = [ln.split(";")[0].strip() for ln in text[m.end():end].split("\n")]
        out.append((m.group(1), [ln for ln in body if ln and not ln.startswith(".")]))
    return out


@pytest.mark.parametrize("src", SOURCES)
def test_m0_is_only_the_dma_helpers(listings, src):
    dma_total = 0
    for name, ins in kernels(listings[src]):
        for i, ln in enumerate(ins):
            if not re.search(r"\bm0\b", ln):
                continue
            assert re.fullmatch(r"s_mov_b32 m0, s\d+", ln), f"{name}: m0 used by `{ln}`"
            assert ins[i + 1] == "s_nop 0", f"{name}: `{ln}` not followed by the helper's nop"
            assert ins[i + 2].startswith("global_load_lds_dwordx4 "), \
                f"{name}: m0 write not followed by its DMA (`{ins[i + 2]}`)"
        dmas = [i for i, ln in enumerate(ins) if ln.startswith("global_load_lds")]
        for i in dmas:
            assert re.fullmatch(r"s_mov_b32 m0, s\d+", ins[i - 2]), \
                f"{name}: DMA at {i} without the helper's m0 write"
        dma_total += len(dmas)
    assert dma_total > 0, f"{src}: no LDS DMA found (listing format changed?)"
