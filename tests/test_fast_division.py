"""CPU check of the division-free rounding step in the gfx950 quantizers.

The kernels compute the int8 code round(x' / S) as rint(x' * RN(1/S)) and
accept it only when the product is more than 1/2 - 2^-15 away from the next
half-integer; the rest divide. The C program emulates the device's IEEE
binary32 operations (no flush to zero, no contraction) where that bound is
tightest and returns nonzero on any mismatch. It needs gcc; without it the
test is skipped.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "exhaustive")


def _run(src, tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "check")
    cmd = [gcc, "-O2", "-ffp-contract=off", "-fno-fast-math", "-o", exe, os.path.join(HERE, src), "-lm"]
    subprocess.run(cmd, check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    print(out.stdout)
    assert out.returncode == 0, out.stdout
    assert " 0 mismatches" in out.stdout


def test_quantize_fast_path(tmp_path):
    _run("quantize_fastpath_check.c", tmp_path)
