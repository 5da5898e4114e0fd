"""CPU checks of the fast paths in the gfx950 kernels.

* Quantizers: the int8 code round(x' / S) as rint(x' * RN(1/S)), accepted
  only when the product is more than 1/2 - 2^-15 away from the next
  half-integer; the rest divide. Checked where that bound is tightest.
* MLP producer: bf16(g / (1 + e^-g) * u) from a binary32 evaluation with a
  bounded error, accepted only away from bf16 rounding boundaries; the rest
  in binary64. Checked for every pair of finite bf16 inputs.

The C programs emulate the device's IEEE binary32 operations (no flush to
zero, no contraction) and return nonzero on any mismatch. They need gcc;
without it the tests are skipped.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "exhaustive")


def _run(src, tmp_path, parallel=False):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "check")
    cmd = [gcc, "-O2", "-ffp-contract=off", "-fno-fast-math", "-o", exe, os.path.join(HERE, src), "-lm"]
    if parallel and subprocess.run(cmd[:1] + ["-fopenmp"] + cmd[1:], capture_output=True).returncode == 0:
        pass                                        # built with OpenMP
    else:
        subprocess.run(cmd, check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    print(out.stdout)
    assert out.returncode == 0, out.stdout
    assert " 0 mismatches" in out.stdout


def test_quantize_fast_path(tmp_path):
    _run("quantize_fastpath_check.c", tmp_path)


def test_silu_fast_path(tmp_path):
    _run("silu_fastpath_check.c", tmp_path, parallel=True)
