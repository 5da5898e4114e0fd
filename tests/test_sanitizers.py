"""Host code under the address and undefined-behaviour sanitizers (CPU only):
the GEMM dispatch rules (csrc/gemm_dispatch.h) over a sweep of shapes up to
the largest the ABI accepts, and the C ABI's argument validation (api.hip's
host code, with every kernel launcher stubbed to abort) over refused and
empty calls at extreme sizes. Any sanitizer report fails the run."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def test_dispatch_rules_under_sanitizers(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no g++")
    exe = str(tmp_path / "dispatch_check")
    subprocess.run([cxx, "-std=c++17", "-O1", "-g", *SAN, "-o", exe,
                    os.path.join(HERE, "dispatch_check.cpp")], check=True)
    ms = [0, 1, 2, 3, 15, 16, 17, 63, 64, 65, 127, 128, 129, 1023, 1024, 1536, 1537, 3000, 4096,
          65535, 2**31 - 1]
    ns = [1, 15, 16, 4096, 16383, 16384, 57344, 2**31 - 1]
    ks = [16, 48, 128, 4096, 8192, 8320, 14336, 28672, 131072]
    lines = [f"{m} {n} {k} {c}\n" for m in ms for n in ns for k in ks for c in (1, 80, 256, 1024)]
    r = subprocess.run([exe], input="".join(lines), capture_output=True, text=True, env=ENV)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-2000:]
    assert len(r.stdout.strip().split("\n")) == len(lines)


def test_abi_validation_under_sanitizers(tmp_path):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clangxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not (os.path.exists(hipcc) and os.path.exists(clangxx)):
        pytest.skip("no ROCm toolchain")
    api_o, chk_o, exe = (str(tmp_path / n) for n in ("api.o", "check.o", "abi_check"))
    # api.hip: device code as usual, host code with the sanitizers
    host_san = []
    for f in SAN:
        host_san += ["-Xarch_host", f]
    subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g",
                    *host_san, "-c", "-o", api_o,
                    os.path.join(ROOT, "int8_w8a8_quantized_token_amd", "csrc", "api.hip")],
                   check=True, capture_output=True)
    subprocess.run([clangxx, "-std=c++17", "-O1", "-g", *SAN, "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROCM, "include"), "-c", "-o", chk_o,
                    os.path.join(HERE, "abi_host_check.cpp")], check=True)
    subprocess.run([clangxx, *SAN, "-o", exe, api_o, chk_o, "-L", os.path.join(ROCM, "lib"),
                    "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV)
    assert r.returncode == 0, r.stdout + r.stderr[-3000:]
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-3000:]
    assert "abi host checks ok" in r.stdout
