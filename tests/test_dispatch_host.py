"""The GEMM dispatch rules (csrc/gemm_dispatch.h) on the host: compiled
with g++ into a small driver, fed shapes, checked against the choices
measured best on MI355X. No GPU."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CUS = 256          # MI355X compute units


@pytest.fixture(scope="module")
def pick(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("dispatch") / "dispatch_check")
    subprocess.run([cxx, "-std=c++17", "-O1", "-Wall", "-Werror", "-o", exe,
                    os.path.join(HERE, "dispatch_check.cpp")], check=True)

    def run(cases):
        text = "".join(f"{m} {n} {k} {c}\n" for m, n, k, c in cases)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True)
        lines = out.stdout.strip().split("\n")
        assert len(lines) == len(cases)
        res = []
        for ln in lines:
            f = ln.split()
            res.append((f[0],) + tuple(int(v) for v in f[1:]) if f[0] in ("mid", "skinny")
                       else tuple(f))
        return res
    return run


# Llama-3.1-8B projections (N, K) and Llama-3-70B ones
L8B = {"qkv": (6144, 4096), "o": (4096, 4096), "gate_up": (28672, 4096), "down": (4096, 14336)}
L70B = {"qkv": (10240, 8192), "o": (8192, 8192), "gate_up": (57344, 8192), "down": (8192, 28672)}


def classes_8b(M, N, K):
    """The fixed N classes measured best on the Llama-3.1-8B shapes, which
    the cost model must reproduce there: 16 channels per workgroup for
    N <= 4096, 32 for 4096 < N < 16384, 32 (one token group) or 64 above."""
    wide, mid, deep = N >= 16384, 4096 < N < 16384, K > 8192
    if M <= 16:
        return (1, 2, 4, 3) if (mid or wide) else (1, 1, 4, 4) if deep else (1, 1, 4, 3)
    if M <= 32:
        return ((2, 4, 4, 3) if wide else (2, 2, 4, 4) if mid else
                (2, 1, 4, 4) if deep else (2, 1, 8, 3))
    if M <= 48:
        return (3, 4, 2, 3) if wide else (3, 2, 4, 3) if mid else (3, 1, 4, 3)
    return (4, 4, 2, 2) if wide else (4, 2, 4, 3) if mid else (4, 1, 4, 3)


def test_decode_reproduces_the_8b_classes(pick):
    cases = [(M, N, K, CUS) for N, K in L8B.values() for M in range(1, 65)]
    got = pick(cases)
    for (M, N, K, _), g in zip(cases, got):
        assert g == ("mid",) + classes_8b(M, N, K), (M, N, K, g)


def test_decode_70b_shapes(pick):
    # qkv 8192 -> 10240: 16 channels per workgroup for one token group, 64
    # from two (the measured best); the other 70B projections keep the classes
    qkv = L70B["qkv"]
    want = {1: (1, 1, 4, 3), 16: (1, 1, 4, 3), 17: (2, 4, 4, 3), 32: (2, 4, 4, 3),
            40: (3, 4, 2, 3), 64: (4, 4, 2, 2)}
    got = pick([(M, *qkv, CUS) for M in want])
    assert got == [("mid",) + want[M] for M in want]
    cases = [(M, N, K, CUS) for p, (N, K) in L70B.items() if p != "qkv" for M in (1, 4, 16, 32, 64)]
    got = pick(cases)
    for (M, N, K, _), g in zip(cases, got):
        assert g == ("mid",) + classes_8b(M, N, K), (M, N, K, g)


def test_decode_and_prefill_limits(pick):
    cases = [(128, 28672, 4096), (129, 28672, 4096), (1024, 4096, 4096), (1025, 4096, 4096),
             (1536, 4096, 14336), (1537, 4096, 14336), (1, 4096, 4096 + 16), (500, 4096, 4096 + 16)]
    got = pick([c + (CUS,) for c in cases])
    assert got[0] == ("mid", 4, 4, 2, 2)
    assert got[1][0] == "prefill"
    assert got[2][0] == "mid" and got[3][0] == "prefill"
    assert got[4][0] == "mid" and got[5][0] == "prefill"
    assert got[6][0] == "skinny" and got[7] == ("tiled",)     # K % 128 != 0


def test_m_tiled_waves_by_rounds(pick):
    # 64 x 64 workgroups: 4 waves unless 2 waves need fewer rounds in units
    # of a 4-wave workgroup (qkv at 256 tokens: 384 workgroups, 2 waves; at
    # 512: 768 workgroups, 4 waves)
    got = pick([(100, 4096, 4096, CUS), (100, 6144, 4096, CUS), (100, 28672, 4096, CUS),
                (256, 6144, 4096, CUS), (512, 6144, 4096, CUS)])
    assert got == [("mid", 4, 2, 4, 3), ("mid", 4, 4, 4, 2), ("mid", 4, 4, 2, 2),
                   ("mid", 4, 4, 2, 2), ("mid", 4, 4, 4, 2)]


def test_prefill_tiles(pick):
    cases = {
        (3000, 4096, 4096): "256x192",      # one round either way: the smaller tile
        (3000, 4096, 14336): "256x192",
        (3000, 6144, 4096): "192x256",
        (4096, 6144, 4096): "192x256",      # 2 rounds of 3/4 tiles against 2 of whole ones
        (4096, 4096, 4096): "256x256",      # a smaller tile would need a second round
        (4096, 28672, 4096): "256x256",
        (3000, 28672, 4096): "256x256",     # 8 rounds of 3/4 tiles are not fewer than 6
        (4096, 4096, 14336): "256x256",
    }
    got = pick([k + (CUS,) for k in cases])
    assert got == [("prefill", v) for v in cases.values()]


def test_rules_follow_the_cu_count(pick):
    # The same shapes on devices with fewer CUs. 6144 channels at one token
    # on 128 CUs: 16 channels per workgroup cost 3 rounds x 32 rows, 32
    # channels 2 x 48, a tie that goes to 16. 4096 x 4096 at 4096 tokens on
    # 128 CUs: 256 x 256 tiles need 2 rounds and 192-row ones 3 of 3/4, so
    # whole tiles; 3000 tokens on 192 CUs: 192 tiles of 256 x 256 fill one
    # round and neither smaller tile still does.
    got = pick([(1, 6144, 4096, 128), (4096, 4096, 4096, 128), (3000, 4096, 4096, 192)])
    assert got[0] == ("mid", 1, 1, 4, 3)
    assert got[1] == ("prefill", "256x256")
    assert got[2] == ("prefill", "256x256")


def test_other_k_routes_and_skinny_classes(pick):
    # K % 128 != 0: the register-staged decode kernel up to 64 tokens, the
    # 128 x 128 tiles below 512 and the 64-byte-stage prefill kernel above;
    # the decode classes by N (wide > 8192, mid 4096..8192), K (deep > 8192)
    # and token count, with late scale loads where the table says so
    cases = {
        (1, 6144, 4112): ("skinny", 1, 2, 8, 8, 0),
        (4, 28672, 4112): ("skinny", 1, 1, 16, 2, 0),
        (1, 4096, 14352): ("skinny", 1, 1, 16, 2, 0),
        (3, 4096, 4112): ("skinny", 1, 1, 16, 8, 0),
        (16, 28672, 4112): ("skinny", 1, 4, 8, 2, 0),
        (16, 6144, 4112): ("skinny", 1, 2, 8, 8, 1),
        (16, 4096, 14352): ("skinny", 1, 1, 8, 4, 0),
        (32, 28672, 4112): ("skinny", 2, 4, 4, 2, 1),
        (48, 6144, 4112): ("skinny", 3, 2, 8, 2, 0),
        (64, 28672, 4112): ("skinny", 4, 4, 4, 2, 1),
        (64, 4096, 14352): ("skinny", 4, 1, 16, 2, 0),
        (64, 4096, 4112): ("skinny", 4, 1, 8, 8, 0),
        (65, 4096, 4112): ("tiled",),
        (511, 4096, 4112): ("tiled",),
        (512, 4096, 4112): ("prefill64",),
    }
    got = pick([k + (CUS,) for k in cases])
    assert got == list(cases.values())

