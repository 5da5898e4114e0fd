"""Host-side logic of bench.py: byte and op counts, step statistics, the
one-GPU guard and the code-hash gate on stored counter figures. No GPU."""
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


# Llama-3.1-8B projections (N, K): the byte counts of one W8A8 linear at 16
# tokens, X bf16 + smoothing fp32 + Wq int8 + channel scales fp32 + Y bf16.
@pytest.mark.parametrize("N,K,expect", [
    (6144, 4096, 25_534_464), (4096, 4096, 17_072_128),
    (28672, 4096, 118_620_160), (4096, 14336, 59_383_808)])
def test_linear_bytes_at_16_tokens(N, K, expect):
    assert bench.lin_bytes(16, N, K) == expect


def test_gemm_and_quantize_bytes():
    # GEMM: int8 codes + fp32 token scales + Wq + channel scales + bf16 out.
    assert bench.gemm_bytes(1, 1, 8) == 8 + 4 + 8 + 4 + 2
    # quantize: bf16 in + fp32 smoothing + int8 codes + fp32 scale.
    assert bench.quant_bytes(3, 8) == 48 + 32 + 24 + 12
    # The linear moves what the GEMM moves minus the codes and token scales
    # (an implementation intermediate), plus X and the smoothing vector.
    for M, N, K in ((1, 4096, 4096), (64, 28672, 4096)):
        assert bench.lin_bytes(M, N, K) == (bench.gemm_bytes(M, N, K) - M * K - 4 * M
                                            + 2 * M * K + 4 * K)


class _Clock:
    """Stand-in for torch: events read a clock that replays advance."""

    def __init__(self, durations):
        self.now, self.durations = 0.0, iter(durations)
        clock = self

        class Event:
            def __init__(self, enable_timing=True):
                self.t = None

            def record(self):
                self.t = clock.now

            def elapsed_time(self, other):
                return other.t - self.t

        self.cuda = types.SimpleNamespace(Event=Event, synchronize=lambda: None)

    def replay(self):
        self.now += next(self.durations)


def test_step_statistics():
    fake = _Clock([1.0] * 2 + list(range(1, 20)) + [100.0])   # 2 warm-up, 20 timed
    mean, st = bench.time_graph(fake, fake, 20, 2, stats=True)
    assert mean == pytest.approx(290.0 / 20)
    assert st == {"median_ms": 10.5, "p95_ms": 19.0, "mean_ms": 14.5}
    fake = _Clock([3.0, 1.0, 2.0])
    assert bench.time_graph(fake, fake, 3, 0, stats=True)[1]["median_ms"] == 2.0
    fake = _Clock([4.0] * 5)
    assert bench.time_graph(fake, fake, 5, 0) == pytest.approx(4.0)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_stored_traffic_follows_the_code(tmp_path, monkeypatch):
    # Stored counter figures are reported for the GEMM code they were taken
    # with and for no other; comments and blank lines do not count as code.
    for rel in bench.GEMM_SRCS:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_text(open(os.path.join(ROOT, rel)).read())
    stored = dict(bench.MEASURED_TRAFFIC, decode=111, prefill=222,
                  gemm_code_sha256=bench.code_sha256([str(tmp_path / r) for r in bench.GEMM_SRCS]))
    monkeypatch.setattr(bench, "MEASURED_TRAFFIC", stored)
    assert bench.measured_traffic(str(tmp_path), "decode") == 111
    assert bench.measured_traffic(str(tmp_path), "prefill") == 222
    gemm = tmp_path / bench.GEMM_SRCS[0]
    gemm.write_text(gemm.read_text() + "\n// a comment\n\n")
    assert bench.measured_traffic(str(tmp_path), "decode") == 111
    gemm.write_text(gemm.read_text() + "static int unused_marker;\n")
    assert bench.measured_traffic(str(tmp_path), "decode") is None
    monkeypatch.setattr(bench, "MEASURED_TRAFFIC", {})
    assert bench.measured_traffic(ROOT, "decode") is None


def test_clock_readout_never_raises():
    c = bench.gpu_clocks()
    assert isinstance(c, dict) and c


def test_clock_readout_parses_amd_smi(monkeypatch):
    import json
    import subprocess as sp
    clk = lambda v: {"clk": {"value": v, "unit": "MHz"}, "min_clk": {"value": 500, "unit": "MHz"}}
    doc = {"gpu_data": [{"gpu": 0, "clock": {
        **{f"gfx_{i}": clk(1700 + i) for i in (0, 2, 1, 10)},
        "mem_0": clk(2000), "vclk_0": {"clk": "N/A"}}}]}
    out = "note before\n" + json.dumps(doc, indent=2) + "\ntrailing text\n"
    monkeypatch.setattr(sp, "run", lambda *a, **k: types.SimpleNamespace(stdout=out, returncode=0))
    assert bench.gpu_clocks() == {"gfx_per_xcd": [1700, 1701, 1702, 1710], "mem": 2000}


def test_oracle_timing_passes_run_until_the_budget():
    calls = []

    def one_pass():
        calls.append(1)
        return 0.4, 10.0
    t, work, passes = bench._time_passes(one_pass, 1.0)
    assert passes == 3 and t == pytest.approx(1.2) and work == 30.0
    host = bench._cpu_host()
    assert host["kind"] == "oracle" and host["cores"] >= 1 and host["cpus_in_affinity"] >= 1


def test_clocks_are_read_while_the_graph_replays(monkeypatch):
    state = {"replays": 0, "at_read": None, "running": True}

    class Graph:
        def replay(self):
            state["replays"] += 1
            import time
            time.sleep(0.002)              # a replay keeps the device busy a while

    def clocks():
        state["at_read"] = state["replays"]
        return {"gfx_per_xcd": [1900] * 8, "mem": 2000}

    fake_torch = types.SimpleNamespace(cuda=types.SimpleNamespace(synchronize=lambda: None))
    monkeypatch.setattr(bench, "gpu_clocks", clocks)
    out = bench.clocks_under_load(fake_torch, Graph(), 2.0, seconds=0.3)
    assert out["gfx_per_xcd"] == [1900] * 8 and out["replays"] == state["replays"]
    # read after the load started and before it ended
    assert 0 < state["at_read"] < state["replays"]
