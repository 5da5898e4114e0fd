#!/usr/bin/env python3
"""Benchmark of the W8A8 INT8 linear layer on one MI355X (gfx950).

Workload: the Llama-3.1-8B projections (qkv 4096->6144, o 4096->4096,
gate_up 4096->28672, down 14336->4096) over 32 layers with distinct weight
buffers (7 GB of int8 weights, far beyond the 256 MB Infinity Cache), on
seeded synthetic bf16 inputs with 1% outlier channels x20.

  * decode step (the headline `value`): one forward through 32 layers x 4
    projections at each token count M in {1, 4, 16, 64}; every linear is a
    w8a8_linear call (quantize + skinny GEMM + epilogue). Metric: algorithmic
    HBM bytes per second, bytes = 2MK + 4K + NK + 4N + 2MN per linear.
  * prefill step (reported under "prefill"): the same 128 linears at
    M = 4096. Metric: int8 TOPS = 2MNK per linear / time.

Each step is captured once in a HIP graph and replayed; W untimed warmup
steps, then K timed steps between two events on the replay stream (one
more event after each replay gives the median, 95th percentile and mean).
The roofline entry times the dominant kernel (the GEMM) alone: a graph of
the step's GEMM launches only, timed the same way; its average launch
duration is the graph time over the number of launches.

Also reported: the decode step split by token count (decode_by_m, whole
linear and GEMM alone against the HBM peak); the same decode step with one
calibrated activation scale per projection (static_decode); a 32-layer
block chain at 3000 tokens with the fused norm and SiLU producers (chain),
with its drift from an unquantized fp32 forward after 1, 8 and 32 layers;
the Llama-3-70B projections at 32 and 2048 tokens (llama70b); the cost of a
kernel boundary in a graph (dispatch_floor_us); the shader and memory clocks
before and after; and the CPU oracle on a bounded sample beside each line
(cpu_baseline at the top level for decode, and inside prefill, chain and
llama70b). --detail adds per-shape
times of the linear, the GEMM alone and the quantizer alone; --counters
only launches every GEMM once for hardware-counter passes.
"""
import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, TOPS
LAYERS = 32
DECODE_MS = (1, 4, 16, 64)
PREFILL_M = 4096
METRIC = "W8A8 GEMM int8 TOPS (prefill) + HBM GB/s (decode), Llama-3.1-8B shapes"


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip timing the CPU oracle")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-chain", action="store_true", help="skip the 32-layer block chain")
    p.add_argument("--no-70b", action="store_true", help="skip the Llama-3-70B projections")
    p.add_argument("--detail", action="store_true", help="per-shape timings on stderr")
    p.add_argument("--counters", action="store_true",
                   help="eager launches for hardware-counter runs (rocprofv3 --pmc); no timing")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# HBM bytes per launch of the two roofline kernels, from two rocprofv3 --pmc
# passes over `bench.py --counters` (FETCH_SIZE, then WRITE_SIZE, KiB per
# dispatch), each scaled by the factor that makes the 1 GiB device copy in the
# same run count exactly its own bytes. "decode": mean over the 16 decode
# (projection, M) GEMMs; "prefill": mean over the 4 GEMMs at M = 4096. The
# figures belong to the GEMM code with the recorded SHA-256 (taken over the
# GEMM sources and the headers they include, comments and blank lines
# removed) only; for any other code the field is null.
MEASURED_TRAFFIC = {
    "gemm_code_sha256": "95bc7ca3ba832f11e7adbf2361ef994f87e348290ae2cda7ea17462d76d21e67",
    "decode": 56273860,
    "prefill": 427229136,
}
GEMM_SRCS = [os.path.join("int8_w8a8_quantized_token_amd", "csrc", f)
             for f in ("gemm.hip", "gemm_common.h", "gemm_dispatch.h", "device_common.h")]


def code_sha256(paths):
    """SHA-256 of C++ sources without their // comments and blank lines."""
    import hashlib
    import re
    lines = []
    for path in paths:
        with open(path, encoding="utf-8") as f:
            for line in f.read().split("\n"):
                line = re.sub(r"//.*$", "", line).rstrip()
                if line.strip():
                    lines.append(line)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def measured_traffic(root, which):
    if not MEASURED_TRAFFIC:
        return None
    if code_sha256([os.path.join(root, p) for p in GEMM_SRCS]) != MEASURED_TRAFFIC["gemm_code_sha256"]:
        return None
    return MEASURED_TRAFFIC[which]


def lin_bytes(M, N, K):
    return 2 * M * K + 4 * K + N * K + 4 * N + 2 * M * N


def quant_bytes(M, K):
    return 2 * M * K + 4 * K + M * K + 4 * M


def gemm_bytes(M, N, K):
    return M * K + 4 * M + N * K + 4 * N + 2 * M * N


class Setup:
    """Device buffers for all layers and token counts."""

    def __init__(self, torch, W, WL, ms):
        self.torch, self.W = torch, W
        wl = WL.WORKLOADS["llama8b_decode"]
        self.shapes = wl.shapes
        self.ms = ms
        dev = "cuda"
        self.s, self.sw, self.wq, self.S_static = {}, {}, {}, {}
        self.x, self.y, self.ws, self.xq, self.st = {}, {}, {}, {}, {}
        self.w_host = {}        # the unquantized bf16 weights (drift reference of the chain)
        t0 = time.time()
        for proj, N, K in self.shapes:
            outl = WL.outlier_channels(K, wl.outlier_frac, wl.name)
            xcal = WL.activations(PREFILL_M, K, wl.name, proj, 0, outliers=outl,
                                  mult=wl.outlier_mult)
            w = WL.weights(N, K, wl.w_std, wl.name, proj, 0)
            self.w_host[proj] = w
            xcal_d = self.bf16(xcal)
            w_d = self.bf16(w)
            # offline prep on the GPU: calibrate, smooth, quantize per channel
            s = W.w8a8_smoothing_factors(W.w8a8_channel_absmax(xcal_d), W.w8a8_channel_absmax(w_d))
            wq, sw = W.w8a8_quantize_weight(w_d, s)
            del w_d
            self.s[proj], self.sw[proj] = s, sw
            # static per-tensor activation scale, entropy-calibrated on the GPU
            amax, _ = W.w8a8_calibrate_minmax(W.w8a8_channel_absmax(xcal_d), s)
            hist = W.w8a8_activation_histogram(xcal_d, s, amax)
            self.S_static[proj], _ = W.w8a8_calibrate_entropy(hist, amax)
            # layer 0 owns the prepared weight; layers 1.. get copies in
            # distinct buffers so every layer streams its own bytes from HBM
            self.wq[proj] = [wq] + [wq.clone() for _ in range(LAYERS - 1)]
            for M in ms:
                xm = xcal_d[:M].clone() if M == PREFILL_M else self.bf16(
                    WL.activations(M, K, wl.name, proj, 0, outliers=outl, mult=wl.outlier_mult))
                self.x[proj, M] = xm
                self.y[proj, M] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                nb = W.w8a8_linear_workspace_bytes(M, K)
                self.ws[proj, M] = torch.empty((nb,), dtype=torch.uint8, device=dev)
                off = (M * K + 255) // 256 * 256
                self.xq[proj, M] = self.ws[proj, M][:M * K].view(torch.int8).view(M, K)
                self.st[proj, M] = self.ws[proj, M][off:off + 4 * M].view(torch.float32)
            del xcal_d
        torch.cuda.synchronize()
        log(f"[bench] setup {time.time() - t0:.1f}s, "
            f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB on device")

    def bf16(self, u16):
        import numpy as np
        t = self.torch.from_numpy(np.ascontiguousarray(u16).view(np.int16))
        return t.cuda().view(self.torch.bfloat16)

    def linear(self, proj, M, layer):
        W = self.W
        W.w8a8_linear(self.x[proj, M], self.s[proj], self.wq[proj][layer], self.sw[proj],
                      y=self.y[proj, M], workspace=self.ws[proj, M])

    def linear_static(self, proj, M, layer):
        self.W.w8a8_linear_static(self.x[proj, M], self.s[proj], self.S_static[proj],
                                  self.wq[proj][layer], self.sw[proj], y=self.y[proj, M],
                                  workspace=self.ws[proj, M])

    def quantize(self, proj, M):
        self.W.w8a8_quantize_act(self.x[proj, M], self.s[proj], xq=self.xq[proj, M],
                                 s_tok=self.st[proj, M])

    def gemm(self, proj, M, layer):
        self.W.w8a8_gemm(self.xq[proj, M], self.st[proj, M], self.wq[proj][layer],
                         self.sw[proj], y=self.y[proj, M])


def capture(torch, fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, steps, warmup, stats=False):
    """Mean ms per replay over `steps` timed replays; with stats, also the
    median, 95th percentile and mean of the single replays (one event after
    each replay, inside the same timed region)."""
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1 if stats else 2)]
    ev[0].record()
    for i in range(steps):
        g.replay()
        if stats:
            ev[i + 1].record()
    ev[-1].record()
    torch.cuda.synchronize()
    mean = ev[0].elapsed_time(ev[-1]) / steps
    if not stats:
        return mean
    each = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    median = each[steps // 2] if steps % 2 else 0.5 * (each[steps // 2 - 1] + each[steps // 2])
    p95 = each[math.ceil(0.95 * steps) - 1]             # nearest rank
    return mean, {"median_ms": round(median, 4), "p95_ms": round(p95, 4),
                  "mean_ms": round(mean, 4)}


def dispatch_floor_us(torch, launches=512, steps=10):
    """Per-launch time of a graph of one-element fills: the cost of a kernel
    boundary in a graph, against which the small decode kernels are read."""
    t = torch.zeros(1, dtype=torch.float32, device="cuda")
    g = capture(torch, lambda: [t.fill_(0.0) for _ in range(launches)])
    ms = time_graph(torch, g, steps, 2)
    return round(ms / launches * 1e3, 3)


def gpu_clocks():
    """Current clocks (MHz) as amd-smi reports them: the shader clock of each
    XCD and the memory clock; the error text instead when the tool is missing
    or prints something else."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "--json"],
                           capture_output=True, text=True, timeout=30)
        doc, _ = json.JSONDecoder().raw_decode(r.stdout[r.stdout.index("{"):])
        clocks = doc["gpu_data"][0]["clock"]
        gfx = [clocks[k]["clk"]["value"] for k in sorted(clocks, key=lambda k: int(k.split("_")[-1]))
               if k.startswith("gfx_") and isinstance(clocks[k].get("clk"), dict)]
        mem = clocks.get("mem_0", {}).get("clk", {})
        return {"gfx_per_xcd": gfx, "mem": mem.get("value") if isinstance(mem, dict) else None}
    except Exception as e:                       # noqa: BLE001 -- reported, not raised
        return {"error": f"{type(e).__name__}: {str(e)[:120]}"}


def clocks_under_load(torch, graph, ms_per_replay, seconds=3.0):
    """The clocks (as gpu_clocks reports them) read while `graph` replays back
    to back for about `seconds`: a side thread reads them a third of the way
    in, while the main thread keeps the queue full."""
    import threading
    res = {}

    def sample():
        time.sleep(seconds / 3)
        res["clk"] = gpu_clocks()

    t = threading.Thread(target=sample)
    t.start()
    end = time.monotonic() + seconds
    n = 0
    while n < 2 or time.monotonic() < end:
        graph.replay()
        n += 1
        if n % 8 == 0:                    # keep at most a few replays queued ahead
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t.join()
    out = dict(res.get("clk", {"error": "no reading"}))
    out["replays"] = n
    out["replay_ms"] = round(ms_per_replay, 3)
    return out


def run_phase(torch, S, ms, steps, warmup, detail, on_gemm_graph=None):
    """Times one step (all layers, projections, token counts) and its GEMMs;
    on_gemm_graph(graph, ms) runs on the timed GEMM graph afterwards."""
    def step():
        for M in ms:
            for layer in range(LAYERS):
                for proj, _, _ in S.shapes:
                    S.linear(proj, M, layer)

    def gemms():
        for M in ms:
            for layer in range(LAYERS):
                for proj, _, _ in S.shapes:
                    S.gemm(proj, M, layer)

    for M in ms:                     # fill the workspaces the GEMM graph reads
        for proj, _, _ in S.shapes:
            S.quantize(proj, M)
    g_step = capture(torch, step)
    ms_step, step_stats = time_graph(torch, g_step, steps, warmup, stats=True)
    g_gemm = capture(torch, gemms)
    ms_gemm = time_graph(torch, g_gemm, steps, warmup)
    if on_gemm_graph is not None:
        on_gemm_graph(g_gemm, ms_gemm)
    launches = len(ms) * LAYERS * len(S.shapes)
    per = {}
    if detail:
        for M in ms:
            for proj, N, K in S.shapes:
                g = capture(torch, lambda: [S.linear(proj, M, l) for l in range(LAYERS)])
                t = time_graph(torch, g, max(steps // 4, 2), 2) / LAYERS
                g2 = capture(torch, lambda: [S.gemm(proj, M, l) for l in range(LAYERS)])
                t2 = time_graph(torch, g2, max(steps // 4, 2), 2) / LAYERS
                g3 = capture(torch, lambda: [S.quantize(proj, M) for _ in range(LAYERS)])
                t3 = time_graph(torch, g3, max(steps // 4, 2), 2) / LAYERS
                per[f"{proj}_M{M}"] = {"linear_us": round(t * 1e3, 2), "gemm_us": round(t2 * 1e3, 2),
                                       "quantize_us": round(t3 * 1e3, 2),
                                       "linear_GBps": round(lin_bytes(M, N, K) / (t * 1e-3) / 1e9, 1),
                                       "gemm_GBps": round(gemm_bytes(M, N, K) / (t2 * 1e-3) / 1e9, 1),
                                       "quantize_GBps": round(quant_bytes(M, K) / (t3 * 1e-3) / 1e9, 1),
                                       "gemm_TOPS": round(2 * M * N * K / (t2 * 1e-3) / 1e12, 1)}
                log(f"[bench] {proj:8s} M={M:5d}: linear {t*1e3:8.2f} us  gemm {t2*1e3:8.2f} us  "
                    f"{per[f'{proj}_M{M}']}")
    return ms_step, ms_gemm, launches, per, step_stats


def counters(torch, S, ms, layers=4):
    """Eager launches for hardware-counter passes: every decode GEMM (projection,
    M) on `layers` distinct weight buffers, every prefill GEMM once per layer on
    two layers, then three copies of 1 GiB between device buffers (the
    calibration: each reads and writes exactly 2^30 bytes)."""
    for M in ms:
        for proj, _, _ in S.shapes:
            S.quantize(proj, M)
    torch.cuda.synchronize()
    for M in ms:
        n = layers if M != PREFILL_M else 2
        for layer in range(n):
            for proj, N, K in S.shapes:
                S.gemm(proj, M, layer)
        torch.cuda.synchronize()
        log(f"[counters] M={M}: {n} layers x {len(S.shapes)} GEMMs")
    src = torch.empty(2**30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("[counters] 3 x 1 GiB device copies")


CHAIN_M = 3000


def run_chain(torch, W, WL, S, args):
    """The Llama-shaped block chain: 32 layers on 3000 tokens, every
    activation entering a linear produced as int8 codes by a fused producer
    (residual add + RMSNorm with the smoothing folded into its weight,
    SiLU-gated product), the q slice of qkv standing in for attention.
    Weights are the decode setup's distinct per-layer buffers."""
    dev = "cuda"
    M, hid, inter = CHAIN_M, 4096, 14336
    shp = {p: (n, k) for p, n, k in S.shapes}
    outl = WL.outlier_channels(hid, 0.01, "llama8b_chain")
    gamma = torch.ones(hid, dtype=torch.float32, device=dev)
    gamma[torch.from_numpy(outl).to(dev)] = 20.0
    g_attn = W.w8a8_fold_gamma(gamma, S.s["qkv"])
    g_mlp = W.w8a8_fold_gamma(gamma, S.s["gate_up"])
    x0 = S.bf16(WL.activations(M, hid, "llama8b_chain", "x", outliers=outl))
    h = torch.empty_like(x0)
    y = {p: torch.empty((M, shp[p][0]), dtype=torch.bfloat16, device=dev) for p in shp}
    xq = torch.empty((M, inter), dtype=torch.int8, device=dev)
    st = torch.empty((M,), dtype=torch.float32, device=dev)

    def q_view(k):
        return xq[:, :k]

    def layers(with_gemm):
        h.copy_(x0)
        pending = None
        for layer in range(LAYERS):
            W.w8a8_rmsnorm_quantize(h, g_attn, 1e-5, residual=pending, xq=q_view(hid), s_tok=st)
            if with_gemm:
                W.w8a8_gemm(q_view(hid), st, S.wq["qkv"][layer], S.sw["qkv"], y=y["qkv"])
            W.w8a8_quantize_act(y["qkv"][:, :hid], S.s["o"], xq=q_view(hid), s_tok=st)
            if with_gemm:
                W.w8a8_gemm(q_view(hid), st, S.wq["o"][layer], S.sw["o"], y=y["o"])
            W.w8a8_rmsnorm_quantize(h, g_mlp, 1e-5, residual=y["o"], xq=q_view(hid), s_tok=st)
            if with_gemm:
                W.w8a8_gemm(q_view(hid), st, S.wq["gate_up"][layer], S.sw["gate_up"],
                            y=y["gate_up"])
            W.w8a8_silu_mul_quantize(y["gate_up"], S.s["down"], xq=xq, s_tok=st)
            if with_gemm:
                W.w8a8_gemm(xq, st, S.wq["down"][layer], S.sw["down"], y=y["down"])
            pending = y["down"]
        W.w8a8_residual_add(h, pending)

    for v in y.values():
        v.zero_()
    g_full = capture(torch, lambda: layers(True))
    t_full = time_graph(torch, g_full, max(args.steps // 4, 3), min(args.warmup, 2))
    del g_full
    g_prod = capture(torch, lambda: layers(False))
    t_prod = time_graph(torch, g_prod, max(args.steps // 4, 3), min(args.warmup, 2))
    del g_prod
    ops = sum(2 * M * n * k for n, k in shp.values()) * LAYERS
    # producer bytes per layer: two norms (read h and the residual, write h,
    # write codes), the q-slice quantizer, the SiLU product (read gate|up,
    # write codes); scales and vectors are negligible
    pbytes = LAYERS * (2 * (2 * M * hid * 3 + M * hid) + (2 * M * hid + M * hid)
                       + (2 * M * 2 * inter + M * inter))
    tops = ops / (t_full * 1e-3) / 1e12
    log(f"[bench] chain: 32 layers x {M} tokens {t_full:.3f} ms ({tops:.0f} TOPS); "
        f"producers alone {t_prod:.3f} ms ({pbytes / (t_prod * 1e-3) / 1e9:.0f} GB/s)")
    out = {"value": round(tops, 1), "unit": "TOPS", "ms_per_forward": round(t_full, 4),
           "producers_ms": round(t_prod, 4),
           "producers_GBps": round(pbytes / (t_prod * 1e-3) / 1e9, 1),
           "config": {"workload": "llama8b_chain: 32 layers x (fused norm/SiLU producers + "
                                  "4 W8A8 GEMMs), 3000 tokens, q slice for attention",
                      "tokens": M}}

    # drift of the W8A8 chain from the unquantized model: the residual stream
    # of sampled token rows after 1, 8 and 32 layers against an fp32 forward
    # of the same block structure with the bf16 weights unquantized (RMSNorm
    # with gamma, no smoothing: it cancels in exact arithmetic)
    import numpy as np
    t0 = time.time()
    rows = np.sort(WL.rng("chain-drift").choice(M, size=8, replace=False))
    rows_d = torch.from_numpy(rows).to(dev)
    snaps = {}
    h.copy_(x0)
    pending = None
    for layer in range(LAYERS):
        W.w8a8_rmsnorm_quantize(h, g_attn, 1e-5, residual=pending, xq=q_view(hid), s_tok=st)
        W.w8a8_gemm(q_view(hid), st, S.wq["qkv"][layer], S.sw["qkv"], y=y["qkv"])
        W.w8a8_quantize_act(y["qkv"][:, :hid], S.s["o"], xq=q_view(hid), s_tok=st)
        W.w8a8_gemm(q_view(hid), st, S.wq["o"][layer], S.sw["o"], y=y["o"])
        W.w8a8_rmsnorm_quantize(h, g_mlp, 1e-5, residual=y["o"], xq=q_view(hid), s_tok=st)
        W.w8a8_gemm(q_view(hid), st, S.wq["gate_up"][layer], S.sw["gate_up"], y=y["gate_up"])
        W.w8a8_silu_mul_quantize(y["gate_up"], S.s["down"], xq=xq, s_tok=st)
        W.w8a8_gemm(xq, st, S.wq["down"][layer], S.sw["down"], y=y["down"])
        pending = y["down"]
        if layer + 1 in (1, 8, LAYERS):
            hs = h.index_select(0, rows_d).contiguous()
            W.w8a8_residual_add(hs, pending.index_select(0, rows_d).contiguous())
            snaps[layer + 1] = hs.view(torch.int16).cpu().numpy().view(np.uint16)
    torch.cuda.synchronize()

    def f32(u16):
        return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32)

    wf = {p: f32(S.w_host[p]) for p in shp}
    gam = np.ones(hid, np.float32)
    gam[outl] = 20.0
    x_host = WL.activations(M, hid, "llama8b_chain", "x", outliers=outl)
    href = f32(x_host[rows]).astype(np.float32)

    def rmsnorm(a):
        return a / np.sqrt(np.mean(a * a, axis=1, keepdims=True) + np.float32(1e-5)) * gam

    drift = {}
    for layer in range(LAYERS):
        qkv = rmsnorm(href) @ wf["qkv"].T
        href = href + qkv[:, :hid] @ wf["o"].T
        gu = rmsnorm(href) @ wf["gate_up"].T
        g, u = gu[:, :inter], gu[:, inter:]
        href = href + ((g / (np.float32(1) + np.exp(-g))) * u) @ wf["down"].T
        if layer + 1 in snaps:
            d = f32(snaps[layer + 1]).astype(np.float64) - href.astype(np.float64)
            drift[str(layer + 1)] = round(float(np.linalg.norm(d) / np.linalg.norm(href)), 5)
    out["drift_vs_fp32"] = {
        "rel_err_after_layers": drift, "rows": len(rows),
        "reference": "fp32 forward of the unquantized block stack (bf16 weights, RMSNorm with "
                     "gamma), sampled token rows; error = ||h_w8a8 - h_fp32|| / ||h_fp32||"}
    log(f"[bench] chain drift vs fp32 ({time.time() - t0:.1f}s): {drift}")
    return out


def run_70b(torch, W, WL, args):
    """Llama-3-70B per-layer projections (qkv 8192->10240, o 8192->8192,
    gate_up 8192->57344, down 28672->8192): w8a8_linear at 32 tokens (GB/s of
    algorithmic bytes) and at 2048 tokens (int8 TOPS). Each shape rotates over
    max(2, ceil(1 GiB / weight bytes)) distinct weight buffers so every call
    streams its weights from HBM."""
    import math as _m
    wl = WL.WORKLOADS["llama70b"]
    m_dec, m_pf = wl.ms
    per_dec, per_pf = {}, {}
    dec_bytes = dec_us = pf_ops = pf_us = 0.0
    t0 = time.time()
    for proj, N, K in wl.shapes:
        outl = WL.outlier_channels(K, wl.outlier_frac, wl.name)
        xcal = WL.activations(m_pf, K, wl.name, proj, 0, outliers=outl, mult=wl.outlier_mult)
        w = WL.weights(N, K, wl.w_std, wl.name, proj, 0)
        xcal_d = _bf16_dev(torch, xcal)
        w_d = _bf16_dev(torch, w)
        del w
        s = W.w8a8_smoothing_factors(W.w8a8_channel_absmax(xcal_d), W.w8a8_channel_absmax(w_d))
        wq, sw = W.w8a8_quantize_weight(w_d, s)
        del w_d
        copies = max(2, _m.ceil(2**30 / (N * K)))
        wqs = [wq] + [wq.clone() for _ in range(copies - 1)]
        for M in (m_dec, m_pf):
            x = xcal_d[:M].clone() if M == m_pf else _bf16_dev(torch, WL.activations(
                M, K, wl.name, proj, 0, outliers=outl, mult=wl.outlier_mult))
            y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            ws = torch.empty((W.w8a8_linear_workspace_bytes(M, K),), dtype=torch.uint8, device="cuda")
            g = capture(torch, lambda: [W.w8a8_linear(x, s, wqs[c], sw, y=y, workspace=ws)
                                        for c in range(copies)])
            us = time_graph(torch, g, max(args.steps // 4, 3), 2) / copies * 1e3
            del g
            if M == m_dec:
                b = lin_bytes(M, N, K)
                per_dec[proj] = {"us": round(us, 2), "GBps": round(b / (us * 1e-6) / 1e9, 1)}
                dec_bytes += b
                dec_us += us
            else:
                ops = 2.0 * M * N * K
                per_pf[proj] = {"us": round(us, 2), "TOPS": round(ops / (us * 1e-6) / 1e12, 1)}
                pf_ops += ops
                pf_us += us
        del wqs, xcal_d
        torch.cuda.empty_cache()
    out = {"decode": {"M": m_dec, "value": round(dec_bytes / (dec_us * 1e-6) / 1e9, 1),
                      "unit": "GB/s", "per_shape": per_dec},
           "prefill": {"M": m_pf, "value": round(pf_ops / (pf_us * 1e-6) / 1e12, 1),
                       "unit": "TOPS", "per_shape": per_pf},
           "config": {"workload": "llama70b: Llama-3-70B qkv/o/gate_up/down, one layer, "
                                  "w8a8_linear per projection, weights rotated over >= 1 GiB"}}
    log(f"[bench] llama70b ({time.time() - t0:.1f}s): decode M={m_dec} "
        f"{out['decode']['value']:.0f} GB/s {per_dec}; prefill M={m_pf} "
        f"{out['prefill']['value']:.0f} TOPS {per_pf}")
    return out


def _bf16_dev(torch, u16):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).cuda().view(torch.bfloat16)


def _cpu_host():
    """BLAS threads the oracle's matmul uses, the CPU model and the CPUs in
    this process's affinity mask."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                         model)
    except OSError:
        pass
    return {"cores": int(threads), "kind": "oracle", "cpu_model": model,
            "cpus_in_affinity": len(os.sched_getaffinity(0))}


def _time_passes(one_pass, min_seconds):
    """Whole passes of one_pass() (which returns (seconds, work)) until the
    oracle time reaches min_seconds. Returns (seconds, work, passes)."""
    t = work = 0.0
    passes = 0
    while t < min_seconds:
        dt, dw = one_pass()
        t += dt
        work += dw
        passes += 1
    return t, work, passes


def cpu_baselines(W, WL, sample_ms, min_seconds=10.0):
    """The oracle, timed on this host beside every GPU line, each on a bounded
    sample of the line's workload (weight preparation untimed):
      decode:  whole passes over one layer's four projections at M in sample_ms;
      prefill: the first 512 of the 4096 token rows of each projection (rows
               are independent, so the rate stands for the whole linear);
      chain:   4 token rows through 2 layers of the block chain;
      llama70b: 1024 output channels of each 70B projection (weights drawn at
               that size), at 32 tokens and at 256 of the 2048 token rows."""
    import numpy as np
    from oracle import w8a8_oracle as O
    host = _cpu_host()
    wl = WL.WORKLOADS["llama8b_decode"]
    prepared = []
    for proj, N, K in wl.shapes:
        outl = WL.outlier_channels(K, wl.outlier_frac, wl.name)
        xcal = WL.activations(PREFILL_M, K, wl.name, proj, 0, outliers=outl, mult=wl.outlier_mult)
        w = WL.weights(N, K, wl.w_std, wl.name, proj, 0)
        aw = np.zeros(K, np.float32)
        for r0 in range(0, N, 4096):
            aw = np.maximum(aw, O.weight_channel_absmax(w[r0:r0 + 4096]))
        s = O.smoothing_factors(O.act_channel_absmax(xcal), aw)
        parts = [O.prepare_weight(w[r0:r0 + 4096], s) for r0 in range(0, N, 4096)]
        wq = np.concatenate([p[0] for p in parts])
        sw = np.concatenate([p[1] for p in parts])
        xs = {M: WL.activations(M, K, wl.name, proj, 0, outliers=outl, mult=wl.outlier_mult)
              for M in sample_ms}
        xs["prefill"] = np.ascontiguousarray(xcal[:512])
        prepared.append((proj, N, K, s, wq, sw, xs))

    def timed_linear(x, s, wq, sw):
        t0 = time.perf_counter()
        O.linear(x, s, wq, sw)
        return time.perf_counter() - t0

    # decode: GB/s of algorithmic bytes
    def decode_pass():
        t = b = 0.0
        for M in sample_ms:
            for proj, N, K, s, wq, sw, xs in prepared:
                t += timed_linear(xs[M], s, wq, sw)
                b += lin_bytes(M, N, K)
        return t, b
    t, nbytes, passes = _time_passes(decode_pass, min_seconds)
    decode = {"value": round(nbytes / t / 1e9, 3), "unit": "GB/s", **host,
              "sample": f"{passes} pass(es) over one layer (qkv, o, gate_up, down) of the decode "
                        f"workload at M in {list(sample_ms)}: {passes * len(sample_ms) * 4} oracle "
                        f"linears, {nbytes / 1e9:.2f} GB algorithmic, {t:.1f} s of oracle time; "
                        f"weight prep untimed"}

    # prefill: TOPS on a row sample of the M = 4096 activations
    def prefill_pass():
        t = ops = 0.0
        for proj, N, K, s, wq, sw, xs in prepared:
            x = xs["prefill"]
            t += timed_linear(x, s, wq, sw)
            ops += 2.0 * x.shape[0] * N * K
        return t, ops
    t, ops, passes = _time_passes(prefill_pass, 0.8 * min_seconds)
    prefill = {"value": round(ops / t / 1e12, 4), "unit": "TOPS", **host,
               "sample": f"{passes} pass(es) of the oracle linear on the first 512 of the 4096 "
                         f"token rows of each projection (qkv, o, gate_up, down; whole weights): "
                         f"{ops / 1e12:.2f} T int8 ops in {t:.1f} s; weight prep untimed"}

    # chain: TOPS of the oracle's block chain on a few token rows
    byp = {p[0]: p for p in prepared}
    hid = 4096
    outl = WL.outlier_channels(hid, 0.01, "llama8b_chain")
    gamma = np.ones(hid, np.float32)
    gamma[outl] = 20.0
    layer = {"g_attn": O.fold_gamma(gamma, byp["qkv"][3]),
             "g_mlp": O.fold_gamma(gamma, byp["gate_up"][3]),
             "s_o": byp["o"][3], "s_down": byp["down"][3],
             **{p: (byp[p][4], byp[p][5]) for p in byp}}
    rows = 4
    x_chain = np.ascontiguousarray(
        WL.activations(CHAIN_M, hid, "llama8b_chain", "x", outliers=outl)[:rows])
    chain_ops = 2.0 * rows * sum(N * K for _, N, K in wl.shapes) * 2

    def chain_pass():
        t0 = time.perf_counter()
        O.chain_forward(x_chain, [layer, layer])
        return time.perf_counter() - t0, chain_ops
    t, ops, passes = _time_passes(chain_pass, 0.6 * min_seconds)
    chain = {"value": round(ops / t / 1e12, 5), "unit": "TOPS", **host,
             "sample": f"{passes} pass(es) of the oracle block chain on {rows} token rows "
                       f"through 2 layers (8 linears, norms, SiLU producer): {ops / 1e9:.1f} G "
                       f"int8 ops in {t:.1f} s; weight prep untimed"}

    # Llama-3-70B: 1024 output channels per projection
    w70 = WL.WORKLOADS["llama70b"]
    m_dec, m_pf = w70.ms
    nsamp, psamp = 1024, 256
    prep70 = []
    for proj, _, K in w70.shapes:
        outl = WL.outlier_channels(K, w70.outlier_frac, w70.name)
        x = WL.activations(m_pf, K, w70.name, proj, 0, outliers=outl, mult=w70.outlier_mult)
        w = WL.weights(nsamp, K, w70.w_std, w70.name, proj, "cpu-sample")
        s = O.smoothing_factors(O.act_channel_absmax(x), O.weight_channel_absmax(w))
        wq, sw = O.prepare_weight(w, s)
        prep70.append((K, s, wq, sw, np.ascontiguousarray(x[:m_dec]),
                       np.ascontiguousarray(x[:psamp])))

    def b70_pass():
        td = tp = b = ops = 0.0
        for K, s, wq, sw, xd, xp in prep70:
            td += timed_linear(xd, s, wq, sw)
            b += lin_bytes(m_dec, nsamp, K)
            tp += timed_linear(xp, s, wq, sw)
            ops += 2.0 * psamp * nsamp * K
        return td + tp, (td, b, tp, ops)
    acc = [0.0, 0.0, 0.0, 0.0]
    spent = 0.0
    passes = 0
    while spent < 0.6 * min_seconds:
        dt, parts = b70_pass()
        spent += dt
        acc = [a + p for a, p in zip(acc, parts)]
        passes += 1
    b70 = {"decode": {"value": round(acc[1] / acc[0] / 1e9, 3), "unit": "GB/s"},
           "prefill": {"value": round(acc[3] / acc[2] / 1e12, 4), "unit": "TOPS"}, **host,
           "sample": f"{passes} pass(es) over the four Llama-3-70B projections with {nsamp} "
                     f"output channels each (weights drawn at that size), at M = {m_dec} and on "
                     f"{psamp} of the {m_pf} token rows: {spent:.1f} s of oracle time; weight "
                     f"prep untimed"}
    return decode, prefill, chain, b70


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this layer is measured on one GPU; --gpus {args.gpus} is not "
              "supported (sharding across GPUs is a design note, not a code path)",
              file=sys.stderr)
        sys.exit(2)
    root = os.path.dirname(os.path.abspath(__file__))
    sys.path.insert(0, root)
    import torch
    import int8_w8a8_quantized_token_amd as W
    from int8_w8a8_quantized_token_amd import workloads as WL
    W.lib()                                           # fail loudly if not built
    torch.cuda.set_device(0)

    ms_all = DECODE_MS + (() if args.no_prefill else (PREFILL_M,))
    S = Setup(torch, W, WL, ms_all)
    if args.counters:
        counters(torch, S, ms_all)
        return

    # decode (headline)
    clocks_before = gpu_clocks()
    d_step, d_gemm, d_launch, d_per, d_stats = run_phase(torch, S, DECODE_MS, args.steps, args.warmup,
                                                args.detail)
    d_bytes = sum(lin_bytes(M, N, K) for M in DECODE_MS for _, N, K in S.shapes) * LAYERS
    d_gbytes = sum(gemm_bytes(M, N, K) for M in DECODE_MS for _, N, K in S.shapes) * LAYERS
    value = d_bytes / (d_step * 1e-3) / 1e9
    gemm_gbps = d_gbytes / (d_gemm * 1e-3) / 1e9
    log(f"[bench] decode step {d_step:.3f} ms -> {value:.0f} GB/s; GEMMs alone "
        f"{d_gemm:.3f} ms ({d_gemm / d_launch * 1e3:.2f} us/launch) -> {gemm_gbps:.0f} GB/s")

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(d_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": "llama8b_decode: Llama-3.1-8B qkv/o/gate_up/down, 32 layers, "
                               "M in {1,4,16,64}, w8a8_linear per projection",
                   "layers": LAYERS, "ms": list(DECODE_MS),
                   "shapes_NK": {p: [n, k] for p, n, k in S.shapes}},
        "roofline": {"bound": "hbm", "achieved": round(gemm_gbps, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gemm_gbps / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(root, "decode"),
                     "algorithmic_bytes_per_launch": round(d_gbytes / LAYERS / len(DECODE_MS) /
                                                           len(S.shapes)),
                     "kernel": "gemm_mid_kernel", "launches_per_step": d_launch,
                     "avg_launch_us": round(d_gemm / d_launch * 1e3, 3)},
        "step_stats": d_stats,
        "dispatch_floor_us": dispatch_floor_us(torch),
    }
    if d_per:
        out["per_shape_decode"] = d_per

    # the same step split by token count: the four projections x 32 layers
    # at one M, whole linear and GEMM alone, against the HBM peak
    by_m = {}
    for M in DECODE_MS:
        m_step, m_gemm, _, _, _ = run_phase(torch, S, (M,), args.steps, args.warmup, False)
        lb = sum(lin_bytes(M, N, K) for _, N, K in S.shapes) * LAYERS
        gb = sum(gemm_bytes(M, N, K) for _, N, K in S.shapes) * LAYERS
        lin, gem = lb / (m_step * 1e-3) / 1e9, gb / (m_gemm * 1e-3) / 1e9
        by_m[str(M)] = {"linear_GBps": round(lin, 1), "linear_frac": round(lin / HBM_PEAK_GBS, 4),
                        "gemm_GBps": round(gem, 1), "gemm_frac": round(gem / HBM_PEAK_GBS, 4)}
    out["decode_by_m"] = by_m
    log(f"[bench] decode by token count: {by_m}")

    # the same decode step with the static (calibrated, per-tensor) activation scale
    def static_step():
        for M in DECODE_MS:
            for layer in range(LAYERS):
                for proj, _, _ in S.shapes:
                    S.linear_static(proj, M, layer)
    g_static = capture(torch, static_step)
    s_step = time_graph(torch, g_static, args.steps, args.warmup)
    del g_static
    s_value = d_bytes / (s_step * 1e-3) / 1e9
    log(f"[bench] static-scale decode step {s_step:.3f} ms -> {s_value:.0f} GB/s")
    out["static_decode"] = {
        "value": round(s_value, 1), "unit": "GB/s", "ms_per_step": round(s_step, 4),
        "config": {"workload": "llama8b_decode as above, w8a8_linear_static with one "
                               "entropy-calibrated activation scale per projection"}}

    if not args.no_chain:
        out["chain"] = run_chain(torch, W, WL, S, args)
    if not args.no_70b:
        out["llama70b"] = run_70b(torch, W, WL, args)

    if not args.no_prefill:
        clk = {}
        p_step, p_gemm, p_launch, p_per, p_stats = run_phase(
            torch, S, (PREFILL_M,), max(args.steps // 4, 3), min(args.warmup, 2), args.detail,
            on_gemm_graph=lambda g, t: clk.update(clocks_under_load(torch, g, t)))
        ops = sum(2 * PREFILL_M * N * K for _, N, K in S.shapes) * LAYERS
        tops = ops / (p_step * 1e-3) / 1e12
        gtops = ops / (p_gemm * 1e-3) / 1e12
        log(f"[bench] prefill step {p_step:.3f} ms -> {tops:.0f} TOPS; GEMMs alone "
            f"{p_gemm:.3f} ms -> {gtops:.0f} TOPS")
        out["prefill"] = {
            "value": round(tops, 1), "unit": "TOPS", "ms_per_step": round(p_step, 4),
            "step_stats": p_stats,
            "config": {"workload": "llama8b_prefill: same 32 layers x 4 projections at M=4096",
                       "m": PREFILL_M},
            "roofline": {"bound": "mfma", "achieved": round(gtops, 1), "peak": INT8_PEAK_TOPS,
                         "unit": "TOPS", "frac": round(gtops / INT8_PEAK_TOPS, 4),
                         "traffic": measured_traffic(root, "prefill"),
                         "algorithmic_bytes_per_launch": round(sum(
                             gemm_bytes(PREFILL_M, N, K) for _, N, K in S.shapes) / len(S.shapes)),
                         "kernel": "gemm_prefill128_kernel",
                         "launches_per_step": p_launch,
                         "avg_launch_us": round(p_gemm / p_launch * 1e3, 3)},
        }
        # the same fraction against the peak at the shader clock read while
        # the GEMM graph replays back to back (the data-sheet peak assumes
        # 2.4 GHz; under this load the chip runs slower, power-limited)
        gfx = clk.get("gfx_per_xcd") or []
        if gfx:
            mhz = sum(gfx) / len(gfx)
            peak_clk = INT8_PEAK_TOPS * mhz / 2400.0
            out["prefill"]["roofline"]["at_clock"] = {
                "sclk_mhz": round(mhz, 1), "peak": round(peak_clk, 1),
                "frac": round(gtops / peak_clk, 4),
                "read": f"amd-smi during {clk['replays']} back-to-back replays of the GEMM graph"}
        else:
            out["prefill"]["roofline"]["at_clock"] = {"error": clk.get("error", "no reading")}
        if p_per:
            out["per_shape_prefill"] = p_per

    out["clocks_mhz"] = {"before": clocks_before, "after": gpu_clocks()}

    if not args.no_cpu_baseline:
        t0 = time.time()
        decode, prefill, chain, b70 = cpu_baselines(W, WL, DECODE_MS)
        out["cpu_baseline"] = decode
        if "prefill" in out:
            out["prefill"]["cpu_baseline"] = prefill
        if "chain" in out:
            out["chain"]["cpu_baseline"] = chain
        if "llama70b" in out:
            out["llama70b"]["cpu_baseline"] = b70
        log(f"[bench] cpu baselines {time.time() - t0:.1f}s: decode {decode}; prefill {prefill}; "
            f"chain {chain}; llama70b {b70}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
