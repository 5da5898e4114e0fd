"""GPU parity of every C-ABI entry point against the CPU oracle, on seeded
inputs at sizes the oracle finishes in seconds: several tiles of each kernel
plus ragged M, N and K tails, crafted edge rows (exact ties, zero rows,
subnormal rows, extremes), strided views and empty calls.

int8 codes, scales and int32 accumulators must be bit-exact; bf16 outputs
within 1 bf16 ulp (relative error <= 2**-8) of the oracle.
"""
import numpy as np
import pytest

import int8_w8a8_quantized_token_amd as W
from int8_w8a8_quantized_token_amd import workloads as WL
from oracle import w8a8_oracle as O
from gpu_util import check_bf16, dev, dev_bf16, host, torch

pytestmark = pytest.mark.gpu

F32 = np.float32


def act(M, K, tag, frac=0.01, mult=20.0):
    return WL.activations(M, K, "parity", tag, frac=frac, mult=mult)


def smooth_for(x_bf16, w_bf16):
    return O.smoothing_factors(O.act_channel_absmax(x_bf16), O.weight_channel_absmax(w_bf16))


def i8(shape, *key):
    return WL.rng("i8", *shape, *key).integers(-128, 128, size=shape, dtype=np.int64).astype(np.int8)


# ---------------------------------------------------------------------------
# quantize_act
# ---------------------------------------------------------------------------

QA_SHAPES = [(1, 16), (2, 48), (3, 64), (15, 4096 + 16), (16, 4096), (17, 2048),
             (63, 512), (64, 14336), (65, 4096), (127, 1040), (255, 256), (4, 40960),
             # many rows (256 or 512 threads per row), ragged M and channel
             # tails, and K beyond the register-resident limit
             (513, 4096), (1024, 4096 + 16), (1100, 14336), (2049, 2048), (8200, 64),
             (600, 40960),
             # the two remaining (threads, vectors per thread) instances:
             # 1024 threads x 4 vectors and 512 threads x 8 vectors
             (100, 20000), (700, 24000),
             # few rows longer than 1024 threads hold in registers (read twice),
             # up to the largest K the library accepts
             (5, 65536 + 16), (1, 131072)]


@pytest.mark.parametrize("M,K", QA_SHAPES, ids=[f"M{m}_K{k}" for m, k in QA_SHAPES])
@pytest.mark.parametrize("use_smooth", [False, True], ids=["plain", "smooth"])
def test_quantize_act_bit_exact(M, K, use_smooth):
    x = act(M, K, "qa")
    smooth = None
    if use_smooth:
        smooth = np.exp(WL.rng("smooth", K).uniform(-3, 3, K)).astype(F32)
    xq_ref, s_ref = O.quantize_act(x, smooth)
    xq, s = W.w8a8_quantize_act(dev_bf16(x), dev(smooth) if smooth is not None else None)
    torch().cuda.synchronize()
    np.testing.assert_array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(host(xq), xq_ref)


def crafted_rows(K):
    """Rows that exercise ties, zeros, subnormals and extremes (K >= 16).
    Every value is exactly representable in bf16."""
    rows = []
    base = np.zeros(K, F32)
    # exact ties: row max 127 * 2**k gives S = 2**k, (n + 1/2) * 2**k are ties
    for k in (-20, -3, 0, 5):
        r = base.copy()
        vals = np.array([127, 62.5, -62.5, 0.5, -0.5, 1.5, -1.5, 126.5, -126.5, 2.5, -2.5,
                         0.25, 63.5, -63.5, 100.5, -0.75], F32)
        r[:16] = vals * F32(2.0 ** k)
        rows.append(r)
    rows.append(base.copy())                                   # all-zero row
    r = base.copy(); r[3] = F32(-2.0 ** -130); rows.append(r)  # one subnormal value
    r = np.full(K, F32(2.0 ** -125)); r[::7] = F32(-1.5 * 2.0 ** -125); rows.append(r)
    r = np.full(K, F32(2.0 ** 100)); r[1] = F32(-1.5 * 2.0 ** 127); rows.append(r)
    rows.append(O.bf16_to_f32(O.round_to_bf16(np.linspace(-1, 1, K))))   # ramp
    return np.stack(rows).astype(F32)


@pytest.mark.parametrize("K", [16, 64, 4096])
def test_quantize_act_crafted_rows(K):
    x32 = crafted_rows(K)
    x = O.round_to_bf16(x32)
    assert np.array_equal(O.bf16_to_f32(x), x32), "crafted values must be bf16-exact"
    xq_ref, s_ref = O.quantize_act(x)
    xq, s = W.w8a8_quantize_act(dev_bf16(x))
    torch().cuda.synchronize()
    np.testing.assert_array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(host(xq), xq_ref)
    # the tie rows really hit the tie rule
    assert host(xq)[2, :16].tolist()[:11] == [127, 63, -63, 1, -1, 2, -2, 127, -127, 3, -3]


@pytest.mark.parametrize("K", [64, 4096])
def test_quantize_act_crafted_rows_many(K):
    # the same edge rows, 60 times over: past 512 rows the many-row kernel runs
    x32 = np.tile(crafted_rows(K), (60, 1))
    x = O.round_to_bf16(x32)
    xq_ref, s_ref = O.quantize_act(x)
    xq, s = W.w8a8_quantize_act(dev_bf16(x))
    torch().cuda.synchronize()
    np.testing.assert_array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(host(xq), xq_ref)


@pytest.mark.parametrize("M", [16, 600])
def test_quantize_act_smoothing_edges(M):
    # smoothing factors at and beyond 2^-20 and 2^20 (up to 2^-30 and 2^30),
    # activations below 2^-80 and exact zeros, and a row of tiny values only:
    # quotients far from 1 through the smoothing division and the code step
    K = 1024
    r = WL.rng("smooth-edges", M, K)
    smooth = np.exp(r.uniform(-3, 3, K)).astype(F32)
    smooth[::17] = F32(2.0 ** -30)
    smooth[5::17] = F32(2.0 ** 30)
    smooth[9::17] = F32(2.0 ** -20)
    smooth[11::17] = F32(2.0 ** 20)
    x32 = O.bf16_to_f32(act(M, K, "smooth-edges"))
    x32[:, ::13] = F32(2.0 ** -100)
    x32[:, 3::13] = F32(-(2.0 ** -81))
    x32[:, 7::13] = F32(0.0)
    x32[1, :] = F32(2.0 ** -90)                  # a row of tiny values only
    x = O.round_to_bf16(x32)
    xq_ref, s_ref = O.quantize_act(x, smooth)
    xq, s = W.w8a8_quantize_act(dev_bf16(x), dev(smooth))
    torch().cuda.synchronize()
    np.testing.assert_array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(host(xq), xq_ref)


def test_quantize_act_strided_and_empty():
    M, K, ld = 33, 4096, 6144
    big = act(M, ld, "strided")
    x = dev_bf16(big)[:, :K]                   # a column slice: ldx = 6144
    xq_full = torch().zeros((M, K + 64), dtype=torch().int8, device="cuda")
    xq = xq_full[:, :K]
    _, s = W.w8a8_quantize_act(x, None, xq=xq)
    torch().cuda.synchronize()
    xq_ref, s_ref = O.quantize_act(big[:, :K])
    np.testing.assert_array_equal(host(xq), xq_ref)
    np.testing.assert_array_equal(host(s), s_ref)
    assert np.all(host(xq_full)[:, K:] == 0), "wrote past the row"
    e = torch().empty((0, K), dtype=torch().bfloat16, device="cuda")
    W.w8a8_quantize_act(e)
    torch().cuda.synchronize()


# ---------------------------------------------------------------------------
# GEMM: int32 accumulators (bit-exact) and bf16 epilogue (<= 1 ulp)
# ---------------------------------------------------------------------------

GEMM_SHAPES = [
    # skinny path (M <= 64)
    (1, 1, 16), (1, 16, 64), (4, 17, 48), (16, 100, 80), (17, 256, 192), (33, 300, 1040),
    (48, 64, 4096), (64, 4096, 4096), (5, 6144, 14336 + 16),
    # skinny classes that load the epilogue scales after the weight stream
    (12, 6000, 1024), (20, 9000, 256), (64, 8320, 512),
    # LDS-staged decode path (M <= 64, K % 128 == 0): every token class x
    # (wide, mid, deep, plain N), N ragged against 16/32/64-channel
    # workgroups, one K stage (fewer stages than waves) and odd stage counts
    (1, 16400, 128), (3, 5000, 8320), (7, 4100, 256), (16, 300, 384), (17, 16400, 1024),
    (24, 4500, 128), (31, 1000, 8320), (33, 16390, 512), (40, 6000, 256), (47, 200, 128),
    (49, 17000, 384), (55, 4200, 1152), (63, 100, 8320), (64, 16, 128),
    (9, 2000, 8320), (2, 4096, 14336),
    # the same kernel in M tiles of 64 rows (ragged last tile), up to the
    # limits of its range, and the prefill kernel just past them (at
    # M < 512 for wide N)
    (65, 300, 256), (128, 16400, 128), (129, 16400, 256), (200, 5000, 512), (300, 17000, 128),
    (700, 300, 1152), (1024, 200, 512), (1025, 200, 512), (1536, 60, 8320), (1537, 60, 8320),
    # tiled path (64 < M < 512, K % 128 != 0; (128, 256, 4096) and
    # (512, 512, 2048) take the M-tiled mid kernel)
    (65, 1, 16), (65, 128, 64), (100, 129, 112), (128, 256, 4096), (130, 300, 1040),
    (257, 515, 208), (512, 512, 2048), (1000, 384, 4096 + 48),
    # 64-byte-stage prefill path (M >= 512, K % 128 != 0): 0..3 full stages,
    # K tails, ragged M/N
    (512, 256, 48), (512, 256, 64), (513, 257, 128), (600, 300, 192), (700, 520, 208),
    (1024, 768, 14336 + 16), (2048, 1000, 1024),
    # full-line prefill path (K % 128 == 0, past the mid kernel's range): 1, 2
    # and 3 stages, several tiles, ragged M/N ((512, 512, 128), (777, 300, 256)
    # and (1024, 1024, 4096) take the mid kernel)
    (512, 512, 128), (777, 300, 256), (1100, 600, 384), (1024, 1024, 4096),
    (1030, 520, 128), (1040, 260, 384),
    # enough tiles that 256-row tiles win over 192-row ones
    (2048, 8192, 256), (2047, 8190, 256),
]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES, ids=[f"M{m}_N{n}_K{k}" for m, n, k in GEMM_SHAPES])
def test_gemm_i32_bit_exact(M, N, K):
    a, b = i8((M, K), "a"), i8((N, K), "b")
    acc = W.w8a8_gemm_i32(dev(a), dev(b))
    torch().cuda.synchronize()
    np.testing.assert_array_equal(host(acc), O.gemm_i32(a, b))


def test_gemm_i32_closed_form_extremes():
    # |acc| at its largest: all 127 x all -127 over K = 28672, both paths
    K = 28672
    for M in (16, 96):
        a = np.full((M, K), 127, np.int8)
        b = np.full((40, K), -127, np.int8)
        b[::2] = 127
        acc = host(W.w8a8_gemm_i32(dev(a), dev(b)))
        torch().cuda.synchronize()
        want = np.where(np.arange(40) % 2 == 0, 16129 * K, -16129 * K)
        assert np.all(acc == want[None, :])


@pytest.mark.parametrize("K", [131072, 131072 - 16], ids=["K131072", "K131056"])
def test_gemm_i32_extremes_at_max_k(K):
    # The largest K the library accepts keeps 127 * 127 * K inside int32;
    # every token count class (decode, M-tiled or tiled, prefill) at that K.
    for M in (1, 96, 1600):
        a = np.full((M, K), 127, np.int8)
        b = np.full((40, K), -127, np.int8)
        b[::2] = 127
        acc = host(W.w8a8_gemm_i32(dev(a), dev(b)))
        torch().cuda.synchronize()
        want = np.where(np.arange(40) % 2 == 0, 16129 * K, -16129 * K)
        assert want.max() < 2**31
        assert np.all(acc == want[None, :]), (M, K)


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES, ids=[f"M{m}_N{n}_K{k}" for m, n, k in GEMM_SHAPES])
def test_gemm_bf16_epilogue(M, N, K):
    a, b = i8((M, K), "a"), i8((N, K), "b")
    r = WL.rng("scales", M, N, K)
    s_tok = np.exp(r.uniform(-12, -2, M)).astype(F32)
    s_chan = np.exp(r.uniform(-10, -3, N)).astype(F32)
    s_tok[0] = 0.0                              # a zero token scale
    y = W.w8a8_gemm(dev(a), dev(s_tok), dev(b), dev(s_chan))
    torch().cuda.synchronize()
    y64, y_ref = O.dequant_epilogue(O.gemm_i32(a, b), s_tok, s_chan)
    check_bf16(host(y), y64, y_ref)


# The full-line prefill kernel picks one of three tiles (256 x 256, 192
# weight rows x 256 tokens, 256 weight rows x 192 tokens) by rounds x tile
# area over the CUs. On a 256-CU device each tile is the one chosen for one
# of these shapes (ragged M and N included); at these sizes the oracle
# recomputes every column of sampled token rows: both edges of the first
# 192- and 256-row tiles and the last, partial tile.
PF_TILE_SHAPES = [
    (4000, 4000, 128),     # 256 x 256
    (4096, 6144, 128),     # 192 x 256 (qkv at M = 4096)
    (3000, 4096, 256),     # 256 x 192 (o and down at M = 3000)
    (2990, 4090, 128),     # 256 x 192, ragged
]


@pytest.mark.parametrize("M,N,K", PF_TILE_SHAPES, ids=[f"M{m}_N{n}_K{k}" for m, n, k in PF_TILE_SHAPES])
def test_gemm_prefill_tiles_sampled_rows(M, N, K):
    a, b = i8((M, K), "pft_a"), i8((N, K), "pft_b")
    r = WL.rng("pft_scales", M, N, K)
    s_tok = np.exp(r.uniform(-12, -2, M)).astype(F32)
    s_chan = np.exp(r.uniform(-10, -3, N)).astype(F32)
    print(f"\n[prefill tiles] M={M} N={N} K={K}", flush=True)
    acc = W.w8a8_gemm_i32(dev(a), dev(b))
    y = W.w8a8_gemm(dev(a), dev(s_tok), dev(b), dev(s_chan))
    torch().cuda.synchronize()
    edges = [0, 1, 191, 192, 255, 256, 383, 384, M - 2, M - 1]
    rows = np.unique(np.concatenate([edges, (M // 192) * 192 + np.arange(2), (M // 256) * 256 + np.arange(2),
                                     r.choice(M, size=12, replace=False)]))
    rows = rows[rows < M]
    acc_ref = O.gemm_i32(a[rows], b)
    np.testing.assert_array_equal(host(acc)[rows], acc_ref)
    y64, y_ref = O.dequant_epilogue(acc_ref, s_tok[rows], s_chan)
    check_bf16(host(y)[rows], y64, y_ref)


def test_gemm_strided_output():
    M, N, K, ldy = 40, 200, 256, 264
    a, b = i8((M, K), "sa"), i8((N, K), "sb")
    s_tok = np.full(M, 1e-3, F32)
    s_chan = np.full(N, 2e-3, F32)
    yfull = torch().zeros((M, ldy), dtype=torch().bfloat16, device="cuda")
    W.w8a8_gemm(dev(a), dev(s_tok), dev(b), dev(s_chan), y=yfull[:, :N])
    torch().cuda.synchronize()
    y64, y_ref = O.dequant_epilogue(O.gemm_i32(a, b), s_tok, s_chan)
    yh = host(yfull)
    check_bf16(yh[:, :N], y64, y_ref)
    assert np.all(yh[:, N:] == 0), "wrote past the row"


# Row strides past K for both operands and an output stride that rules out
# vector stores, on every kernel route: LDS-staged decode (one and several M
# tiles; K = 3968 with weight rows 4096 bytes apart, where the K walk is
# rotated, over 31 stages), register-staged skinny (K % 128 != 0), tiled,
# and both prefill kernels.
STRIDED = [(1, 300, 512, 4096), (33, 200, 3968, 4096), (200, 130, 256, 384), (5, 70, 1040, 1104),
           (100, 90, 208, 272), (1100, 140, 256, 320), (600, 60, 192, 256)]


@pytest.mark.parametrize("M,N,K,ldw", STRIDED, ids=[f"M{m}_N{n}_K{k}_ldw{l}" for m, n, k, l in STRIDED])
def test_gemm_strided_operands(M, N, K, ldw):
    ldq, ldy = K + 64, N + 3
    a, b = i8((M, K), "st-a"), i8((N, K), "st-b")
    r = WL.rng("st-scales", M, N, K)
    s_tok = np.exp(r.uniform(-12, -2, M)).astype(F32)
    s_chan = np.exp(r.uniform(-10, -3, N)).astype(F32)
    t = torch()
    aq = t.zeros((M, ldq), dtype=t.int8, device="cuda")
    aq[:, :K] = dev(a)
    bw = t.zeros((N, ldw), dtype=t.int8, device="cuda")
    bw[:, :K] = dev(b)
    yfull = t.zeros((M, ldy), dtype=t.bfloat16, device="cuda")
    W.w8a8_gemm(aq[:, :K], dev(s_tok), bw[:, :K], dev(s_chan), y=yfull[:, :N])
    acc = W.w8a8_gemm_i32(aq[:, :K], bw[:, :K])
    t.cuda.synchronize()
    acc_ref = O.gemm_i32(a, b)
    np.testing.assert_array_equal(host(acc), acc_ref)
    y64, y_ref = O.dequant_epilogue(acc_ref, s_tok, s_chan)
    yh = host(yfull)
    check_bf16(yh[:, :N], y64, y_ref)
    assert np.all(yh[:, N:] == 0), "wrote past the row"


@pytest.mark.parametrize("M", [1, 2])
def test_linear_one_launch_strided(M):
    # the one-launch linear on a column slice of a wider input, into an
    # output whose row stride rules out vector stores
    K, N, ldx, ldy = 1024, 300, 1536, 303
    big = act(M, ldx, "fused-slice")
    w = WL.weights(N, K, 0.02, "fused-slice")
    xs = big[:, :K]
    s_ref = smooth_for(xs, w)
    wq_ref, sw_ref = O.prepare_weight(w, s_ref)
    ref = O.linear(xs, s_ref, wq_ref, sw_ref)
    t = torch()
    xd = dev_bf16(big)[:, :K]
    wd = dev_bf16(w)
    s = W.w8a8_smoothing_factors(W.w8a8_channel_absmax(xd), W.w8a8_channel_absmax(wd))
    wq, sw = W.w8a8_quantize_weight(wd, s)
    yfull = t.zeros((M, ldy), dtype=t.bfloat16, device="cuda")
    W.w8a8_linear(xd, s, wq, sw, y=yfull[:, :N])
    t.cuda.synchronize()
    yh = host(yfull)
    check_bf16(yh[:, :N], ref["y64"], ref["y"])
    assert np.all(yh[:, N:] == 0), "wrote past the row"


# ---------------------------------------------------------------------------
# offline prep kernels (bit-exact)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(3, 16), (100, 4096), (4096, 4096), (17, 14336)])
def test_prep_bit_exact(N, K):
    M = 37
    x = act(M, K, "prep")
    w = WL.weights(N, K, 0.02, "prep")
    ax = W.w8a8_channel_absmax(dev_bf16(x[:20]))
    W.w8a8_channel_absmax(dev_bf16(x[20:]), absmax=ax)       # accumulate a second batch
    aw = W.w8a8_channel_absmax(dev_bf16(w))
    s = W.w8a8_smoothing_factors(ax, aw)
    wq, sw = W.w8a8_quantize_weight(dev_bf16(w), s)
    wq0, sw0 = W.w8a8_quantize_weight(dev_bf16(w))
    torch().cuda.synchronize()
    ax_ref, aw_ref = O.act_channel_absmax(x), O.weight_channel_absmax(w)
    np.testing.assert_array_equal(host(ax), ax_ref)
    np.testing.assert_array_equal(host(aw), aw_ref)
    s_ref = O.smoothing_factors(ax_ref, aw_ref)
    np.testing.assert_array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    wq_ref, sw_ref = O.prepare_weight(w, s_ref)
    np.testing.assert_array_equal(host(sw).view(np.uint32), sw_ref.view(np.uint32))
    np.testing.assert_array_equal(host(wq), wq_ref)
    wq0_ref, sw0_ref = O.quantize_weight(w)
    np.testing.assert_array_equal(host(sw0), sw0_ref)
    np.testing.assert_array_equal(host(wq0), wq0_ref)


def test_smoothing_factor_edge_values():
    ax = np.array([0, 4, 1, 0, 3.5e38, 1e-38, 7], F32)
    aw = np.array([1, 1, 0, 0, 1e-3, 1e3, 7], F32)
    s = host(W.w8a8_smoothing_factors(dev(ax), dev(aw)))
    torch().cuda.synchronize()
    np.testing.assert_array_equal(s.view(np.uint32), O.smoothing_factors(ax, aw).view(np.uint32))


# ---------------------------------------------------------------------------
# whole linear
# ---------------------------------------------------------------------------

LIN_SHAPES = [(1, 64, 4096), (16, 4096, 4096), (17, 300, 1040), (64, 1024, 14336),
              (65, 512, 2048), (300, 700, 4096),
              (2, 64, 131072)]          # the largest K the library accepts


@pytest.mark.parametrize("M,N,K", LIN_SHAPES, ids=[f"M{m}_N{n}_K{k}" for m, n, k in LIN_SHAPES])
def test_linear_against_oracle(M, N, K):
    x = act(M, K, "lin")
    w = WL.weights(N, K, 0.02, "lin")
    # each side prepares its own weights from the same bf16 inputs
    s_ref = smooth_for(x, w)
    wq_ref, sw_ref = O.prepare_weight(w, s_ref)
    ref = O.linear(x, s_ref, wq_ref, sw_ref)
    xd, wd = dev_bf16(x), dev_bf16(w)
    s = W.w8a8_smoothing_factors(W.w8a8_channel_absmax(xd), W.w8a8_channel_absmax(wd))
    wq, sw = W.w8a8_quantize_weight(wd, s)
    y = W.w8a8_linear(xd, s, wq, sw)
    xq, st = W.w8a8_quantize_act(xd, s)
    acc = W.w8a8_gemm_i32(xq, wq)
    torch().cuda.synchronize()
    np.testing.assert_array_equal(host(xq), ref["xq"])
    np.testing.assert_array_equal(host(st), ref["s_tok"])
    np.testing.assert_array_equal(host(acc), ref["acc"])
    check_bf16(host(y), ref["y64"], ref["y"])


# The one-launch linear (M <= 2, N < 16384, K % 128 == 0, K <= 4096): both
# entry points against the oracle, with and without smoothing, a zero row,
# one K stage, N ragged against 16- and 32-channel workgroups, and the
# shapes just outside its range (N = 16384, K = 4224: quantize + GEMM).
FUSED_SHAPES = [(1, 1, 128), (1, 100, 4096), (1, 4096, 4096), (1, 4100, 256), (1, 16383, 1024),
                (2, 17, 128), (2, 6144, 4096), (2, 4096, 384), (1, 16384, 4096), (2, 300, 4224)]


@pytest.mark.parametrize("M,N,K", FUSED_SHAPES, ids=[f"M{m}_N{n}_K{k}" for m, n, k in FUSED_SHAPES])
@pytest.mark.parametrize("use_smooth", [False, True], ids=["plain", "smooth"])
def test_linear_one_launch_against_oracle(M, N, K, use_smooth):
    x = act(M, K, "fused")
    if M == 2:
        x[1] = 0                                   # zero row: S = 0, codes 0, y = 0
    wq = i8((N, K), "fused-w")
    sw = (WL.rng("fused-sw", N, K).uniform(0.5, 2.0, N) * 1e-3).astype(F32)
    smooth = np.exp(WL.rng("fused-s", K).uniform(-2, 2, K)).astype(F32) if use_smooth else None
    ref = O.linear(x, smooth, wq, sw)
    S = F32(0.04)
    ref_st = O.linear_static(x, smooth, S, wq, sw)
    xd, wqd, swd = dev_bf16(x), dev(wq), dev(sw)
    sd = dev(smooth) if use_smooth else None
    y = W.w8a8_linear(xd, sd, wqd, swd)
    y_st = W.w8a8_linear_static(xd, sd, dev(np.array([S], F32)), wqd, swd)
    torch().cuda.synchronize()
    check_bf16(host(y), ref["y64"], ref["y"])
    check_bf16(host(y_st), ref_st["y64"], ref_st["y"], "y static")


def test_linear_single_workload_full():
    """The 16-token 4096x4096 layer, every output compared."""
    wl = WL.WORKLOADS["single"]
    (proj, N, K), M = wl.shapes[0], wl.ms[0]
    x, w = WL.layer_inputs(wl, proj, N, K, M)
    s_ref = smooth_for(x, w)
    wq_ref, sw_ref = O.prepare_weight(w, s_ref)
    ref = O.linear(x, s_ref, wq_ref, sw_ref)
    xd, wd = dev_bf16(x), dev_bf16(w)
    s = W.w8a8_smoothing_factors(W.w8a8_channel_absmax(xd), W.w8a8_channel_absmax(wd))
    wq, sw = W.w8a8_quantize_weight(wd, s)
    ws = torch().empty(W.w8a8_linear_workspace_bytes(M, K), dtype=torch().uint8, device="cuda")
    y = W.w8a8_linear(xd, s, wq, sw, workspace=ws)
    torch().cuda.synchronize()
    np.testing.assert_array_equal(host(wq), wq_ref)
    check_bf16(host(y), ref["y64"], ref["y"])


def test_linear_reads_strided_input_slice():
    """o_proj consuming the first 4096 columns of a qkv-shaped [M, 6144] output."""
    M, K, N = 24, 4096, 512
    big = act(M, 6144, "slice")
    w = WL.weights(N, K, 0.02, "slice")
    xs = big[:, :K]
    s_ref = smooth_for(xs, w)
    wq_ref, sw_ref = O.prepare_weight(w, s_ref)
    ref = O.linear(xs, s_ref, wq_ref, sw_ref)
    xd = dev_bf16(big)[:, :K]
    wd = dev_bf16(w)
    s = W.w8a8_smoothing_factors(W.w8a8_channel_absmax(xd), W.w8a8_channel_absmax(wd))
    wq, sw = W.w8a8_quantize_weight(wd, s)
    y = W.w8a8_linear(xd, s, wq, sw)
    torch().cuda.synchronize()
    check_bf16(host(y), ref["y64"], ref["y"])
