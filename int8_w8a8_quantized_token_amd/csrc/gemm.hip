// Int8 x int8 -> int32 GEMM with the dequantizing bf16 epilogue, on gfx950
// matrix cores (MFMA).
//
//   acc[m,n] = sum_k xq[m,k] * wq[n,k]
//   y[m,n]   = bf16_rne((float(acc) * s_tok[m]) * s_chan[n])
//
// The per-token scale s_tok and the per-output-channel scale s_chan both
// factor out of the channel sum, so they are applied once to the exact int32
// accumulator (Red Hat, "Understanding W8A8 INT8 LLM quantization: Half the
// size, better performance, same accuracy", section "Why activation
// quantization is hard, and how SmoothQuant fixes it"). Both operands are
// K-contiguous ("NT"), as the quantizers write them.
//
// Kernels:
//   * mid (M <= 64, decode, K % 128 == 0): the weight matrix is streamed
//     once from HBM; a workgroup owns 16*RW output channels and all token
//     rows, its waves split K, and each wave feeds its own ring of LDS
//     stages by direct global -> LDS loads of whole lines; partial int32
//     tiles are summed in LDS. v_mfma_i32_16x16x64_i8: the weight rows are
//     the A operand, the token rows the B operand.
//   * skinny (M <= 64, other K): the same work split, operands loaded
//     straight into MFMA registers.
//   * prefill (M >= 512) and tiled (64 < M < 512): LDS-staged tiles with
//     v_mfma_i32_32x32x32_i8.
//
// MFMA operand layout: for both operands lane l supplies row (l % R) of its
// matrix and a 16-byte group of K selected by l / R (R = 16 or 32). The
// kernels give A and B the same K grouping, so the K permutation inside the
// instruction cancels (integer addition is exact in any order). Output lane
// l, register e holds D[i][j] with j = l % R and
//   16x16: i = 4*(l/16) + e
//   32x32: i = 8*(e/4) + 4*(l/32) + (e%4).

#include <atomic>

#include "device_common.h"
#include "gemm_common.h"
#include "gemm_dispatch.h"
#include "launchers.h"

namespace w8a8 {

// ---------------------------------------------------------------------------
// Skinny kernel (decode): M <= 16*MT tokens. A workgroup owns 16*RW output
// channels; its NW waves take interleaved 64-byte K chunks, U chunks in
// flight per wave. Each token fragment is reused for RW weight fragments and
// each weight fragment for MT token fragments.
// ---------------------------------------------------------------------------

template <int MT, int RW, int NW, int U>
struct SkinnyCfg {
  static constexpr int kThreads = NW * kWave;
  static constexpr int kRows = 16 * RW;
  static_assert(MT >= 1 && MT <= 4 && RW >= 1 && NW >= 1 && U >= 1, "");
  static_assert(NW * RW * MT <= 64, "LDS reduction buffer at most 64 KB");
};

template <int MT, int RW, int NW, int U, bool I32OUT, bool LATE = false>
__global__ __launch_bounds__(NW * kWave) void gemm_skinny_kernel(
    const int8_t* __restrict__ xq, int64_t ldq, const float* __restrict__ s_tok,
    const int8_t* __restrict__ wq, int64_t ldw, const float* __restrict__ s_chan, int M, int N,
    int K, uint16_t* __restrict__ y, int64_t ldy, int32_t* __restrict__ c, int64_t ldc,
    bool vec_out) {
  __shared__ v4i red[NW][RW * MT][kWave];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16 * RW;

  // Rows past N or M read a valid row; their results land only in outputs
  // that are never stored, since D[i][j] depends on A row i and B row j only.
  const int8_t* wp[RW];
#pragma unroll
  for (int rw = 0; rw < RW; ++rw) wp[rw] = wq + (int64_t)min(n0 + 16 * rw + r, N - 1) * ldw + g * 16;
  const int8_t* xp[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xp[mt] = xq + (int64_t)min(mt * 16 + r, M - 1) * ldq + g * 16;

  // Epilogue scales: fetched before the weight stream (their latency hides
  // under it) or, with LATE, after it (they then cost no registers during the
  // stream and their latency overlaps the LDS reduction).
  float st[MT], sc[RW][4];
  auto load_scales = [&]() {
    if constexpr (!I32OUT) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) st[mt] = s_tok[min(mt * 16 + r, M - 1)];
#pragma unroll
      for (int rw = 0; rw < RW; ++rw) load_chan4(s_chan, n0 + 16 * rw + 4 * g, N, sc[rw]);
    }
  };
  if constexpr (!LATE) load_scales();

  v4i acc[RW][MT];
#pragma unroll
  for (int rw = 0; rw < RW; ++rw)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[rw][mt] = v4i{0, 0, 0, 0};

  const int nfull = K / 64;
  int ch = wave;
  for (; ch + (U - 1) * NW < nfull; ch += U * NW) {
    v4i b[U][RW], a[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int rw = 0; rw < RW; ++rw) b[u][rw] = ldg16(wp[rw] + (int64_t)(ch + u * NW) * 64);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) a[u][mt] = ldg16(xp[mt] + (int64_t)(ch + u * NW) * 64);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int rw = 0; rw < RW; ++rw)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[rw][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b[u][rw], a[u][mt], acc[rw][mt], 0, 0, 0);
  }
  for (; ch < nfull; ch += NW) {
    v4i b[RW], a[MT];
#pragma unroll
    for (int rw = 0; rw < RW; ++rw) b[rw] = ldg16(wp[rw] + (int64_t)ch * 64);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) a[mt] = ldg16(xp[mt] + (int64_t)ch * 64);
#pragma unroll
    for (int rw = 0; rw < RW; ++rw)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[rw][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b[rw], a[mt], acc[rw][mt], 0, 0, 0);
  }
  // K % 64 in {16, 32, 48}: the last chunk is partial; groups past K are zero.
  const int tail = K - nfull * 64;
  if (tail > 0 && wave == nfull % NW) {
    const bool in = g * 16 < tail;
    const v4i zero = {0, 0, 0, 0};
    v4i b[RW], a[MT];
#pragma unroll
    for (int rw = 0; rw < RW; ++rw) b[rw] = in ? ldg16(wp[rw] + (int64_t)nfull * 64) : zero;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) a[mt] = in ? ldg16(xp[mt] + (int64_t)nfull * 64) : zero;
#pragma unroll
    for (int rw = 0; rw < RW; ++rw)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[rw][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b[rw], a[mt], acc[rw][mt], 0, 0, 0);
  }

  if constexpr (LATE) load_scales();
#pragma unroll
  for (int rw = 0; rw < RW; ++rw)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[wave][rw * MT + mt][lane] = acc[rw][mt];
  __syncthreads();

  // Tile t = rw * MT + mt is finished by wave t % NW: sum the NW partial
  // tiles, then lane l holds token m = 16 mt + l % 16 and the 4 output
  // channels 16 rw + 4 (l / 16) + e.
#pragma unroll
  for (int rw = 0; rw < RW; ++rw)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if ((rw * MT + mt) % NW != wave) continue;
      v4i sum = red[0][rw * MT + mt][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) sum += red[w][rw * MT + mt][lane];
      const int m = mt * 16 + r;
      const int n = n0 + 16 * rw + 4 * g;
      if (m < M && n < N) {
        const float stm = I32OUT ? 0.0f : st[mt];
        store4<I32OUT>(y, ldy, c, ldc, m, n, N, vec_out, stm, sc[rw], sum[0], sum[1], sum[2],
                       sum[3]);
      }
    }
}

// ---------------------------------------------------------------------------
// Tiled kernel: TN weight rows x TM token rows per workgroup, BK bytes of K
// per stage, WN x WM waves, each wave (TN/WN) x (TM/WM) via 32x32 fragments.
// ---------------------------------------------------------------------------

template <int TN, int TM, int BK, int WN, int WM>
struct TiledCfg {
  static constexpr int kThreads = WN * WM * kWave;
  static constexpr int kLdsRow = BK + 16;             // padded row, bytes
  static constexpr int kFN = TN / WN / 32;
  static constexpr int kFM = TM / WM / 32;
  static constexpr int kVecPerRow = BK / 16;
  static constexpr int kWVecs = TN * kVecPerRow / kThreads;
  static constexpr int kXVecs = TM * kVecPerRow / kThreads;
  static_assert(TN * kVecPerRow % kThreads == 0 && TM * kVecPerRow % kThreads == 0, "");
  static_assert(kFN >= 1 && kFM >= 1 && BK % 32 == 0, "");
};

template <int TN, int TM, int BK, int WN, int WM, bool I32OUT>
__global__ __launch_bounds__(WN * WM * kWave) void gemm_tiled_kernel(
    const int8_t* __restrict__ xq, int64_t ldq, const float* __restrict__ s_tok,
    const int8_t* __restrict__ wq, int64_t ldw, const float* __restrict__ s_chan, int M, int N,
    int K, uint16_t* __restrict__ y, int64_t ldy, int32_t* __restrict__ c, int64_t ldc,
    bool vec_out) {
  using C = TiledCfg<TN, TM, BK, WN, WM>;
  constexpr int LR = C::kLdsRow, FN = C::kFN, FM = C::kFM;
  __shared__ __attribute__((aligned(16))) int8_t lds_w[2][TN * LR];
  __shared__ __attribute__((aligned(16))) int8_t lds_x[2][TM * LR];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wn = wave % WN, wm = wave / WN;
  const int n0 = blockIdx.x * TN;
  const int m0 = blockIdx.y * TM;

  // Global -> register staging: vector v of the W tile is row v / VPR,
  // 16-byte column v % VPR. Rows past N/M read a valid row (results unused).
  const int8_t* wsrc[C::kWVecs];
  int wdst[C::kWVecs], wcol[C::kWVecs];
#pragma unroll
  for (int i = 0; i < C::kWVecs; ++i) {
    const int v = tid + i * C::kThreads;
    const int row = v / C::kVecPerRow, col = v % C::kVecPerRow;
    wsrc[i] = wq + (int64_t)min(n0 + row, N - 1) * ldw + col * 16;
    wdst[i] = row * LR + col * 16;
    wcol[i] = col * 16;
  }
  const int8_t* xsrc[C::kXVecs];
  int xdst[C::kXVecs], xcol[C::kXVecs];
#pragma unroll
  for (int i = 0; i < C::kXVecs; ++i) {
    const int v = tid + i * C::kThreads;
    const int row = v / C::kVecPerRow, col = v % C::kVecPerRow;
    xsrc[i] = xq + (int64_t)min(m0 + row, M - 1) * ldq + col * 16;
    xdst[i] = row * LR + col * 16;
    xcol[i] = col * 16;
  }

  v4i wreg[C::kWVecs], xreg[C::kXVecs];
  const v4i zero = {0, 0, 0, 0};
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::kWVecs; ++i) wreg[i] = (k0 + wcol[i] < K) ? ldg16(wsrc[i] + k0) : zero;
#pragma unroll
    for (int i = 0; i < C::kXVecs; ++i) xreg[i] = (k0 + xcol[i] < K) ? ldg16(xsrc[i] + k0) : zero;
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::kWVecs; ++i) *reinterpret_cast<v4i*>(&lds_w[buf][wdst[i]]) = wreg[i];
#pragma unroll
    for (int i = 0; i < C::kXVecs; ++i) *reinterpret_cast<v4i*>(&lds_x[buf][xdst[i]]) = xreg[i];
  };

  v16i acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  // LDS read offsets: row l % 32 of each fragment, K group 16 * (l / 32).
  const int frag_row = lane & 31, frag_k = 16 * (lane >> 5);
  const int wbase = (wn * FN * 32 + frag_row) * LR + frag_k;
  const int xbase = (wm * FM * 32 + frag_row) * LR + frag_k;

  const int nk = (K + BK - 1) / BK;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_stage((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      v4i a[FN], b[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i)
        a[i] = *reinterpret_cast<const v4i*>(&lds_w[buf][wbase + i * 32 * LR + ks * 32]);
#pragma unroll
      for (int j = 0; j < FM; ++j)
        b[j] = *reinterpret_cast<const v4i*>(&lds_x[buf][xbase + j * 32 * LR + ks * 32]);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_stage(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds token m = .. + l % 32 and, per group of 4 registers,
  // four consecutive output channels.
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int m = m0 + wm * FM * 32 + j * 32 + (lane & 31);
      if (m >= M) continue;
      const float st = I32OUT ? 0.0f : s_tok[m];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * FN * 32 + i * 32 + 8 * q + 4 * (lane >> 5);
        if (n < N) {
          float sc[4] = {0, 0, 0, 0};
          if constexpr (!I32OUT) load_chan4(s_chan, n, N, sc);
          store4<I32OUT>(y, ldy, c, ldc, m, n, N, vec_out, st, sc, acc[i][j][4 * q],
                         acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        }
      }
    }
}

// ---------------------------------------------------------------------------
// Prefill kernel: 256 x 256 output tile per workgroup, BK = 64 bytes of K per
// stage, NS LDS stages fed by direct global -> LDS loads
// (global_load_lds_dwordx4), 4 waves in a 2 x 2 grid, each owning a
// 128 x 128 sub-tile as 4 x 4 v_mfma_i32_32x32x32_i8 fragments (256
// accumulator registers per lane, held in AGPRs).
//
// LDS layout of a stage: W tile [256 rows][64 B] then X tile [256][64 B].
// Row r's 16-byte chunk c sits at chunk slot c ^ swz(r),
// swz(r) = ((r >> 1) ^ (r >> 2)) & 3, so the 32 rows one fragment read
// touches spread over all banks (conflict-free for 8-lane/32-bank and
// 16-lane/64-bank service alike). A DMA instruction writes 64 consecutive
// chunks (1 KB) of LDS; the swizzle is applied by choosing which global
// chunk each lane fetches.
//
// Pipeline per stage s: wait for this wave's DMA of stage s (vmcnt), one
// s_barrier (all waves' DMA of stage s landed, all reads of stage s-1 done),
// issue the DMA of stage s + NS - 1 into the buffer stage s - 1 used, then
// run stage s's ds_reads and MFMAs. The barrier is a bare s_barrier: a
// fence would wait for every outstanding DMA and serialize the stages.
// Each stage buffer is its own __shared__ array so the compiler knows that
// reading one buffer does not depend on DMA into another.
// ---------------------------------------------------------------------------

namespace pf {
constexpr int TN = 256, TM = 256, BK = 64, NS = 4;
constexpr int TILE_BYTES = TN * BK;               // 16 KB per operand per stage
constexpr int STAGE_BYTES = 2 * TILE_BYTES;       // W then X
constexpr int GROUP_M = 4;                        // M tiles per tile group
}  // namespace pf

__device__ __forceinline__ int lds_swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

// WN x WM waves; wave (wn, wm) owns output channels [wn*TN/WN, +TN/WN) and
// tokens [wm*TM/WM, +TM/WM) of the tile as FN x FM 32x32 fragments.
template <int WN, int WM>
struct PrefillCfg {
  static constexpr int kThreads = WN * WM * kWave;
  static constexpr int kFN = pf::TN / WN / 32, kFM = pf::TM / WM / 32;
  static constexpr int kDmaPerOperand = pf::TILE_BYTES / (kThreads * 16);
  static constexpr int kDmaPerStage = 2 * kDmaPerOperand;
  static_assert(kDmaPerOperand * kThreads * 16 == pf::TILE_BYTES, "");
};

template <int WN, int WM, bool I32OUT>
__global__ __launch_bounds__(WN * WM * kWave, 1) void gemm_prefill_kernel(
    const int8_t* __restrict__ xq, int64_t ldq, const float* __restrict__ s_tok,
    const int8_t* __restrict__ wq, int64_t ldw, const float* __restrict__ s_chan, int M, int N,
    int K, uint16_t* __restrict__ y, int64_t ldy, int32_t* __restrict__ c, int64_t ldc,
    bool vec_out) {
  using namespace pf;
  using C = PrefillCfg<WN, WM>;
  constexpr int THREADS = C::kThreads, FN = C::kFN, FM = C::kFM;
  constexpr int DPO = C::kDmaPerOperand, DPS = C::kDmaPerStage;
  __shared__ __attribute__((aligned(1024))) int8_t buf0[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) int8_t buf1[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) int8_t buf2[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) int8_t buf3[STAGE_BYTES];
  static_assert(NS == 4, "four stage buffers are declared");

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wn = wave % WN, wm = wave / WN;

  // ---- tile index: XCD-aware, then grouped along M ----
  const int tiles_n = (N + TN - 1) / TN, tiles_m = (M + TM - 1) / TM;
  const int T = tiles_n * tiles_m;
  const int b = blockIdx.x;
  const int Tq = T / 8;
  // workgroups are dealt round-robin to the 8 XCDs: give each XCD a run of
  // consecutive tiles so that its L2 sees shared W and X panels
  const int t = (b < 8 * Tq) ? (b % 8) * Tq + b / 8 : b;
  const int group = t / (GROUP_M * tiles_n);
  const int first_m = group * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int in_group = t % (GROUP_M * tiles_n);
  const int tile_m = first_m + in_group % gsize;
  const int tile_n = in_group / gsize;
  const int n0 = tile_n * TN, m0 = tile_m * TM;

  // ---- DMA sources: instruction i of this wave fills LDS chunks
  // [i*THREADS + wave*64, +64); chunk p holds row p/4, global chunk (p%4)^swz ----
  const int8_t* wsrc[DPO];
  const int8_t* xsrc[DPO];
#pragma unroll
  for (int i = 0; i < DPO; ++i) {
    const int p = i * THREADS + wave * kWave + lane;
    const int row = p >> 2, cidx = (p & 3) ^ lds_swz(p >> 2);
    wsrc[i] = wq + (int64_t)min(n0 + row, N - 1) * ldw + cidx * 16;
    xsrc[i] = xq + (int64_t)min(m0 + row, M - 1) * ldq + cidx * 16;
  }
  auto issue = [&](int stage, int8_t* bufp) {
    const int64_t k0 = (int64_t)stage * BK;
    const uint32_t base = lds_addr(bufp) + wave * kWave * 16;
#pragma unroll
    for (int i = 0; i < DPO; ++i) dma16(wsrc[i] + k0, base + i * THREADS * 16);
#pragma unroll
    for (int i = 0; i < DPO; ++i) dma16(xsrc[i] + k0, base + TILE_BYTES + i * THREADS * 16);
  };

  // ---- fragment read offsets: row (l % 32) of a fragment, K chunk 2ks + l/32 ----
  const int frow = lane & 31;
  const int sw = lds_swz(frow);           // fragment bases are multiples of 32 rows
  int foff[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) foff[ks] = frow * BK + (((2 * ks + (lane >> 5)) ^ sw) << 4);
  const int wbase = wn * FN * 32 * BK, xbase = TILE_BYTES + wm * FM * 32 * BK;

  v16i acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  // Epilogue scales of this tile (256 channel + 256 token scales), fetched
  // now so their latency hides under the K loop; parked in LDS at the end.
  constexpr int kScalesPerThread = (TN + TM) / THREADS;
  float scale_pre[kScalesPerThread];
  if constexpr (!I32OUT) {
#pragma unroll
    for (int r = 0; r < kScalesPerThread; ++r) {
      const int idx = tid + r * THREADS;
      scale_pre[r] = idx < TN ? s_chan[min(n0 + idx, N - 1)] : s_tok[min(m0 + idx - TN, M - 1)];
    }
  }

  auto compute = [&](const int8_t* bufp) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v4i a[FN], bb[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i)
        a[i] = *reinterpret_cast<const v4i*>(bufp + wbase + i * 32 * BK + foff[ks]);
#pragma unroll
      for (int j = 0; j < FM; ++j)
        bb[j] = *reinterpret_cast<const v4i*>(bufp + xbase + j * 32 * BK + foff[ks]);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], bb[j], acc[i][j], 0, 0, 0);
    }
  };

  const int nfull = K / BK;
  if (0 < nfull) issue(0, buf0);
  if (1 < nfull) issue(1, buf1);
  if (2 < nfull) issue(2, buf2);

#define W8A8_PF_STAGE(J, CUR, NEXT)                                  \
  {                                                                  \
    const int st = s0 + (J);                                         \
    if (st < nfull) {                                                \
      if (st + NS - 2 < nfull) W8A8_WAIT_VM((NS - 2) * DPS);         \
      else W8A8_WAIT_VM(0);                                          \
      barrier_no_fence();                                            \
      if (st + NS - 1 < nfull) issue(st + NS - 1, NEXT);             \
      compute(CUR);                                                  \
    }                                                                \
  }
  for (int s0 = 0; s0 < nfull; s0 += NS) {
    W8A8_PF_STAGE(0, buf0, buf3)
    W8A8_PF_STAGE(1, buf1, buf0)
    W8A8_PF_STAGE(2, buf2, buf1)
    W8A8_PF_STAGE(3, buf3, buf2)
  }
#undef W8A8_PF_STAGE

  // ---- K tail (K % 64 in {16, 32, 48}): staged through registers with
  // zero fill into the buffer the next stage would use ----
  if (nfull * BK < K) {
    int8_t* tb = (nfull % NS == 0) ? buf0 : (nfull % NS == 1) ? buf1 : (nfull % NS == 2) ? buf2 : buf3;
    const int64_t k0 = (int64_t)nfull * BK;
    const v4i zero = {0, 0, 0, 0};
    v4i wv[DPO], xv[DPO];
#pragma unroll
    for (int i = 0; i < DPO; ++i) {
      const int p = i * THREADS + wave * kWave + lane;
      const int cidx = (p & 3) ^ lds_swz(p >> 2);
      const bool in = k0 + cidx * 16 < K;
      wv[i] = in ? ldg16(wsrc[i] + k0) : zero;
      xv[i] = in ? ldg16(xsrc[i] + k0) : zero;
    }
    W8A8_WAIT_VM(0);
    barrier_no_fence();       // every wave is done reading the buffer about to be refilled
#pragma unroll
    for (int i = 0; i < DPO; ++i) {
      *reinterpret_cast<v4i*>(tb + (i * THREADS + wave * kWave + lane) * 16) = wv[i];
      *reinterpret_cast<v4i*>(tb + TILE_BYTES + (i * THREADS + wave * kWave + lane) * 16) = xv[i];
    }
    __syncthreads();
    compute(tb);
  }

  // ---- epilogue: lane holds token m = .. + l % 32 and, per group of 4
  // registers, four consecutive output channels ----
  float* scale_lds = reinterpret_cast<float*>(buf0);   // [TN channel scales | TM token scales]
  if constexpr (!I32OUT) {
    __syncthreads();                                   // all waves are done with buf0
#pragma unroll
    for (int r = 0; r < kScalesPerThread; ++r) scale_lds[tid + r * THREADS] = scale_pre[r];
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int ml = wm * FM * 32 + j * 32 + (lane & 31);
    const int m = m0 + ml;
    if (m >= M) continue;
    const float st = I32OUT ? 0.0f : scale_lds[TN + ml];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = wn * FN * 32 + i * 32 + 8 * q + 4 * (lane >> 5);
        const int n = n0 + nl;
        if (n < N) {
          float sc[4] = {0, 0, 0, 0};
          if constexpr (!I32OUT) {
            const float4 v = *reinterpret_cast<const float4*>(scale_lds + nl);
            sc[0] = v.x; sc[1] = v.y; sc[2] = v.z; sc[3] = v.w;
          }
          store4<I32OUT>(y, ldy, c, ldc, m, n, N, vec_out, st, sc, acc[i][j][4 * q],
                         acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        }
      }
  }
}

// Output tile of workgroup t_lin: tiles are dealt round-robin to the 8 XCDs,
// so each XCD first gets a run of consecutive tiles (shared W and X panels in
// its L2), then tiles go in groups of GROUP_M along M.
__device__ __forceinline__ void prefill_tile_coords(int t_lin, int tiles_n, int tiles_m, int tn,
                                                    int tm, int& n0, int& m0) {
  const int T = tiles_n * tiles_m;
  const int Tq = T / 8;
  const int t = (t_lin < 8 * Tq) ? (t_lin % 8) * Tq + t_lin / 8 : t_lin;
  const int group = t / (pf::GROUP_M * tiles_n);
  const int first_m = group * pf::GROUP_M;
  const int gsize = min(tiles_m - first_m, pf::GROUP_M);
  const int in_group = t % (pf::GROUP_M * tiles_n);
  m0 = (first_m + in_group % gsize) * tm;
  n0 = (in_group / gsize) * tn;
}

// ---------------------------------------------------------------------------
// Prefill kernel, full-line variant (K % 128 == 0): each stage carries 128
// bytes of K per row, so every DMA request covers whole 128-byte lines
// (measured on MI355X: 91 GB/s per CU against 54 GB/s for 64-byte
// half-lines). Two stages: the DMA of stage s + 1 lands while stage s is
// multiplied. Fragment reads are double-buffered in registers: k-step
// ks + 1's LDS reads go out while k-step ks multiplies.
//
// Schedule inside a stage. LDS serves both the fragment reads (192 KB per
// stage per CU) and the DMA writes (64 KB); at the full MFMA rate (2048
// cycles per stage) the reads alone need 96 B/clk, about three quarters of
// what a read-only loop reaches on MI355X, so bursts stall the matrix
// cores. Two things spread
// the load: each k-step's reads are interleaved one-for-one with its MFMAs
// (scheduling group barriers), and the next stage's DMA goes out in two
// halves, one right after the barrier and one after k-step 0's MFMAs.
// Measured on MI355X at M = 4096 against issuing all reads, then all MFMAs,
// with the whole DMA after the barrier: 4-10% faster on the Llama-3.1-8B
// projections (gate_up 494 -> 445 us, down 210 -> 199 us).
//
// The tile is TNV weight rows by TMV token rows with 8 waves: 256 x 256
// (waves 2 x 4), 192 x 256 (2 x 4) or 256 x 192 (4 x 2); the choice is
// launch_prefill128_auto's.
//
// LDS row = 128 B = 8 chunks; row r's chunk c sits at slot
// c ^ swz8(r), swz8(r) = (r & 7) ^ ((r >> 3) & 1): the 8 rows one 8-lane
// group reads, and the 8 even / 8 odd rows of a 16-lane group, all land in
// distinct banks. swz8 depends on the low 4 row bits only, so it is the same
// for every 32-row fragment.
// ---------------------------------------------------------------------------

namespace pf128 {
constexpr int BK = 128, THREADS = 8 * kWave;
}  // namespace pf128

// TNV weight rows x TMV token rows per workgroup, 8 waves in a WNV x WMV grid,
// each wave owning FN x FM 32x32 output fragments.
template <int TNV, int TMV, int WNV, int WMV>
struct Prefill128Cfg {
  static constexpr int kWBytes = TNV * pf128::BK, kXBytes = TMV * pf128::BK;
  static constexpr int kStageBytes = kWBytes + kXBytes;
  static constexpr int kFN = TNV / WNV / 32, kFM = TMV / WMV / 32;
  static constexpr int kDmaW = kWBytes / (pf128::THREADS * 16);
  static constexpr int kDmaX = kXBytes / (pf128::THREADS * 16);
  static constexpr int kScales = TNV + TMV;
  static_assert(WNV * WMV * kWave == pf128::THREADS, "8 waves");
  static_assert(kFN * WNV * 32 == TNV && kFM * WMV * 32 == TMV, "whole fragments per wave");
  static_assert(kDmaW * pf128::THREADS * 16 == kWBytes && kDmaX * pf128::THREADS * 16 == kXBytes,
                "whole DMA instructions per operand tile");
  static_assert(kFN * kFM >= kFN + kFM, "one MFMA per fragment read in the interleaved schedule");
  static_assert(2 * kStageBytes + 4 * kScales <= 160 * 1024, "LDS");
};

template <int TNV, int TMV, int WNV, int WMV, bool I32OUT>
__global__ __launch_bounds__(pf128::THREADS, 1) void gemm_prefill128_kernel(
    const int8_t* __restrict__ xq, int64_t ldq, const float* __restrict__ s_tok,
    const int8_t* __restrict__ wq, int64_t ldw, const float* __restrict__ s_chan, int M, int N,
    int K, uint16_t* __restrict__ y, int64_t ldy, int32_t* __restrict__ c, int64_t ldc,
    bool vec_out) {
  using pf128::BK;
  using pf128::THREADS;
  using C = Prefill128Cfg<TNV, TMV, WNV, WMV>;
  constexpr int TM = TMV, WN = WNV;
  constexpr int FN = C::kFN, FM = C::kFM, DW = C::kDmaW, DX = C::kDmaX;
  constexpr int SB = C::kStageBytes, WB = C::kWBytes;
  __shared__ __attribute__((aligned(1024))) int8_t stages[2 * SB];
  __shared__ __attribute__((aligned(16))) float scale_lds[C::kScales];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wn = wave % WN, wm = wave / WN;
  const int tiles_n = (N + TNV - 1) / TNV, tiles_m = (M + TM - 1) / TM;
  int n0, m0;
  prefill_tile_coords(blockIdx.x, tiles_n, tiles_m, TNV, TM, n0, m0);

  // DMA: instruction i of this wave fills LDS chunks [i*THREADS + wave*64, +64)
  // of an operand tile; chunk p holds row p / 8, global chunk (p % 8) ^ swz8.
  const int8_t* wsrc[DW];
  const int8_t* xsrc[DX];
#pragma unroll
  for (int i = 0; i < DW; ++i) {
    const int p = i * THREADS + tid;
    wsrc[i] = wq + (int64_t)min(n0 + (p >> 3), N - 1) * ldw + ((p & 7) ^ lds_swz8(p >> 3)) * 16;
  }
#pragma unroll
  for (int i = 0; i < DX; ++i) {
    const int p = i * THREADS + tid;
    xsrc[i] = xq + (int64_t)min(m0 + (p >> 3), M - 1) * ldq + ((p & 7) ^ lds_swz8(p >> 3)) * 16;
  }
  const uint32_t lds_base = lds_addr(stages) + wave * kWave * 16;
  // DMA instructions [q0, q1) of stage `stage`: weight tile first, then tokens
  auto issue = [&](int stage, int q0, int q1) {
    const uint32_t base = lds_base + (uint32_t)((stage & 1) * SB);
    const int64_t k0 = (int64_t)stage * BK;
#pragma unroll
    for (int q = 0; q < DW + DX; ++q) {
      if (q < q0 || q >= q1) continue;
      if (q < DW) dma16(wsrc[q] + k0, base + q * THREADS * 16);
      else dma16(xsrc[q - DW] + k0, base + WB + (q - DW) * THREADS * 16);
    }
  };

  // scales for the epilogue, fetched before the K loop
  constexpr int kScalesPerThread = (C::kScales + THREADS - 1) / THREADS;
  float scale_pre[kScalesPerThread];
  if constexpr (!I32OUT) {
#pragma unroll
    for (int r = 0; r < kScalesPerThread; ++r) {
      const int idx = tid + r * THREADS;
      scale_pre[r] = idx < TNV ? s_chan[min(n0 + idx, N - 1)]
                               : s_tok[min(m0 + min(idx - TNV, TM - 1), M - 1)];
    }
  }

  const int frow = lane & 31;
  const int sw = lds_swz8(frow);
  int foff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) foff[ks] = frow * BK + (((2 * ks + (lane >> 5)) ^ sw) << 4);
  const int wbase = wn * FN * 32 * BK, xbase = WB + wm * FM * 32 * BK;

  v16i acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  v4i fa[2][FN], fb[2][FM];
  auto read_frags = [&](const int8_t* bufp, int ks, v4i (&a)[FN], v4i (&b)[FM]) {
#pragma unroll
    for (int i = 0; i < FN; ++i)
      a[i] = *reinterpret_cast<const v4i*>(bufp + wbase + i * 32 * BK + foff[ks]);
#pragma unroll
    for (int j = 0; j < FM; ++j)
      b[j] = *reinterpret_cast<const v4i*>(bufp + xbase + j * 32 * BK + foff[ks]);
  };

  const int nst = K / BK;
  issue(0, 0, DW + DX);
  for (int s = 0; s < nst; ++s) {
    W8A8_WAIT_VM(0);                 // this wave's DMA of stage s has landed
    barrier_no_fence();              // everyone's has; stage s - 1 is fully read
    const bool more = s + 1 < nst;
    if (more) issue(s + 1, 0, (DW + DX) / 2);
    const int8_t* bufp = stages + (s & 1) * SB;
    read_frags(bufp, 0, fa[0], fb[0]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      __builtin_amdgcn_sched_barrier(0);
      if (ks < 3) read_frags(bufp, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[ks & 1][i], fb[ks & 1][j], acc[i][j],
                                                            0, 0, 0);
      // one MFMA, one LDS read, ..., then the remaining MFMAs
      if (ks < 3) {
#pragma unroll
        for (int q = 0; q < FN + FM; ++q) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, FN * FM - FN - FM, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, FN * FM, 0);
      }
      if (ks == 0 && more) {
        __builtin_amdgcn_sched_barrier(0);
        issue(s + 1, (DW + DX) / 2, DW + DX);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // epilogue
  if constexpr (!I32OUT) {
#pragma unroll
    for (int r = 0; r < kScalesPerThread; ++r) {
      const int idx = tid + r * THREADS;
      if (idx < C::kScales) scale_lds[idx] = scale_pre[r];
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int ml = wm * FM * 32 + j * 32 + (lane & 31);
    const int m = m0 + ml;
    if (m >= M) continue;
    const float st = I32OUT ? 0.0f : scale_lds[TNV + ml];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = wn * FN * 32 + i * 32 + 8 * q + 4 * (lane >> 5);
        const int n = n0 + nl;
        if (n < N) {
          float sc[4] = {0, 0, 0, 0};
          if constexpr (!I32OUT) {
            const float4 v = *reinterpret_cast<const float4*>(scale_lds + nl);
            sc[0] = v.x; sc[1] = v.y; sc[2] = v.z; sc[3] = v.w;
          }
          store4<I32OUT>(y, ldy, c, ldc, m, n, N, vec_out, st, sc, acc[i][j][4 * q],
                         acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Mid kernel (decode batches up to a few hundred tokens, K % 128 == 0). The
// skinny kernel's split of the work: a workgroup owns 16*RW output channels
// and 16*MT token rows (M tile blockIdx.y), its NW waves take interleaved K
// stages of 128 bytes and
// sum their partial tiles in LDS at the end. But each wave brings its
// operands in through LDS with direct global -> LDS loads of whole 128-byte
// lines (the token tile is most of the bytes once M > 16, and register
// loads of its 64-byte fragment rows move half lines), NS stages deep in
// a ring of stage buffers of its own. A wave reads only what it loaded, so
// the K loop has no workgroup barrier, and no operand bytes wait in
// registers: NS - 1 stages of every wave are in flight while it multiplies.
//
// Stage layout: W rows [16*RW][128 B] then X rows [16*MT][128 B]; row r's
// 16-byte chunk c sits at slot c ^ swz8(r) (conflict-free reads of the
// 16x16x64 fragments: lane l reads row l % 16, chunk 4 h + l / 16).
//
// Workgroup b walks K starting at stage (b * rot) mod (K / 128) (integer sums
// are exact in any order). With weight rows a multiple of 4 KB apart,
// workgroups walking K in step would read addresses that agree in their low
// 12 bits; the host passes rot = 9 there, which measured 2.6 us faster for
// the 28672 x 4096 projection at one token (23.8 -> 21.1 us) and 0.3-0.5 us
// for the 4096- and 6144-row ones; other strides gain nothing (rot = 0).
// ---------------------------------------------------------------------------

template <int MT, int RW, int NW, int NS>
struct MidCfg {
  static constexpr int kBK = 128;
  static constexpr int kWBytes = 16 * RW * kBK, kXBytes = 16 * MT * kBK;
  static constexpr int kStageBytes = kWBytes + kXBytes;
  static constexpr int kDmaW = kWBytes / (kWave * 16), kDmaX = kXBytes / (kWave * 16);
  static constexpr int kDma = kDmaW + kDmaX;              // DMA instructions per stage
  static constexpr int kLdsBytes = NW * NS * kStageBytes;
  static_assert(MT >= 1 && MT <= 4 && RW >= 1 && NW >= 1 && NS >= 2 && NS <= 4, "");
  static_assert((NS - 1) * kDma <= 63, "vmcnt holds at most 63 outstanding loads");
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
  static_assert(NW * RW * MT * kWave * 16 <= kLdsBytes, "partial tiles fit in the stage buffers");
};

template <int MT, int RW, int NW, int NS, bool I32OUT>
__global__ __launch_bounds__(NW * kWave) void gemm_mid_kernel(
    const int8_t* __restrict__ xq, int64_t ldq, const float* __restrict__ s_tok,
    const int8_t* __restrict__ wq, int64_t ldw, const float* __restrict__ s_chan, int M, int N,
    int K, uint16_t* __restrict__ y, int64_t ldy, int32_t* __restrict__ c, int64_t ldc,
    bool vec_out, int rot) {
  using C = MidCfg<MT, RW, NW, NS>;
  constexpr int BK = C::kBK, SB = C::kStageBytes, DW = C::kDmaW, DX = C::kDmaX;
  __shared__ __attribute__((aligned(1024))) int8_t lds[C::kLdsBytes];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16 * RW, m0 = blockIdx.y * 16 * MT;

  float st[MT], sc[RW][4];
  if constexpr (!I32OUT) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) st[mt] = s_tok[min(m0 + mt * 16 + r, M - 1)];
#pragma unroll
    for (int rw = 0; rw < RW; ++rw) load_chan4(s_chan, n0 + 16 * rw + 4 * g, N, sc[rw]);
  }

  // DMA sources: instruction i fills chunks [64 i, 64 i + 64) of an operand
  // tile; chunk p holds row p / 8, global chunk (p % 8) ^ swz8(p / 8). Rows
  // past N or M read a valid row; their outputs are never stored.
  const int8_t* wsrc[DW];
  const int8_t* xsrc[DX];
#pragma unroll
  for (int i = 0; i < DW; ++i) {
    const int p = i * kWave + lane;
    wsrc[i] = wq + (int64_t)min(n0 + (p >> 3), N - 1) * ldw + ((p & 7) ^ lds_swz8(p >> 3)) * 16;
  }
#pragma unroll
  for (int i = 0; i < DX; ++i) {
    const int p = i * kWave + lane;
    xsrc[i] = xq + (int64_t)min(m0 + (p >> 3), M - 1) * ldq + ((p & 7) ^ lds_swz8(p >> 3)) * 16;
  }
  const int nst = K / BK;
  const int first = (int)((int64_t)blockIdx.x * rot % nst);
  int8_t* const ring = lds + wave * NS * SB;
  const uint32_t ring_addr = lds_addr(ring);
  auto issue = [&](int stage, int slot) {
    const uint32_t base = ring_addr + slot * SB;
    const int ks = stage + first < nst ? stage + first : stage + first - nst;
    const int64_t k0 = (int64_t)ks * BK;
#pragma unroll
    for (int i = 0; i < DW; ++i) dma16(wsrc[i] + k0, base + i * kWave * 16);
#pragma unroll
    for (int i = 0; i < DX; ++i) dma16(xsrc[i] + k0, base + C::kWBytes + i * kWave * 16);
  };

  int foff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) foff[h] = r * BK + (((4 * h + g) ^ lds_swz8(r)) << 4);

  v4i acc[RW][MT];
#pragma unroll
  for (int rw = 0; rw < RW; ++rw)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[rw][mt] = v4i{0, 0, 0, 0};

  // This wave's stages: wave, wave + NW, ...; stage j sits in slot j % NS.
  const int nj = nst > wave ? (nst - wave + NW - 1) / NW : 0;
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < nj) issue(wave + j * NW, j);
  for (int j = 0; j < nj; ++j) {
    if (j + NS - 1 < nj) {
      W8A8_WAIT_LGKM0();   // the reads of the slot about to be refilled have returned
      issue(wave + (j + NS - 1) * NW, (j + NS - 1) % NS);
    }
    wait_stages<C::kDma>(min(nj - 1 - j, NS - 1));
    const int8_t* bp = ring + (j % NS) * SB;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v4i a[RW], b[MT];
#pragma unroll
      for (int rw = 0; rw < RW; ++rw) a[rw] = *reinterpret_cast<const v4i*>(bp + rw * 16 * BK + foff[h]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        b[mt] = *reinterpret_cast<const v4i*>(bp + C::kWBytes + mt * 16 * BK + foff[h]);
#pragma unroll
      for (int rw = 0; rw < RW; ++rw)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[rw][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[rw], b[mt], acc[rw][mt], 0, 0, 0);
    }
  }

  // Sum the NW partial tiles (stage buffers reused once every wave is done);
  // tile t = rw * MT + mt is finished by wave t % NW, whose lane l then holds
  // token 16 mt + l % 16 and channels 16 rw + 4 (l / 16) + e.
  __syncthreads();
  v4i* red = reinterpret_cast<v4i*>(lds);
#pragma unroll
  for (int rw = 0; rw < RW; ++rw)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[(wave * RW * MT + rw * MT + mt) * kWave + lane] = acc[rw][mt];
  __syncthreads();
#pragma unroll
  for (int rw = 0; rw < RW; ++rw)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int t = rw * MT + mt;
      if (t % NW != wave) continue;
      v4i sum = red[t * kWave + lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) sum += red[(w * RW * MT + t) * kWave + lane];
      const int m = m0 + mt * 16 + r;
      const int n = n0 + 16 * rw + 4 * g;
      if (m < M && n < N) {
        const float stm = I32OUT ? 0.0f : st[mt];
        store4<I32OUT>(y, ldy, c, ldc, m, n, N, vec_out, stm, sc[rw], sum[0], sum[1], sum[2],
                       sum[3]);
      }
    }
}

// Compute units of the current device, queried once per device and kept
// (the launchers call this on every GEMM; concurrent first calls store the
// same value).
static int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < kMaxDevices && (cus = cached[dev].load(std::memory_order_relaxed)) > 0)
    return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (dev >= 0 && dev < kMaxDevices) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

template <int TNV, int TMV, int WNV, int WMV, bool I32OUT>
static void launch_prefill128(const int8_t* xq, int64_t ldq, const float* s_tok, const int8_t* wq,
                              int64_t ldw, const float* s_chan, int M, int N, int K, uint16_t* y,
                              int64_t ldy, int32_t* c, int64_t ldc, bool vec_out, hipStream_t s) {
  const int tiles = ((N + TNV - 1) / TNV) * ((M + TMV - 1) / TMV);
  hipLaunchKernelGGL((gemm_prefill128_kernel<TNV, TMV, WNV, WMV, I32OUT>), dim3((unsigned)tiles),
                     dim3(pf128::THREADS), 0, s, xq, ldq, s_tok, wq, ldw, s_chan, M, N, K, y, ldy,
                     c, ldc, vec_out);
}

// Tile of the full-line prefill kernel: dispatch::prefill_tile.
template <bool I32OUT>
static void launch_prefill128_auto(const int8_t* xq, int64_t ldq, const float* s_tok,
                                   const int8_t* wq, int64_t ldw, const float* s_chan, int M,
                                   int N, int K, uint16_t* y, int64_t ldy, int32_t* c, int64_t ldc,
                                   bool vec_out, hipStream_t s) {
  switch (dispatch::prefill_tile(M, N, device_cus())) {
    case dispatch::PrefillTile::k256x192:
      launch_prefill128<256, 192, 4, 2, I32OUT>(xq, ldq, s_tok, wq, ldw, s_chan, M, N, K, y, ldy,
                                                c, ldc, vec_out, s);
      break;
    case dispatch::PrefillTile::k192x256:
      launch_prefill128<192, 256, 2, 4, I32OUT>(xq, ldq, s_tok, wq, ldw, s_chan, M, N, K, y, ldy,
                                                c, ldc, vec_out, s);
      break;
    default:
      launch_prefill128<256, 256, 2, 4, I32OUT>(xq, ldq, s_tok, wq, ldw, s_chan, M, N, K, y, ldy,
                                                c, ldc, vec_out, s);
  }
}

template <int WN, int WM, bool I32OUT>
static void launch_prefill(const int8_t* xq, int64_t ldq, const float* s_tok, const int8_t* wq,
                           int64_t ldw, const float* s_chan, int M, int N, int K, uint16_t* y,
                           int64_t ldy, int32_t* c, int64_t ldc, bool vec_out, hipStream_t s) {
  const int tiles = ((N + pf::TN - 1) / pf::TN) * ((M + pf::TM - 1) / pf::TM);
  hipLaunchKernelGGL((gemm_prefill_kernel<WN, WM, I32OUT>), dim3((unsigned)tiles),
                     dim3(PrefillCfg<WN, WM>::kThreads), 0, s, xq, ldq, s_tok, wq, ldw, s_chan, M,
                     N, K, y, ldy, c, ldc, vec_out);
}

// ---------------------------------------------------------------------------
// Dispatch
// ---------------------------------------------------------------------------


template <int MT, int RW, int NW, int U, bool I32OUT, bool LATE = false>
static void launch_skinny(const int8_t* xq, int64_t ldq, const float* s_tok, const int8_t* wq,
                          int64_t ldw, const float* s_chan, int M, int N, int K, uint16_t* y,
                          int64_t ldy, int32_t* c, int64_t ldc, bool vec_out, hipStream_t s) {
  using C = SkinnyCfg<MT, RW, NW, U>;
  const dim3 grid((unsigned)((N + C::kRows - 1) / C::kRows)), block(C::kThreads);
  hipLaunchKernelGGL((gemm_skinny_kernel<MT, RW, NW, U, I32OUT, LATE>), grid, block, 0, s, xq, ldq,
                     s_tok, wq, ldw, s_chan, M, N, K, y, ldy, c, ldc, vec_out);
}

template <int MT, int RW, int NW, int NS, bool I32OUT>
static void launch_mid(const int8_t* xq, int64_t ldq, const float* s_tok, const int8_t* wq,
                       int64_t ldw, const float* s_chan, int M, int N, int K, uint16_t* y,
                       int64_t ldy, int32_t* c, int64_t ldc, bool vec_out, hipStream_t s) {
  const dim3 grid((unsigned)((N + 16 * RW - 1) / (16 * RW)), (unsigned)((M + 16 * MT - 1) / (16 * MT))),
      block(NW * kWave);
  const int rot = ldw % 4096 == 0 ? kMidRotation : 0;
  hipLaunchKernelGGL((gemm_mid_kernel<MT, RW, NW, NS, I32OUT>), grid, block, 0, s, xq, ldq, s_tok,
                     wq, ldw, s_chan, M, N, K, y, ldy, c, ldc, vec_out, rot);
}

// One register-staged decode-kernel instance if its arguments are the chosen ones.
template <int MT, int RW, int NW, int U, bool LATE, bool I32OUT>
static bool launch_skinny_if(const dispatch::SkinnyConfig& k, const int8_t* xq, int64_t ldq,
                             const float* s_tok, const int8_t* wq, int64_t ldw,
                             const float* s_chan, int M, int N, int K, uint16_t* y, int64_t ldy,
                             int32_t* c, int64_t ldc, bool vec_out, hipStream_t s) {
  if (k.mt != MT || k.rw != RW || k.nw != NW || k.u != U || k.late != LATE) return false;
  launch_skinny<MT, RW, NW, U, I32OUT, LATE>(xq, ldq, s_tok, wq, ldw, s_chan, M, N, K, y, ldy, c,
                                              ldc, vec_out, s);
  return true;
}

// One decode-kernel instance if its template arguments are the chosen ones.
template <int MT, int RW, int NW, int NS, bool I32OUT>
static bool launch_mid_if(const dispatch::MidConfig& m, const int8_t* xq, int64_t ldq,
                          const float* s_tok, const int8_t* wq, int64_t ldw, const float* s_chan,
                          int M, int N, int K, uint16_t* y, int64_t ldy, int32_t* c, int64_t ldc,
                          bool vec_out, hipStream_t s) {
  if (m.mt != MT || m.rw != RW || m.nw != NW || m.ns != NS) return false;
  launch_mid<MT, RW, NW, NS, I32OUT>(xq, ldq, s_tok, wq, ldw, s_chan, M, N, K, y, ldy, c, ldc,
                                     vec_out, s);
  return true;
}

template <bool I32OUT>
static hipError_t launch_gemm_t(const int8_t* xq, int64_t ldq, const float* s_tok,
                                const int8_t* wq, int64_t ldw, const float* s_chan, int M,
                                int N, int K, uint16_t* y, int64_t ldy, int32_t* c, int64_t ldc,
                                bool vec_out, hipStream_t s) {
  const dispatch::GemmPath path = dispatch::gemm_path(M, N, K);
  if (path == dispatch::GemmPath::kMid) {
    // Every configuration dispatch::mid_config can return has an instance.
    const dispatch::MidConfig m = dispatch::mid_config(M, N, K, device_cus());
#define W8A8_MID(MTV, RWV, NWV, NSV)                                                       \
  launch_mid_if<MTV, RWV, NWV, NSV, I32OUT>(m, xq, ldq, s_tok, wq, ldw, s_chan, M, N, K, y, \
                                            ldy, c, ldc, vec_out, s)
    const bool launched =
        W8A8_MID(1, 2, 4, 3) || W8A8_MID(1, 1, 4, 4) || W8A8_MID(1, 1, 4, 3) ||
        W8A8_MID(2, 4, 4, 3) || W8A8_MID(2, 2, 4, 4) || W8A8_MID(2, 1, 4, 4) ||
        W8A8_MID(2, 1, 8, 3) || W8A8_MID(3, 4, 2, 3) || W8A8_MID(3, 2, 4, 3) ||
        W8A8_MID(3, 1, 4, 3) || W8A8_MID(4, 4, 2, 2) || W8A8_MID(4, 2, 4, 3) ||
        W8A8_MID(4, 1, 4, 3) || W8A8_MID(4, 4, 4, 2);
#undef W8A8_MID
    if (!launched) return hipErrorInvalidValue;
  } else if (path == dispatch::GemmPath::kSkinny) {
    // Every configuration dispatch::skinny_config can return has an instance.
    const dispatch::SkinnyConfig k = dispatch::skinny_config(M, N, K);
#define W8A8_SKINNY(MTV, RWV, NWV, UV, LATEV)                                                     \
  launch_skinny_if<MTV, RWV, NWV, UV, LATEV, I32OUT>(k, xq, ldq, s_tok, wq, ldw, s_chan, M, N, K, \
                                                     y, ldy, c, ldc, vec_out, s)
    const bool launched =
        W8A8_SKINNY(1, 2, 8, 8, false) || W8A8_SKINNY(1, 1, 16, 2, false) ||
        W8A8_SKINNY(1, 1, 16, 8, false) || W8A8_SKINNY(1, 4, 8, 2, false) ||
        W8A8_SKINNY(1, 2, 8, 8, true) || W8A8_SKINNY(1, 1, 8, 4, false) ||
        W8A8_SKINNY(2, 4, 4, 2, true) || W8A8_SKINNY(2, 2, 8, 4, false) ||
        W8A8_SKINNY(2, 1, 16, 4, false) || W8A8_SKINNY(3, 4, 4, 2, false) ||
        W8A8_SKINNY(3, 2, 8, 2, false) || W8A8_SKINNY(3, 1, 16, 2, false) ||
        W8A8_SKINNY(4, 4, 4, 2, true) || W8A8_SKINNY(4, 2, 8, 2, false) ||
        W8A8_SKINNY(4, 1, 16, 2, false) || W8A8_SKINNY(4, 1, 8, 8, false);
#undef W8A8_SKINNY
    if (!launched) return hipErrorInvalidValue;
  } else if (path == dispatch::GemmPath::kPrefill128) {
    launch_prefill128_auto<I32OUT>(xq, ldq, s_tok, wq, ldw, s_chan, M, N, K, y, ldy, c, ldc,
                                   vec_out, s);
  } else if (path == dispatch::GemmPath::kPrefill64) {
    launch_prefill<2, 4, I32OUT>(xq, ldq, s_tok, wq, ldw, s_chan, M, N, K, y, ldy, c, ldc, vec_out,
                                 s);
  } else {
    constexpr int TN = 128, TM = 128, BK = 64, WN = 2, WM = 2;
    const dim3 grid((unsigned)((N + TN - 1) / TN), (unsigned)((M + TM - 1) / TM));
    hipLaunchKernelGGL((gemm_tiled_kernel<TN, TM, BK, WN, WM, I32OUT>), grid,
                       dim3(TiledCfg<TN, TM, BK, WN, WM>::kThreads), 0, s, xq, ldq, s_tok, wq, ldw,
                       s_chan, M, N, K, y, ldy, c, ldc, vec_out);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const int8_t* xq, int64_t ldq, const float* s_tok, const int8_t* wq,
                       int64_t ldw, const float* s_chan, int64_t M, int64_t N, int64_t K,
                       uint16_t* y, int64_t ldy, int32_t* acc, int64_t ldc, hipStream_t s) {
  if (acc) {
    const bool vec = (reinterpret_cast<uintptr_t>(acc) % 16 == 0) && (ldc % 4 == 0);
    return launch_gemm_t<true>(xq, ldq, nullptr, wq, ldw, nullptr, (int)M, (int)N, (int)K,
                               nullptr, 0, acc, ldc, vec, s);
  }
  const bool vec = (reinterpret_cast<uintptr_t>(y) % 8 == 0) && (ldy % 4 == 0);
  return launch_gemm_t<false>(xq, ldq, s_tok, wq, ldw, s_chan, (int)M, (int)N, (int)K, y, ldy,
                              nullptr, 0, vec, s);
}

}  // namespace w8a8
