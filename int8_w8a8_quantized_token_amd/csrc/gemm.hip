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
// Two kernels:
//   * skinny (M <= 64, decode): the weight matrix is streamed once from HBM
//     directly into MFMA operand registers; a workgroup owns 16 output
//     channels and its waves split K; partial int32 tiles are summed in LDS.
//     v_mfma_i32_16x16x64_i8: the weight rows are the A operand, the token
//     rows the B operand.
//   * tiled (prefill): LDS-staged, double-buffered tiles with
//     v_mfma_i32_32x32x32_i8.
//
// MFMA operand layout: for both operands lane l supplies row (l % R) of its
// matrix and a 16-byte group of K selected by l / R (R = 16 or 32). The
// kernels give A and B the same K grouping, so the K permutation inside the
// instruction cancels (integer addition is exact in any order). Output lane
// l, register e holds D[i][j] with j = l % R and
//   16x16: i = 4*(l/16) + e
//   32x32: i = 8*(e/4) + 4*(l/32) + (e%4).

#include "device_common.h"
#include "launchers.h"

namespace w8a8 {

__device__ __forceinline__ v4i ldg16(const int8_t* p) {
  return *reinterpret_cast<const v4i*>(p);
}

__device__ __forceinline__ float dequant(int acc, float st, float sc) {
  return ((float)acc * st) * sc;
}

// Writes 4 consecutive outputs of row m starting at column n (n % 4 == 0).
// vec: the output rows allow one 8-byte (bf16) or 16-byte (int32) store
// per group of 4 (checked on the host: base and row stride aligned).
template <bool I32OUT>
__device__ __forceinline__ void store4(uint16_t* __restrict__ y, int64_t ldy,
                                       int32_t* __restrict__ c, int64_t ldc,
                                       const float* __restrict__ s_tok,
                                       const float* __restrict__ s_chan, int m, int n, int N,
                                       bool vec, int a0, int a1, int a2, int a3) {
  if constexpr (I32OUT) {
    int32_t* p = c + (int64_t)m * ldc + n;
    if (vec && n + 3 < N) {
      *reinterpret_cast<v4i*>(p) = v4i{a0, a1, a2, a3};
    } else {
      const int a[4] = {a0, a1, a2, a3};
      for (int e = 0; e < 4 && n + e < N; ++e) p[e] = a[e];
    }
  } else {
    const float st = s_tok[m];
    uint16_t* p = y + (int64_t)m * ldy + n;
    if (vec && n + 3 < N) {
      const uint32_t b0 = f32_to_bf16_rne(dequant(a0, st, s_chan[n]));
      const uint32_t b1 = f32_to_bf16_rne(dequant(a1, st, s_chan[n + 1]));
      const uint32_t b2 = f32_to_bf16_rne(dequant(a2, st, s_chan[n + 2]));
      const uint32_t b3 = f32_to_bf16_rne(dequant(a3, st, s_chan[n + 3]));
      *reinterpret_cast<uint2*>(p) = uint2{b0 | (b1 << 16), b2 | (b3 << 16)};
    } else {
      const int a[4] = {a0, a1, a2, a3};
      for (int e = 0; e < 4 && n + e < N; ++e)
        p[e] = (uint16_t)f32_to_bf16_rne(dequant(a[e], st, s_chan[n + e]));
    }
  }
}

// ---------------------------------------------------------------------------
// Skinny kernel: M <= 16*MT tokens, 16 output channels per workgroup.
// ---------------------------------------------------------------------------

constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyUnroll = 8;

template <int MT, bool I32OUT>
__global__ __launch_bounds__(kSkinnyWaves * kWave) void gemm_skinny_kernel(
    const int8_t* __restrict__ xq, int64_t ldq, const float* __restrict__ s_tok,
    const int8_t* __restrict__ wq, int64_t ldw, const float* __restrict__ s_chan, int M, int N,
    int K, uint16_t* __restrict__ y, int64_t ldy, int32_t* __restrict__ c, int64_t ldc,
    bool vec_out) {
  constexpr int NW = kSkinnyWaves, U = kSkinnyUnroll;
  __shared__ v4i red[NW][MT][kWave];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16;

  // Rows past N or M read a valid row; their results land only in outputs
  // that are never stored, since D[i][j] depends on A row i and B row j only.
  const int8_t* wp = wq + (int64_t)min(n0 + r, N - 1) * ldw + g * 16;
  const int8_t* xp[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xp[mt] = xq + (int64_t)min(mt * 16 + r, M - 1) * ldq + g * 16;

  v4i acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = v4i{0, 0, 0, 0};

  const int nfull = K / 64;
  int ch = wave;
  for (; ch + (U - 1) * NW < nfull; ch += U * NW) {
    v4i b[U], a[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) b[u] = ldg16(wp + (int64_t)(ch + u * NW) * 64);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) a[u][mt] = ldg16(xp[mt] + (int64_t)(ch + u * NW) * 64);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b[u], a[u][mt], acc[mt], 0, 0, 0);
  }
  for (; ch < nfull; ch += NW) {
    const v4i b = ldg16(wp + (int64_t)ch * 64);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      acc[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b, ldg16(xp[mt] + (int64_t)ch * 64), acc[mt],
                                                      0, 0, 0);
  }
  // K % 64 in {16, 32, 48}: the last chunk is partial; groups past K are zero.
  const int tail = K - nfull * 64;
  if (tail > 0 && wave == nfull % NW) {
    const bool in = g * 16 < tail;
    const v4i zero = {0, 0, 0, 0};
    const v4i b = in ? ldg16(wp + (int64_t)nfull * 64) : zero;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const v4i a = in ? ldg16(xp[mt] + (int64_t)nfull * 64) : zero;
      acc[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b, a, acc[mt], 0, 0, 0);
    }
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) red[wave][mt][lane] = acc[mt];
  __syncthreads();

  // Wave w finishes token tile w (MT <= NW).
  if (wave < MT) {
    const int mt = wave;
    v4i sum = red[0][mt][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) sum += red[w][mt][lane];
    const int m = mt * 16 + r;
    const int n = n0 + 4 * g;
    if (m < M && n < N) store4<I32OUT>(y, ldy, c, ldc, s_tok, s_chan, m, n, N, vec_out, sum[0], sum[1],
                                  sum[2], sum[3]);
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
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * FN * 32 + i * 32 + 8 * q + 4 * (lane >> 5);
        if (n < N)
          store4<I32OUT>(y, ldy, c, ldc, s_tok, s_chan, m, n, N, vec_out, acc[i][j][4 * q],
                         acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
      }
    }
}

// ---------------------------------------------------------------------------
// Dispatch
// ---------------------------------------------------------------------------

constexpr int kSkinnyMaxM = 64;

template <bool I32OUT>
static hipError_t launch_gemm_t(const int8_t* xq, int64_t ldq, const float* s_tok,
                                const int8_t* wq, int64_t ldw, const float* s_chan, int M,
                                int N, int K, uint16_t* y, int64_t ldy, int32_t* c, int64_t ldc,
                                bool vec_out, hipStream_t s) {
  if (M <= kSkinnyMaxM) {
    const dim3 grid((unsigned)((N + 15) / 16)), block(kSkinnyWaves * kWave);
#define W8A8_SKINNY(MTV)                                                                    \
  hipLaunchKernelGGL((gemm_skinny_kernel<MTV, I32OUT>), grid, block, 0, s, xq, ldq, s_tok, wq, \
                     ldw, s_chan, M, N, K, y, ldy, c, ldc, vec_out)
    if (M <= 16) W8A8_SKINNY(1);
    else if (M <= 32) W8A8_SKINNY(2);
    else if (M <= 48) W8A8_SKINNY(3);
    else W8A8_SKINNY(4);
#undef W8A8_SKINNY
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
