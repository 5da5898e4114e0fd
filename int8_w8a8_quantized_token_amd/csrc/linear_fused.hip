// The whole W8A8 linear for one or two tokens in one gfx950 launch:
// activation quantization, the int8 x int8 -> int32 product and the
// dequantizing bf16 epilogue.
//
// What is computed (Red Hat, "Understanding W8A8 INT8 LLM quantization: Half
// the size, better performance, same accuracy", section "Why activation
// quantization is hard, and how SmoothQuant fixes it"): each token row is
// divided channel-wise by the smoothing factors; its scale is max|x'| / 127
// (or, with a static scale, the one calibrated scale); its codes round half
// away from zero and clamp to [-127, 127]; the exact int32 channel sum is
// rescaled by the token's and the output channel's scales and rounded to
// bf16.
//
// Design. At decode sizes the linear is a stream of the weight matrix, and a
// separate quantize launch costs as much again in launch latency as its own
// work. Here the weight stream is the mid GEMM's: a workgroup owns 16*RW
// output channels, its NW waves take interleaved 128-byte K stages, and each
// wave feeds a private ring of NS LDS stages with direct global -> LDS loads
// of whole lines. Those loads hold no registers, so every wave issues its
// first NS - 1 stages and then, while they are in flight, the workgroup
// quantizes the token rows itself, with the same operations in the same
// order as the quantizers (the codes and scales are the same bits), into an
// LDS code buffer the MFMAs read as their B operand. Every workgroup repeats
// the quantization (M*K values), which is why this serves M <= 2, K <= 4096
// and N < 16384 only: measured on MI355X, it saves 1.0-2.1 us per call on
// the 4096 x 4096 and 6144 x 4096 projections at one token and is slower
// than quantize + GEMM on the wide (28672) and deep (14336) ones, whose
// many or long rows make the repeated quantization cost more than the
// launch it saves.

#include "device_common.h"
#include "gemm_common.h"
#include "launchers.h"

namespace w8a8 {

template <int MQ, int KMAX, int RW, int NW, int NS>
struct FusedCfg {
  static constexpr int kBK = 128;
  static constexpr int kThreads = NW * kWave;
  static constexpr int kPV = (KMAX / 8 + kThreads - 1) / kThreads;  // vectors per thread and row
  static constexpr int kLdk = KMAX + 16;             // code row stride (rows on other banks)
  static constexpr int kStageBytes = 16 * RW * kBK;  // weight rows only
  static constexpr int kDma = kStageBytes / (kWave * 16);
  static constexpr int kRingBytes = NW * NS * kStageBytes;
  static constexpr int kCodeBytes = MQ * kLdk;
  static_assert(MQ == 1 || MQ == 2, "");
  static_assert(KMAX % kBK == 0 && NS >= 2 && NS <= 4, "");
  static_assert((NS - 1) * kDma <= 63, "vmcnt holds at most 63 outstanding loads");
  static_assert(NW * RW * kWave * 16 <= kRingBytes, "partial tiles fit in the ring");
  static_assert(kRingBytes + kCodeBytes <= 160 * 1024, "LDS");
};

// STATIC: one scale for every token, read from scale[0]; otherwise per-token
// dynamic scales. Requires M <= MQ, K % 128 == 0 and K <= KMAX.
template <int MQ, int KMAX, int RW, int NW, int NS, bool SMOOTH, bool STATIC>
__global__ __launch_bounds__(NW * kWave) void linear_fused_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const float* __restrict__ smooth,
    const float* __restrict__ scale, const int8_t* __restrict__ wq, int64_t ldw,
    const float* __restrict__ s_chan, int M, int N, int K, uint16_t* __restrict__ y, int64_t ldy,
    bool vec_out, int rot) {
  using C = FusedCfg<MQ, KMAX, RW, NW, NS>;
  constexpr int BK = C::kBK, SB = C::kStageBytes, PV = C::kPV, LDK = C::kLdk;
  constexpr int BS = C::kThreads;
  __shared__ __attribute__((aligned(1024))) int8_t ring_lds[C::kRingBytes];
  __shared__ __attribute__((aligned(16))) int8_t codes[C::kCodeBytes];
  __shared__ float part[NW][MQ];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16 * RW;
  const int nvk = K / 8;

  // 1. Token rows and smoothing factors first: vector loads complete in
  //    issue order, so the wait for them must not cover the weight stages
  //    issued after them. Thread tid takes the 8-channel vectors tid + i * BS.
  uint4 raw[PV][MQ];
  float sv[PV][8];
#pragma unroll
  for (int i = 0; i < PV; ++i) {
    const int kv = tid + i * BS;
#pragma unroll
    for (int m = 0; m < MQ; ++m)
      raw[i][m] = (kv < nvk && m < M)
                      ? *reinterpret_cast<const uint4*>(x + (int64_t)m * ldx + (int64_t)kv * 8)
                      : uint4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[i][e] = (SMOOTH && kv < nvk) ? smooth[kv * 8 + e] : 1.0f;
  }
  float sc[RW][4];
#pragma unroll
  for (int rw = 0; rw < RW; ++rw) load_chan4(s_chan, n0 + 16 * rw + 4 * g, N, sc[rw]);
  float S_static = 0.0f;
  if constexpr (STATIC) S_static = scale[0];

  // 2. The weight stages of this wave (wave, wave + NW, ...): stage j in
  //    slot j % NS; the first NS - 1 go out now. Chunk p of a stage holds
  //    weight row p / 8, global chunk (p % 8) ^ swz8(p / 8); rows past N read
  //    row N - 1, whose outputs are not stored.
  const int8_t* wsrc[C::kDma];
#pragma unroll
  for (int i = 0; i < C::kDma; ++i) {
    const int p = i * kWave + lane;
    wsrc[i] = wq + (int64_t)min(n0 + (p >> 3), N - 1) * ldw + ((p & 7) ^ lds_swz8(p >> 3)) * 16;
  }
  // Workgroup b walks K from stage (b * rot) mod nst, as the mid GEMM does.
  const int nst = K / BK;
  const int first = (int)((int64_t)blockIdx.x * rot % nst);
  auto kstage = [&](int stage) { return stage + first < nst ? stage + first : stage + first - nst; };
  int8_t* const ring = ring_lds + wave * NS * SB;
  const uint32_t ring_addr = lds_addr(ring);
  auto issue = [&](int stage, int slot) {
    const uint32_t base = ring_addr + slot * SB;
    const int64_t k0 = (int64_t)kstage(stage) * BK;
#pragma unroll
    for (int i = 0; i < C::kDma; ++i) dma16(wsrc[i] + k0, base + i * kWave * 16);
  };
  const int nj = nst > wave ? (nst - wave + NW - 1) / NW : 0;
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < nj) issue(wave + j * NW, j);

  // 3. Quantize the token rows into LDS (codes row m at codes + m * LDK).
  float v[PV][MQ][8];
#pragma unroll
  for (int i = 0; i < PV; ++i)
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
      const uint32_t w[4] = {raw[i][m].x, raw[i][m].y, raw[i][m].z, raw[i][m].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[i][m][2 * e] = bf16_lo(w[e]);
        v[i][m][2 * e + 1] = bf16_hi(w[e]);
      }
      if constexpr (SMOOTH) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[i][m][e] = v[i][m][e] / sv[i][e];
      }
    }
  float S[MQ];
  if constexpr (STATIC) {
#pragma unroll
    for (int m = 0; m < MQ; ++m) S[m] = S_static;
  } else {
    float amax[MQ];
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
      amax[m] = 0.0f;
#pragma unroll
      for (int i = 0; i < PV; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) amax[m] = fmaxf(amax[m], fabsf(v[i][m][e]));
      amax[m] = wave_max(amax[m]);
    }
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < MQ; ++m) part[wave][m] = amax[m];
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
      float a = part[0][m];
#pragma unroll
      for (int w = 1; w < NW; ++w) a = fmaxf(a, part[w][m]);
      S[m] = a / kQMax;
    }
  }
#pragma unroll
  for (int m = 0; m < MQ; ++m) {
    const bool fast = code_fast_ok(S[m]);
    const float R = fast ? 1.0f / S[m] : 0.0f;
    if (m < M) {
#pragma unroll
      for (int i = 0; i < PV; ++i) {
        const int kv = tid + i * BS;
        if (kv < nvk)
          *reinterpret_cast<uint2*>(codes + m * LDK + kv * 8) = codes8(v[i][m], S[m], R, fast);
      }
    }
  }
  __syncthreads();

  // 4. The weight stream. Lane (r, g) reads weight row r and token row
  //    r % MQ, bytes [64 h + 16 g, +16) of each stage; token rows past M hold
  //    anything (their outputs are not stored).
  int foff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) foff[h] = r * BK + (((4 * h + g) ^ lds_swz8(r)) << 4);
  const int8_t* cp = codes + (r & (MQ - 1)) * LDK + g * 16;
  v4i acc[RW];
#pragma unroll
  for (int rw = 0; rw < RW; ++rw) acc[rw] = v4i{0, 0, 0, 0};
  for (int j = 0; j < nj; ++j) {
    if (j + NS - 1 < nj) {
      W8A8_WAIT_LGKM0();   // the reads of the slot about to be refilled have returned
      issue(wave + (j + NS - 1) * NW, (j + NS - 1) % NS);
    }
    wait_stages<C::kDma>(min(nj - 1 - j, NS - 1));
    const int8_t* bp = ring + (j % NS) * SB;
    const int stage = kstage(wave + j * NW);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const v4i b = *reinterpret_cast<const v4i*>(cp + stage * BK + h * 64);
#pragma unroll
      for (int rw = 0; rw < RW; ++rw) {
        const v4i a = *reinterpret_cast<const v4i*>(bp + rw * 16 * BK + foff[h]);
        acc[rw] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[rw], 0, 0, 0);
      }
    }
  }

  // 5. Sum the NW partial tiles (the ring is reused once every wave is
  //    done); tile rw is finished by wave rw % NW, whose lane l holds token
  //    l % 16 and channels 16 rw + 4 (l / 16) + e.
  __syncthreads();
  v4i* red = reinterpret_cast<v4i*>(ring_lds);
#pragma unroll
  for (int rw = 0; rw < RW; ++rw) red[(wave * RW + rw) * kWave + lane] = acc[rw];
  __syncthreads();
#pragma unroll
  for (int rw = 0; rw < RW; ++rw) {
    if (rw % NW != wave) continue;
    v4i sum = red[rw * kWave + lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) sum += red[(w * RW + rw) * kWave + lane];
    const int n = n0 + 16 * rw + 4 * g;
    if (r < M && n < N) {
      const float st = (MQ == 2 && r == 1) ? S[MQ - 1] : S[0];
      store4<false>(y, ldy, nullptr, 0, r, n, N, vec_out, st, sc[rw], sum[0], sum[1], sum[2],
                    sum[3]);
    }
  }
}

template <int MQ, int KMAX, int RW, int NW, int NS, bool STATIC>
static void launch_fused(const uint16_t* x, int64_t ldx, const float* smooth, const float* scale,
                         const int8_t* wq, int64_t ldw, const float* s_chan, int M, int N, int K,
                         uint16_t* y, int64_t ldy, bool vec, hipStream_t s) {
  const dim3 grid((unsigned)((N + 16 * RW - 1) / (16 * RW))), block(NW * kWave);
  const int rot = ldw % 4096 == 0 ? kMidRotation : 0;
  if (smooth)
    hipLaunchKernelGGL((linear_fused_kernel<MQ, KMAX, RW, NW, NS, true, STATIC>), grid, block, 0,
                       s, x, ldx, smooth, scale, wq, ldw, s_chan, M, N, K, y, ldy, vec, rot);
  else
    hipLaunchKernelGGL((linear_fused_kernel<MQ, KMAX, RW, NW, NS, false, STATIC>), grid, block, 0,
                       s, x, ldx, smooth, scale, wq, ldw, s_chan, M, N, K, y, ldy, vec, rot);
}

bool linear_fused_supported(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= kLinearFusedMaxM && N < kLinearFusedMaxN && K % 128 == 0 &&
         K <= kLinearFusedMaxK;
}

// 32 channels per workgroup for N > 4096, else 16 (measured): with 8 waves
// for per-token scales (half the partial maxima to combine), 16 for the
// static scale (no reduction).
template <bool STATIC>
static hipError_t launch_fused_t(const uint16_t* x, int64_t ldx, const float* smooth,
                                 const float* scale, const int8_t* wq, int64_t ldw,
                                 const float* s_chan, int64_t M, int64_t N, int64_t K, uint16_t* y,
                                 int64_t ldy, hipStream_t s) {
  const bool vec = (reinterpret_cast<uintptr_t>(y) % 8 == 0) && (ldy % 4 == 0);
  const int m = (int)M, n = (int)N, k = (int)K;
  const bool mid = N > 4096;
  constexpr int KM = (int)kLinearFusedMaxK;
#define W8A8_FUSED(MQV, RWV, NWV, NSV)                                                          \
  launch_fused<MQV, KM, RWV, NWV, NSV, STATIC>(x, ldx, smooth, scale, wq, ldw, s_chan, m, n, k, \
                                               y, ldy, vec, s)
  constexpr int NWN = STATIC ? 16 : 8;
  if (M == 1) {
    if (mid) W8A8_FUSED(1, 2, 8, 3);
    else W8A8_FUSED(1, 1, NWN, 3);
  } else {
    if (mid) W8A8_FUSED(2, 2, 8, 3);
    else W8A8_FUSED(2, 1, NWN, 3);
  }
#undef W8A8_FUSED
  return hipGetLastError();
}

hipError_t launch_linear_fused(const uint16_t* x, int64_t ldx, const float* smooth,
                               const int8_t* wq, int64_t ldw, const float* s_chan, int64_t M,
                               int64_t N, int64_t K, uint16_t* y, int64_t ldy, hipStream_t s) {
  return launch_fused_t<false>(x, ldx, smooth, nullptr, wq, ldw, s_chan, M, N, K, y, ldy, s);
}

hipError_t launch_linear_fused_static(const uint16_t* x, int64_t ldx, const float* smooth,
                                      const float* scale, const int8_t* wq, int64_t ldw,
                                      const float* s_chan, int64_t M, int64_t N, int64_t K,
                                      uint16_t* y, int64_t ldy, hipStream_t s) {
  return launch_fused_t<true>(x, ldx, smooth, scale, wq, ldw, s_chan, M, N, K, y, ldy, s);
}

}  // namespace w8a8
