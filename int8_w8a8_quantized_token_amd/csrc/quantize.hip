// Per-row symmetric int8 quantization on gfx950, plus the calibration
// reductions that feed the SmoothQuant factors.
//
// Row quantization follows the Red Hat article "Understanding W8A8 INT8 LLM
// quantization: Half the size, better performance, same accuracy":
//   * activations, section "Why activation quantization is hard, and how
//     SmoothQuant fixes it": one scale per token, max|x| / 127, at run time,
//     after dividing each channel by its smoothing factor;
//   * weights, section "The problem with naive quantization": one scale per
//     output channel; section "How the SmoothQuant smoothing factor is
//     computed": the weight is first scaled by the factor and kept in bf16.
// Codes round half away from zero and are clamped to [-127, 127] (the worked
// example of "How SmoothQuant prevents outliers in activation tensors").
//
// Design (HBM-bound): one workgroup per row (1024 threads when there are few
// rows, 256 otherwise); each thread reads 16-byte vectors (8 bf16) at a
// stride of one block, so a wavefront reads 1 KB contiguous per load. The row
// stays in registers between the absmax pass and the quantize pass (rows up
// to 32768 channels), so HBM sees each input byte once and each output byte
// once. Every floating-point step is one correctly
// rounded binary32 operation in the order written (no contraction, true
// divisions), which is what makes the codes bit-exact.

#include "device_common.h"
#include "launchers.h"

namespace w8a8 {

constexpr int kRowThreads = 256;      // threads per row, large M
constexpr int kRowThreadsLongK = 512; // threads per row, large M and K > 8192
constexpr int kRowThreadsSmallM = 1024; // threads per row when few rows fill the chip
constexpr int64_t kSmallM = 512;

template <RowMode MODE, bool SMOOTH>
__device__ __forceinline__ float prep_value(float v, const float* __restrict__ smooth, int k) {
  if constexpr (!SMOOTH) {
    return v;
  } else if constexpr (MODE == RowMode::kActivation) {
    return v / smooth[k];
  } else {
    return __uint_as_float(f32_to_bf16_rne(v * smooth[k]) << 16);
  }
}

template <RowMode MODE, bool SMOOTH>
__device__ __forceinline__ void load_prep8(const uint16_t* __restrict__ xr,
                                           const float* __restrict__ smooth, int vi,
                                           float (&out)[8]) {
  const uint4 raw = *reinterpret_cast<const uint4*>(xr + (int64_t)vi * 8);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    out[2 * e] = prep_value<MODE, SMOOTH>(bf16_lo(w[e]), smooth, vi * 8 + 2 * e);
    out[2 * e + 1] = prep_value<MODE, SMOOTH>(bf16_hi(w[e]), smooth, vi * 8 + 2 * e + 1);
  }
}

// Codes of 8 values under one row scale, stored as 8 bytes.
__device__ __forceinline__ void store_codes8(int8_t* __restrict__ qr, int vi, const float (&v)[8],
                                             float scale, float R, bool fast) {
  *reinterpret_cast<uint2*>(qr + (int64_t)vi * 8) = codes8(v, scale, R, fast);
}

// Block-wide max of nonnegative values; every thread gets the result.
template <int BS>
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < BS / kWave; ++w) r = fmaxf(r, red[w]);
  return r;
}

// One BS-thread workgroup per row.
// NV > 0: each thread keeps NV vectors in registers (K <= NV * 8 * BS).
// NV == 0: rows longer than that are read twice (second read hits L2).
template <int BS, int NV, RowMode MODE, bool SMOOTH>
__global__ __launch_bounds__(BS) void quantize_rows_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const float* __restrict__ smooth, int K,
    int8_t* __restrict__ q, int64_t ldq, float* __restrict__ scale) {
  __shared__ float red[BS / kWave];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * ldx;
  int8_t* qr = q + row * ldq;
  const int nvec = K / 8;
  const int tid = threadIdx.x;

  if constexpr (NV > 0) {
    float v[NV][8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vi = tid + i * BS;
      if (vi < nvec) {
        load_prep8<MODE, SMOOTH>(xr, smooth, vi, v[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[i][e]));
      }
    }
    amax = block_max<BS>(amax, red);
    const float S = amax / kQMax;
    if (tid == 0) scale[row] = S;
    const bool fast = code_fast_ok(S);
    const float R = fast ? 1.0f / S : 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vi = tid + i * BS;
      if (vi < nvec) store_codes8(qr, vi, v[i], S, R, fast);
    }
  } else {
    float amax = 0.0f;
    for (int vi = tid; vi < nvec; vi += BS) {
      float v[8];
      load_prep8<MODE, SMOOTH>(xr, smooth, vi, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
    }
    amax = block_max<BS>(amax, red);
    const float S = amax / kQMax;
    if (tid == 0) scale[row] = S;
    const bool fast = code_fast_ok(S);
    const float R = fast ? 1.0f / S : 0.0f;
    for (int vi = tid; vi < nvec; vi += BS) {
      float v[8];
      load_prep8<MODE, SMOOTH>(xr, smooth, vi, v);
      store_codes8(qr, vi, v, S, R, fast);
    }
  }
}

template <int BS, RowMode MODE, bool SMOOTH>
static hipError_t launch_rows_bs(const uint16_t* x, int64_t ldx, const float* smooth,
                                 int64_t rows, int64_t K, int8_t* q, int64_t ldq, float* scale,
                                 hipStream_t s) {
  const int64_t per_thread = (K / 8 + BS - 1) / BS;
  const dim3 grid((unsigned)rows), block(BS);
  const int k = (int)K;
#define W8A8_LAUNCH_NV(NVV)                                                                    \
  hipLaunchKernelGGL((quantize_rows_kernel<BS, NVV, MODE, SMOOTH>), grid, block, 0, s, x, ldx, \
                     smooth, k, q, ldq, scale)
  if (per_thread <= 1) W8A8_LAUNCH_NV(1);
  else if (per_thread <= 2) W8A8_LAUNCH_NV(2);
  else if (per_thread <= 4) W8A8_LAUNCH_NV(4);
  else if (per_thread <= 8) W8A8_LAUNCH_NV(8);
  else {
    if constexpr (BS == kRowThreads) {
      if (per_thread <= 16) {
        W8A8_LAUNCH_NV(16);
        return hipGetLastError();
      }
    }
    W8A8_LAUNCH_NV(0);
  }
#undef W8A8_LAUNCH_NV
  return hipGetLastError();
}

// Few rows cannot fill the chip, so each row gets 1024 threads (shorter
// per-thread chains of divisions); many rows use 256 threads per row.
template <RowMode MODE, bool SMOOTH>
static hipError_t launch_rows_nv(const uint16_t* x, int64_t ldx, const float* smooth,
                                 int64_t rows, int64_t K, int8_t* q, int64_t ldq, float* scale,
                                 hipStream_t s) {
  if (rows <= kSmallM)
    return launch_rows_bs<kRowThreadsSmallM, MODE, SMOOTH>(x, ldx, smooth, rows, K, q, ldq, scale, s);
  if (K > 8192)
    return launch_rows_bs<kRowThreadsLongK, MODE, SMOOTH>(x, ldx, smooth, rows, K, q, ldq, scale, s);
  return launch_rows_bs<kRowThreads, MODE, SMOOTH>(x, ldx, smooth, rows, K, q, ldq, scale, s);
}

hipError_t launch_quantize_rows(RowMode mode, const uint16_t* x, int64_t ldx,
                                const float* smooth, int64_t rows, int64_t K, int8_t* q,
                                int64_t ldq, float* scale, hipStream_t s) {
  if (mode == RowMode::kActivation) {
    return smooth ? launch_rows_nv<RowMode::kActivation, true>(x, ldx, smooth, rows, K, q, ldq, scale, s)
                  : launch_rows_nv<RowMode::kActivation, false>(x, ldx, smooth, rows, K, q, ldq, scale, s);
  }
  return smooth ? launch_rows_nv<RowMode::kWeight, true>(x, ldx, smooth, rows, K, q, ldq, scale, s)
                : launch_rows_nv<RowMode::kWeight, false>(x, ldx, smooth, rows, K, q, ldq, scale, s);
}

// ---------------------------------------------------------------------------
// Calibration: per-channel absmax over rows (accumulating), SmoothQuant factor
// ---------------------------------------------------------------------------

constexpr int kAbsmaxRowsPerBlock = 64;

// Thread t of block (bx, by) owns channels [8*(bx*256+t), +8) over the row
// chunks by, by + gridDim.y, ... of 64 rows each. Nonnegative binary32 values order like their bit
// patterns, so an unsigned atomic max is an exact, order-free reduction.
__global__ __launch_bounds__(kRowThreads) void channel_absmax_kernel(
    const uint16_t* __restrict__ a, int64_t lda, int64_t rows, int K,
    float* __restrict__ absmax) {
  const int vi = blockIdx.x * kRowThreads + threadIdx.x;
  if (vi >= K / 8) return;
  float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int64_t r0 = (int64_t)blockIdx.y * kAbsmaxRowsPerBlock; r0 < rows;
       r0 += (int64_t)gridDim.y * kAbsmaxRowsPerBlock) {
    const int64_t r1 = min(rows, r0 + kAbsmaxRowsPerBlock);
    for (int64_t r = r0; r < r1; ++r) {
      const uint4 raw = *reinterpret_cast<const uint4*>(a + r * lda + (int64_t)vi * 8);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        m[2 * e] = fmaxf(m[2 * e], fabsf(bf16_lo(w[e])));
        m[2 * e + 1] = fmaxf(m[2 * e + 1], fabsf(bf16_hi(w[e])));
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e)
    atomicMax(reinterpret_cast<unsigned int*>(absmax + vi * 8 + e), __float_as_uint(m[e]));
}

hipError_t launch_channel_absmax(const uint16_t* a, int64_t lda, int64_t rows, int64_t K,
                                 float* absmax, hipStream_t s) {
  const int64_t nvec = K / 8;
  const int64_t row_blocks = (rows + kAbsmaxRowsPerBlock - 1) / kAbsmaxRowsPerBlock;
  const dim3 grid((unsigned)((nvec + kRowThreads - 1) / kRowThreads),
                  (unsigned)(row_blocks < 65535 ? row_blocks : 65535));
  hipLaunchKernelGGL(channel_absmax_kernel, grid, dim3(kRowThreads), 0, s, a, lda, rows, (int)K,
                     absmax);
  return hipGetLastError();
}

// smooth[k] = sqrt(ax[k] / aw[k]) (correctly rounded binary32 division and
// square root); 1 where either maximum is 0.
__global__ __launch_bounds__(kRowThreads) void smoothing_factors_kernel(
    const float* __restrict__ ax, const float* __restrict__ aw, int64_t K,
    float* __restrict__ smooth) {
  const int64_t k = (int64_t)blockIdx.x * kRowThreads + threadIdx.x;
  if (k >= K) return;
  const float a = ax[k], w = aw[k];
  smooth[k] = (a > 0.0f && w > 0.0f) ? sqrtf(a / w) : 1.0f;
}

hipError_t launch_smoothing_factors(const float* ax, const float* aw, int64_t K, float* smooth,
                                    hipStream_t s) {
  const dim3 grid((unsigned)((K + kRowThreads - 1) / kRowThreads));
  hipLaunchKernelGGL(smoothing_factors_kernel, grid, dim3(kRowThreads), 0, s, ax, aw, K, smooth);
  return hipGetLastError();
}

}  // namespace w8a8
