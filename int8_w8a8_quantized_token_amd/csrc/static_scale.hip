// Static per-tensor activation scale on gfx950: offline calibration (min-max
// and entropy) and the run-time quantizer that applies one fixed scale to
// every token.
//
// The article "INT8 Post-Training Quantization for LLM Inference on NVIDIA
// GPUs", section "The Heart of PTQ: Entropy-Based Calibration", fixes the
// activation scale ahead of time: min-max calibration maps the largest
// magnitude seen to 127; entropy calibration clips at the threshold T whose
// clipped-and-quantized histogram diverges least (Kullback-Leibler) from the
// clipped one, and uses S = T / 127. At run time the quantizer then needs no
// reduction, and the clamp to [-127, 127] binds beyond the threshold.
//
// Conventions shared with the per-token quantizer: x' = x / s (true binary32
// division), codes round half away from zero and clamp to [-127, 127]; the
// histogram and the entropy search follow the readings stated at
// calibrate_entropy_kernel.

#include "device_common.h"
#include "launchers.h"

namespace w8a8 {

constexpr int kStaticThreads = 256;
constexpr int kStaticRowsPerBlock = 16;

// ---------------------------------------------------------------------------
// Run time: one fixed scale for every token
// ---------------------------------------------------------------------------

// Thread t of block (bx, by) owns channels [8 (bx * 256 + t), +8) of rows
// by, by + gridDim.y, ...: one row per block at a time, so at decode sizes
// every load is independent of the others. Every row also receives
// s_tok[row] = S, so the GEMM applies the static scale through the same
// per-token epilogue.
template <bool SMOOTH>
__global__ __launch_bounds__(kStaticThreads) void quantize_static_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const float* __restrict__ smooth,
    const float* __restrict__ scale, int64_t M, int K, int8_t* __restrict__ q, int64_t ldq,
    float* __restrict__ s_tok) {
  const int vi = blockIdx.x * kStaticThreads + threadIdx.x;
  const int nvec = K / 8;
  const float S = scale[0];
  if (vi == 0)
    for (int64_t r = blockIdx.y; r < M; r += gridDim.y) s_tok[r] = S;
  if (vi >= nvec) return;
  float sv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sv[e] = SMOOTH ? smooth[vi * 8 + e] : 1.0f;
  const bool fast = code_fast_ok(S);
  const float R = fast ? 1.0f / S : 0.0f;
  for (int64_t r = blockIdx.y; r < M; r += gridDim.y) {
    const uint4 raw = *reinterpret_cast<const uint4*>(x + r * ldx + (int64_t)vi * 8);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf16_lo(w[e]);
      v[2 * e + 1] = bf16_hi(w[e]);
    }
    if constexpr (SMOOTH) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = v[e] / sv[e];
    }
    *reinterpret_cast<uint2*>(q + r * ldq + (int64_t)vi * 8) = codes8(v, S, R, fast);
  }
}

static dim3 static_grid(int64_t rows, int64_t K) {
  const int64_t nvec = K / 8;
  const int64_t row_blocks = (rows + kStaticRowsPerBlock - 1) / kStaticRowsPerBlock;
  return dim3((unsigned)((nvec + kStaticThreads - 1) / kStaticThreads),
              (unsigned)(row_blocks < 65535 ? row_blocks : 65535));
}

hipError_t launch_quantize_static(const uint16_t* x, int64_t ldx, const float* smooth,
                                  const float* scale, int64_t M, int64_t K, int8_t* q,
                                  int64_t ldq, float* s_tok, hipStream_t s) {
  const dim3 grid((unsigned)((K / 8 + kStaticThreads - 1) / kStaticThreads),
                  (unsigned)(M < 65535 ? M : 65535)),
      block(kStaticThreads);
  if (smooth)
    hipLaunchKernelGGL(quantize_static_kernel<true>, grid, block, 0, s, x, ldx, smooth, scale, M,
                       (int)K, q, ldq, s_tok);
  else
    hipLaunchKernelGGL(quantize_static_kernel<false>, grid, block, 0, s, x, ldx, smooth, scale, M,
                       (int)K, q, ldq, s_tok);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Calibration: min-max
// ---------------------------------------------------------------------------

constexpr int kCalThreads = 1024;

// amax = max_k RN(act_absmax[k] / smooth[k]) (RN is monotone, so this is the
// largest |x'| over the calibration tokens), scale = RN(amax / 127). One
// workgroup; nonnegative binary32 values order like their bit patterns.
__global__ __launch_bounds__(kCalThreads) void calibrate_minmax_kernel(
    const float* __restrict__ act_absmax, const float* __restrict__ smooth, int64_t K,
    float* __restrict__ amax_out, float* __restrict__ scale_out) {
  __shared__ float red[kCalThreads / kWave];
  float m = 0.0f;
  for (int64_t k = threadIdx.x; k < K; k += kCalThreads) {
    const float a = smooth ? act_absmax[k] / smooth[k] : act_absmax[k];
    m = fmaxf(m, a);
  }
  m = wave_max(m);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
    for (int w = 1; w < kCalThreads / kWave; ++w) r = fmaxf(r, red[w]);
    amax_out[0] = r;
    scale_out[0] = r / kQMax;
  }
}

hipError_t launch_calibrate_minmax(const float* act_absmax, const float* smooth, int64_t K,
                                   float* amax, float* scale, hipStream_t s) {
  hipLaunchKernelGGL(calibrate_minmax_kernel, dim3(1), dim3(kCalThreads), 0, s, act_absmax,
                     smooth, K, amax, scale);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Calibration: histogram of |x'|
// ---------------------------------------------------------------------------

// bin = floor(min(RN(|x'| / w), bins - 1)), w = RN(amax / bins); when w is 0
// (amax 0 or below 2^-138) every value goes to bin 0. Counts gather in LDS and are added
// to the global histogram once per workgroup (accumulating across calls).
template <bool SMOOTH>
__global__ __launch_bounds__(kStaticThreads) void abs_histogram_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const float* __restrict__ smooth, int64_t rows,
    int K, const float* __restrict__ amax, int bins, uint32_t* __restrict__ hist) {
  extern __shared__ uint32_t lh[];
  for (int b = threadIdx.x; b < bins; b += kStaticThreads) lh[b] = 0u;
  __syncthreads();
  const int vi = blockIdx.x * kStaticThreads + threadIdx.x;
  const int nvec = K / 8;
  const float a = amax[0];
  const float w = a / (float)bins;
  const float top = (float)(bins - 1);
  if (vi < nvec) {
    float sv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[e] = SMOOTH ? smooth[vi * 8 + e] : 1.0f;
    for (int64_t r0 = (int64_t)blockIdx.y * kStaticRowsPerBlock; r0 < rows;
         r0 += (int64_t)gridDim.y * kStaticRowsPerBlock) {
      const int64_t r1 = min(rows, r0 + kStaticRowsPerBlock);
      for (int64_t r = r0; r < r1; ++r) {
        const uint4 raw = *reinterpret_cast<const uint4*>(x + r * ldx + (int64_t)vi * 8);
        const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = bf16_lo(wd[e]);
          v[2 * e + 1] = bf16_hi(wd[e]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xs = SMOOTH ? v[e] / sv[e] : v[e];
          const int b = (w == 0.0f) ? 0 : (int)floorf(fminf(fabsf(xs) / w, top));
          atomicAdd(&lh[b], 1u);
        }
      }
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < bins; b += kStaticThreads)
    if (lh[b] != 0u) atomicAdd(&hist[b], lh[b]);
}

hipError_t launch_abs_histogram(const uint16_t* x, int64_t ldx, const float* smooth, int64_t rows,
                                int64_t K, const float* amax, int64_t bins, uint32_t* hist,
                                hipStream_t s) {
  const dim3 grid = static_grid(rows, K), block(kStaticThreads);
  const size_t lds = (size_t)bins * sizeof(uint32_t);
  if (smooth)
    hipLaunchKernelGGL(abs_histogram_kernel<true>, grid, block, lds, s, x, ldx, smooth, rows,
                       (int)K, amax, (int)bins, hist);
  else
    hipLaunchKernelGGL(abs_histogram_kernel<false>, grid, block, lds, s, x, ldx, smooth, rows,
                       (int)K, amax, (int)bins, hist);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Calibration: entropy (KL) threshold search
// ---------------------------------------------------------------------------

// One workgroup. For each candidate i in [L, bins] (L = 128 code magnitudes),
// threshold T_i = i * w:
//   P_i = h[0..i) with the mass beyond T_i added to bin i-1 (saturation);
//   Q_i = the values below T_i: h[0..i) split into L groups
//         [g i / L, (g+1) i / L), each group's count spread evenly over its
//         bins with h > 0;
//   KL_i = sum over P_i > 0 of p log(p / q), P_i and Q_i each normalized,
//          binary64; +inf where Q_i is 0 under mass of P_i.
// The smallest i with the minimal KL wins: scale = RN(RN(i * w) / 127).
// kl (optional) receives KL_i at index i, NaN below L.
__global__ __launch_bounds__(kCalThreads) void calibrate_entropy_kernel(
    const uint32_t* __restrict__ hist, int bins, const float* __restrict__ amax,
    float* __restrict__ scale_out, double* __restrict__ kl_out) {
  extern __shared__ uint32_t h[];
  __shared__ double best_kl[kCalThreads];
  __shared__ int best_i[kCalThreads];
  __shared__ double total_s;
  constexpr int L = kQuantLevels;
  for (int b = threadIdx.x; b < bins; b += kCalThreads) h[b] = hist[b];
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int b = 0; b < bins; ++b) t += (double)h[b];
    total_s = t;
  }
  if (kl_out)
    for (int i = threadIdx.x; i < L; i += kCalThreads) kl_out[i] = __builtin_nan("");
  __syncthreads();
  const double total = total_s;

  double my_kl = __builtin_inf();
  int my_i = bins + 1;
  for (int i = L + threadIdx.x; i <= bins; i += kCalThreads) {
    double kl;
    if (total == 0.0) {
      kl = 0.0;
    } else {
      double above = 0.0, below = 0.0;
      for (int j = 0; j < bins; ++j) {
        if (j < i) below += (double)h[j];
        else above += (double)h[j];
      }
      if (below == 0.0) {
        kl = __builtin_inf();
      } else {
        kl = 0.0;
        for (int g = 0; g < L && kl != __builtin_inf(); ++g) {
          const int lo = g * i / L, hi = (g + 1) * i / L;
          double seg = 0.0;
          int nz = 0;
          for (int j = lo; j < hi; ++j) {
            seg += (double)h[j];
            nz += h[j] != 0u;
          }
          const double qv = nz ? seg / nz : 0.0;
          for (int j = lo; j < hi; ++j) {
            const double p = (double)h[j] + (j == i - 1 ? above : 0.0);
            if (p == 0.0) continue;
            const double q = h[j] != 0u ? qv : 0.0;
            if (q == 0.0) {
              kl = __builtin_inf();
              break;
            }
            const double pn = p / total, qn = q / below;
            kl += pn * log(pn / qn);
          }
        }
      }
    }
    if (kl_out) kl_out[i] = kl;
    if (kl < my_kl) {          // candidates rise with i: the first minimum stays
      my_kl = kl;
      my_i = i;
    }
  }
  best_kl[threadIdx.x] = my_kl;
  best_i[threadIdx.x] = my_i;
  __syncthreads();
  for (int stride = kCalThreads / 2; stride > 0; stride >>= 1) {
    if (threadIdx.x < stride) {
      const double k2 = best_kl[threadIdx.x + stride];
      const int i2 = best_i[threadIdx.x + stride];
      if (k2 < best_kl[threadIdx.x] || (k2 == best_kl[threadIdx.x] && i2 < best_i[threadIdx.x])) {
        best_kl[threadIdx.x] = k2;
        best_i[threadIdx.x] = i2;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int i = best_i[0] <= bins ? best_i[0] : bins;
    const float w = amax[0] / (float)bins;
    const float T = (float)i * w;
    scale_out[0] = T / kQMax;
  }
}

hipError_t launch_calibrate_entropy(const uint32_t* hist, int64_t bins, const float* amax,
                                    float* scale, double* kl, hipStream_t s) {
  const size_t lds = (size_t)bins * sizeof(uint32_t);
  hipLaunchKernelGGL(calibrate_entropy_kernel, dim3(1), dim3(kCalThreads), lds, s, hist,
                     (int)bins, amax, scale, kl);
  return hipGetLastError();
}

}  // namespace w8a8
