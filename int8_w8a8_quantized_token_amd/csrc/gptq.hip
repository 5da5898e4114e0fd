// GPTQ weight quantization on gfx950: an offline alternative to per-channel
// round-to-nearest that produces the same int8 weights and per-output-channel
// scales, with the rounding errors compensated.
//
// The Red Hat article "Understanding W8A8 INT8 LLM quantization: Half the
// size, better performance, same accuracy", section "The solution: How GPTQ
// improves on naive quantization", quantizes a layer's weights one input
// column at a time and after each pushes the rounding error onto the columns
// not yet quantized, weighted through the Hessian of the calibration
// activations. With U the upper Cholesky factor of the damped inverse
// Hessian (H + lambda I)^-1 = U^T U, column j of every output row w becomes
//   q_j = clamp(round(RN32(w_j) / s)),  err = (w_j - q_j s) / U_jj,
//   w_k -= err * U_jk                   for k > j,
// one binary64 product and one difference per update. Rows are independent.
//
// Kernels:
//   * hessian: H += 2 X'^T X' (binary64), X' the smoothed calibration rows;
//   * factor: A = J (H + lambda I) J (J reverses the index order), its lower
//     Cholesky factor L (K column steps), V = L^-1 (one forward substitution
//     per column), U = J V J; then U^T U = (H + lambda I)^-1 with U upper;
//   * quantize: 64-column panels. The panel kernel runs the column loop inside
//     the panel for a block of rows; the update kernel then applies the
//     panel's 64 errors to the later columns one column at a time, in order.
//     Every weight therefore receives exactly the updates of the plain column
//     loop, in the same order and rounding, which makes the codes identical
//     to that loop's for the same U.

#include "device_common.h"
#include "launchers.h"

namespace w8a8 {

constexpr int kPanel = 64;

// ---------------------------------------------------------------------------
// Hessian: H[i][j] += 2 sum_m x'[m,i] x'[m,j]
// ---------------------------------------------------------------------------

constexpr int kHT = 64;     // output tile
constexpr int kHM = 16;     // rows of X per LDS stage

__global__ __launch_bounds__(256) void gptq_hessian_kernel(const uint16_t* __restrict__ x,
                                                           int64_t ldx,
                                                           const float* __restrict__ smooth,
                                                           int64_t n, int K,
                                                           double* __restrict__ H) {
  __shared__ double xi[kHM][kHT], xj[kHM][kHT];
  const int i0 = blockIdx.y * kHT, j0 = blockIdx.x * kHT;
  const int tid = threadIdx.x;
  const int ti = tid / 16, tj = tid % 16;        // 4 x 4 outputs per thread
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  for (int64_t m0 = 0; m0 < n; m0 += kHM) {
    for (int e = tid; e < kHM * kHT; e += 256) {
      const int r = e / kHT, c = e % kHT;
      const int64_t m = m0 + r;
      double vi = 0.0, vj = 0.0;
      if (m < n) {
        if (i0 + c < K) {
          float f = __uint_as_float((uint32_t)x[m * ldx + i0 + c] << 16);
          if (smooth) f = f / smooth[i0 + c];
          vi = (double)f;
        }
        if (j0 + c < K) {
          float f = __uint_as_float((uint32_t)x[m * ldx + j0 + c] << 16);
          if (smooth) f = f / smooth[j0 + c];
          vj = (double)f;
        }
      }
      xi[r][c] = vi;
      xj[r][c] = vj;
    }
    __syncthreads();
#pragma unroll 4
    for (int r = 0; r < kHM; ++r) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] += xi[r][ti * 4 + a] * xj[r][tj * 4 + b];
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int i = i0 + ti * 4 + a, j = j0 + tj * 4 + b;
      if (i < K && j < K) H[(int64_t)i * K + j] += 2.0 * acc[a][b];
    }
}

hipError_t launch_gptq_hessian(const uint16_t* x, int64_t ldx, const float* smooth, int64_t n,
                               int64_t K, double* H, hipStream_t s) {
  const dim3 grid((unsigned)((K + kHT - 1) / kHT), (unsigned)((K + kHT - 1) / kHT));
  hipLaunchKernelGGL(gptq_hessian_kernel, grid, dim3(256), 0, s, x, ldx, smooth, n, (int)K, H);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Factor of the damped inverse Hessian
// ---------------------------------------------------------------------------

// lambda = damp * mean(d), d the diagonal with zeros replaced by 1.
__global__ __launch_bounds__(1024) void gptq_damping_kernel(const double* __restrict__ H, int K,
                                                            double damp,
                                                            double* __restrict__ lambda) {
  __shared__ double red[1024 / kWave];
  double sum = 0.0;
  for (int i = threadIdx.x; i < K; i += 1024) {
    const double d = H[(int64_t)i * K + i];
    sum += d == 0.0 ? 1.0 : d;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int w = 0; w < 1024 / kWave; ++w) t += red[w];
    lambda[0] = damp * (t / (double)K);
  }
}

// A[i][j] = Hd[K-1-i][K-1-j], Hd = H with zero diagonal entries set to 1,
// plus lambda on the diagonal.
__global__ __launch_bounds__(256) void gptq_reverse_kernel(const double* __restrict__ H, int K,
                                                           const double* __restrict__ lambda,
                                                           double* __restrict__ A) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)K * K) return;
  const int i = (int)(e / K), j = (int)(e % K);
  double v = H[(int64_t)(K - 1 - i) * K + (K - 1 - j)];
  if (i == j) v = (v == 0.0 ? 1.0 : v) + lambda[0];
  A[e] = v;
}

// Cholesky column step j: A[i][j] /= sqrt(A[j][j]) for i > j. Every thread
// reads the pivot; it is replaced by its square root only in the next launch
// (the trailing update, which never reads it), or here when no row is below.
__global__ __launch_bounds__(256) void chol_column_kernel(double* __restrict__ A, int K, int j) {
  const double d = sqrt(A[(int64_t)j * K + j]);
  const int i = j + 1 + blockIdx.x * 256 + threadIdx.x;
  if (i < K) A[(int64_t)i * K + j] /= d;
  if (j == K - 1 && threadIdx.x == 0) A[(int64_t)j * K + j] = d;
}

// Trailing update of step j: A[i][k] -= A[i][j] A[k][j] for j < k <= i, and
// the pivot A[j][j] becomes its square root.
__global__ __launch_bounds__(256) void chol_update_kernel(double* __restrict__ A, int K, int j) {
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
    A[(int64_t)j * K + j] = sqrt(A[(int64_t)j * K + j]);
  const int k = j + 1 + blockIdx.x * 256 + threadIdx.x;
  const int i = j + 1 + blockIdx.y;
  if (k > i || i >= K) return;
  const double t = A[(int64_t)i * K + j] * A[(int64_t)k * K + j];
  A[(int64_t)i * K + k] = A[(int64_t)i * K + k] - t;
}

// V = L^-1, one lower-triangular column per thread: V[c][c] = 1 / L[c][c],
// V[i][c] = -(sum_{k=c}^{i-1} L[i][k] V[k][c]) / L[i][i].
__global__ __launch_bounds__(64) void tri_inverse_kernel(const double* __restrict__ L, int K,
                                                         double* __restrict__ V) {
  const int c = blockIdx.x * 64 + threadIdx.x;
  if (c >= K) return;
  for (int i = 0; i < c; ++i) V[(int64_t)i * K + c] = 0.0;
  V[(int64_t)c * K + c] = 1.0 / L[(int64_t)c * K + c];
  for (int i = c + 1; i < K; ++i) {
    double s = 0.0;
    for (int k = c; k < i; ++k) s += L[(int64_t)i * K + k] * V[(int64_t)k * K + c];
    V[(int64_t)i * K + c] = -s / L[(int64_t)i * K + i];
  }
}

// U[i][j] = V[K-1-i][K-1-j]: lower becomes upper.
__global__ __launch_bounds__(256) void gptq_unreverse_kernel(const double* __restrict__ V, int K,
                                                             double* __restrict__ U) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)K * K) return;
  const int i = (int)(e / K), j = (int)(e % K);
  U[e] = V[(int64_t)(K - 1 - i) * K + (K - 1 - j)];
}

hipError_t launch_gptq_factor(const double* H, int64_t K, double damp, double* U, double* work,
                              hipStream_t s) {
  // work: A [K*K], then lambda [1]
  double* A = work;
  double* lambda = work + K * K;
  const int k = (int)K;
  const unsigned n2 = (unsigned)((K * K + 255) / 256);
  hipLaunchKernelGGL(gptq_damping_kernel, dim3(1), dim3(1024), 0, s, H, k, damp, lambda);
  hipLaunchKernelGGL(gptq_reverse_kernel, dim3(n2), dim3(256), 0, s, H, k, lambda, A);
  for (int j = 0; j < k; ++j) {
    const int rest = k - j - 1;
    hipLaunchKernelGGL(chol_column_kernel, dim3((unsigned)(rest / 256 + 1)), dim3(256), 0, s, A, k,
                       j);
    if (rest > 0)
      hipLaunchKernelGGL(chol_update_kernel, dim3((unsigned)((rest + 255) / 256), (unsigned)rest),
                         dim3(256), 0, s, A, k, j);
  }
  // V = L^-1 into U's storage, then U = J V J back into A's storage, copied over
  hipLaunchKernelGGL(tri_inverse_kernel, dim3((unsigned)((K + 63) / 64)), dim3(64), 0, s, A, k, U);
  hipLaunchKernelGGL(gptq_unreverse_kernel, dim3(n2), dim3(256), 0, s, U, k, A);
  return hipMemcpyAsync(U, A, (size_t)(K * K) * sizeof(double), hipMemcpyDeviceToDevice, s);
}

// ---------------------------------------------------------------------------
// Quantization with error feedback
// ---------------------------------------------------------------------------

// Per output row: W' = bf16(w * smooth) (as the RTN weight quantizer), kept in
// binary64, and the RTN scale max|W'| / 127.
__global__ __launch_bounds__(256) void gptq_init_kernel(const uint16_t* __restrict__ w,
                                                        int64_t ldw,
                                                        const float* __restrict__ smooth, int K,
                                                        double* __restrict__ Wf,
                                                        float* __restrict__ s_chan) {
  __shared__ float red[256 / kWave];
  const int64_t n = blockIdx.x;
  float m = 0.0f;
  for (int k = threadIdx.x; k < K; k += 256) {
    float v = __uint_as_float((uint32_t)w[n * ldw + k] << 16);
    if (smooth) v = __uint_as_float(f32_to_bf16_rne(v * smooth[k]) << 16);
    Wf[n * K + k] = (double)v;
    m = fmaxf(m, fabsf(v));
  }
  m = wave_max(m);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
    for (int i = 1; i < 256 / kWave; ++i) r = fmaxf(r, red[i]);
    s_chan[n] = r / kQMax;
  }
}

// Panel [p0, p0 + pw), pw <= 64: one thread per output row runs the column
// loop inside the panel. The rows' panel values sit in LDS column by column
// (thread t's weight of column k at wl[k][t], so a wave's accesses are
// consecutive), U's panel block beside them; codes go to wq, errors to Err.
__global__ __launch_bounds__(64) void gptq_panel_kernel(double* __restrict__ Wf, int K,
                                                        const double* __restrict__ U, int p0,
                                                        int pw, const float* __restrict__ s_chan,
                                                        int N, int8_t* __restrict__ wq,
                                                        int64_t ldwq, double* __restrict__ Err) {
  __shared__ double ub[kPanel][kPanel];
  __shared__ double wl[kPanel][64];
  for (int e = threadIdx.x; e < kPanel * kPanel; e += 64) {
    const int a = e / kPanel, b = e % kPanel;
    ub[a][b] = (a < pw && b < pw) ? U[(int64_t)(p0 + a) * K + p0 + b] : 0.0;
  }
  const int t = threadIdx.x;
  const int n = blockIdx.x * 64 + t;
  const bool live = n < N;
  for (int c = 0; c < pw; ++c) wl[c][t] = live ? Wf[(int64_t)n * K + p0 + c] : 0.0;
  __syncthreads();
  if (!live) return;
  const float s = s_chan[n];
  const double s64 = (double)s;
  for (int j = 0; j < pw; ++j) {
    const double wj = wl[j][t];
    const float wf = (float)wj;
    const int q = (s == 0.0f) ? 0 : int8_code(wf / s);
    wq[(int64_t)n * ldwq + p0 + j] = (int8_t)q;
    const double err = (wj - (double)q * s64) / ub[j][j];
    Err[(int64_t)n * kPanel + j] = err;
    for (int k = j + 1; k < pw; ++k) {
      const double tt = err * ub[j][k];
      wl[k][t] = wl[k][t] - tt;
    }
  }
}

// Columns after the panel: W[n][k] -= Err[n][j] * U[p0 + j][k] for j in panel
// order. A workgroup covers 16 rows x 256 columns, one column per thread.
__global__ __launch_bounds__(256) void gptq_update_kernel(double* __restrict__ Wf, int K,
                                                         const double* __restrict__ U, int p0,
                                                         int pw, int N,
                                                         const double* __restrict__ Err) {
  __shared__ double eb[16][kPanel];
  const int n0 = blockIdx.y * 16;
  for (int e = threadIdx.x; e < 16 * kPanel; e += 256) {
    const int r = e / kPanel, c = e % kPanel;
    eb[r][c] = (n0 + r < N && c < pw) ? Err[(int64_t)(n0 + r) * kPanel + c] : 0.0;
  }
  __syncthreads();
  const int k = p0 + pw + blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  double wr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) wr[r] = n0 + r < N ? Wf[(int64_t)(n0 + r) * K + k] : 0.0;
  for (int j = 0; j < pw; ++j) {
    const double u = U[(int64_t)(p0 + j) * K + k];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const double t = eb[r][j] * u;
      wr[r] = wr[r] - t;
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (n0 + r < N) Wf[(int64_t)(n0 + r) * K + k] = wr[r];
}

hipError_t launch_gptq_quantize(const uint16_t* w, int64_t ldw, const float* smooth,
                                const double* U, int64_t N, int64_t K, int8_t* wq, int64_t ldwq,
                                float* s_chan, double* Wf, double* Err, hipStream_t s) {
  const int n = (int)N, k = (int)K;
  hipLaunchKernelGGL(gptq_init_kernel, dim3((unsigned)N), dim3(256), 0, s, w, ldw, smooth, k, Wf,
                     s_chan);
  for (int p0 = 0; p0 < k; p0 += kPanel) {
    const int pw = k - p0 < kPanel ? k - p0 : kPanel;
    hipLaunchKernelGGL(gptq_panel_kernel, dim3((unsigned)((N + 63) / 64)), dim3(64), 0, s, Wf, k,
                       U, p0, pw, s_chan, n, wq, ldwq, Err);
    const int rest = k - p0 - pw;
    if (rest > 0)
      hipLaunchKernelGGL(gptq_update_kernel,
                         dim3((unsigned)((rest + 255) / 256), (unsigned)((N + 15) / 16)),
                         dim3(256), 0, s, Wf, k, U, p0, pw, n, Err);
  }
  return hipGetLastError();
}

}  // namespace w8a8
