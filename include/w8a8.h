/*
 * w8a8.h -- C ABI of the MI355X (gfx950) W8A8 INT8 linear layer.
 *
 * The layer is the one the Red Hat articles "Understanding W8A8 INT8 LLM
 * quantization: Half the size, better performance, same accuracy" (part 1)
 * and "... Accuracy and performance results" (part 2) describe: activations
 * are quantized per token at run time, multiplied as int8 against int8
 * weights that carry one scale per output channel, and the int32 result is
 * converted back to bf16.
 *
 * Conventions for every entry point below
 *   - Data pointers are DEVICE pointers on the current HIP device unless a
 *     parameter says otherwise. bf16 tensors are passed as raw 16-bit words
 *     (uint16_t). Scales and smoothing factors are IEEE binary32.
 *   - Matrices are row-major with the last dimension contiguous; ld* is the
 *     distance between consecutive rows, in elements.
 *       X, Xq : [M, K]   tokens x input channels
 *       W, Wq : [N, K]   output channels x input channels
 *       Y, acc: [M, N]
 *   - Every call is enqueued on `stream` (0 = the null stream) and returns
 *     before the GPU work completes. The caller owns all memory; inputs and
 *     outputs must stay valid until the stream reaches the call. The library
 *     never allocates device memory; the only state it keeps between calls
 *     is each device's compute-unit count, read once for tile choices, and
 *     each device's address of the fixed workspace array that
 *     w8a8_linear_noalloc uses (8 MiB per device, held until the process
 *     ends).
 *   - Arguments are validated on the host before any HIP call. A failed
 *     check returns an error status and enqueues nothing. Device faults
 *     surface at the caller's next synchronization, as for any HIP kernel.
 *   - No C++ exception crosses this interface.
 *   - M == 0 or N == 0 is a valid empty call: W8A8_SUCCESS, nothing launched.
 *   - Activation, weight and scale values are finite; a non-finite input
 *     value gives unspecified codes, scales and outputs (never a fault).
 *   - Requirements shared by the entry points that read int8/bf16 rows:
 *       K % 16 == 0, 0 < K <= 131072 (so |acc| <= 128*128*K stays in int32);
 *       pointers to K-long rows (x, xq, w, wq) 16-byte aligned, with
 *       ld * element_size a multiple of 16. Outputs with N columns (y, acc)
 *       need only element alignment and any ld >= N.
 *     Violations give W8A8_ERROR_UNSUPPORTED (K) or W8A8_ERROR_MISALIGNED.
 *   - Token and output-channel counts (M, N, and the rows of the quantizers
 *     and producers) are at most 2^22 - 1, and M * N at most 2^37; the
 *     calibration reductions and the residual add take up to 2^31 - 65536
 *     rows; GPTQ takes at most 2^19 output channels. Larger sizes give
 *     W8A8_ERROR_UNSUPPORTED.
 *   - Thread-safe: calls on different streams may run concurrently.
 */
#ifndef W8A8_H
#define W8A8_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W8A8_ABI_VERSION 1

typedef enum {
  W8A8_SUCCESS = 0,
  W8A8_ERROR_INVALID_VALUE = 1, /* NULL required pointer, negative size, ld too small */
  W8A8_ERROR_MISALIGNED = 2,    /* pointer or row stride below required alignment   */
  W8A8_ERROR_UNSUPPORTED = 3,   /* K % 16 != 0, K > 131072, size past the limits  */
  W8A8_ERROR_WORKSPACE = 4,     /* workspace NULL or smaller than required          */
  W8A8_ERROR_HIP = 5            /* the HIP runtime rejected a kernel launch         */
} w8a8_status_t;

/* Static, NUL-terminated description of a status code (any int: values
 * that are not a w8a8_status_t give "unknown status"). Never NULL. */
const char* w8a8_status_string(int status);

/* W8A8_ABI_VERSION of the loaded library. */
int w8a8_abi_version(void);

/*
 * Per-token dynamic activation quantization (smooth, scale, round, clamp).
 *   x'[m,k]  = x[m,k] / smooth[k]                (binary32 division; skipped
 *                                                  when smooth == NULL)
 *   s_tok[m] = max_k |x'[m,k]| / 127              (binary32)
 *   xq[m,k]  = clamp(round(x'[m,k] / s_tok[m]), -127, 127), round half away
 *              from zero; a row whose absmax is 0 gets s_tok = 0, xq = 0.
 * Cited: part 1, "Why activation quantization is hard, and how SmoothQuant
 * fixes it" (one scale per token across its channels, computed at run time)
 * and "How SmoothQuant prevents outliers in activation tensors" (the
 * smoothing division and the rounding of the worked example); part 2,
 * "Inter-token latency (ITL)" (measure range, compute scale, convert).
 *   x      [M, K] bf16, row stride ldx >= K          (read)
 *   smooth [K] fp32, every entry finite and > 0, or NULL (read)
 *   xq     [M, K] int8, row stride ldq >= K          (written)
 *   s_tok  [M] fp32                                  (written)
 */
w8a8_status_t w8a8_quantize_act(const uint16_t* x, int64_t ldx, const float* smooth,
                                int64_t M, int64_t K, int8_t* xq, int64_t ldq,
                                float* s_tok, hipStream_t stream);

/*
 * Int8 GEMM with the dequantizing epilogue.
 *   acc[m,n] = sum_k xq[m,k] * wq[n,k]              (exact int32)
 *   y[m,n]   = bf16_rne((float(acc) * s_tok[m]) * s_chan[n])
 * Cited: part 1, "How we compressed the model" (int8 x int8 matrix multiply
 * on int8 matrix units) and "Why activation quantization is hard" (the
 * per-token scale factors out of the channel sum and is applied after it);
 * part 2, "Inter-token latency (ITL)" (convert back to bf16).
 * With K % 128 == 0, decode sizes and batches up to about a thousand
 * tokens take the LDS-staged kernel (token tiles of up to 64 rows), larger
 * M the MFMA prefill kernel, whose tile shape the launcher picks from M, N
 * and the CU count; other K take register- or LDS-staged kernels by M. All
 * give identical results.
 *   xq [M, K] int8, ldq >= K;  s_tok [M] fp32          (read)
 *   wq [N, K] int8, ldw >= K;  s_chan [N] fp32         (read)
 *   y  [M, N] bf16, ldy >= N                           (written)
 */
w8a8_status_t w8a8_gemm(const int8_t* xq, int64_t ldq, const float* s_tok,
                        const int8_t* wq, int64_t ldw, const float* s_chan,
                        int64_t M, int64_t N, int64_t K,
                        uint16_t* y, int64_t ldy, hipStream_t stream);

/*
 * The same GEMM kernels with an int32 epilogue: acc[m,n] = sum_k xq*wq.
 * Exposes the accumulators for bit-exact checks. ldc >= N, acc 4-byte
 * aligned.
 */
w8a8_status_t w8a8_gemm_i32(const int8_t* xq, int64_t ldq,
                            const int8_t* wq, int64_t ldw,
                            int64_t M, int64_t N, int64_t K,
                            int32_t* acc, int64_t ldc, hipStream_t stream);

/*
 * Bytes of workspace w8a8_linear needs for M tokens and K input channels:
 * xq [M, K] int8 followed by s_tok [M] fp32, each 256-byte aligned.
 * Returns 0 for M <= 0 or K <= 0.
 */
size_t w8a8_linear_workspace_bytes(int64_t M, int64_t K);

/*
 * The whole linear: w8a8_quantize_act into the workspace, then w8a8_gemm,
 * in stream order. One quantize-dequantize cycle per call, as part 2,
 * "Inter-token latency (ITL)" counts them per layer and request. For
 * M <= 2, N < 16384, K % 128 == 0 and K <= 4096 both steps run in one
 * kernel launch (every workgroup quantizes the rows itself) and the
 * workspace is not touched; y is the same either way.
 *   x [M, K] bf16, ldx >= K; smooth [K] or NULL         (read)
 *   wq [N, K] int8, ldw >= K; s_chan [N]                (read)
 *   y [M, N] bf16, ldy >= N                             (written)
 *   workspace: device memory of at least
 *              w8a8_linear_workspace_bytes(M, K) bytes, 256-byte aligned;
 *              contents afterwards unspecified; must not be shared by
 *              calls that may overlap.
 */
w8a8_status_t w8a8_linear(const uint16_t* x, int64_t ldx, const float* smooth,
                          const int8_t* wq, int64_t ldw, const float* s_chan,
                          int64_t M, int64_t N, int64_t K,
                          uint16_t* y, int64_t ldy,
                          void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * w8a8_linear for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and results, with the workspace taken from one fixed
 * device array inside the library instead of a caller buffer. The call
 * itself allocates nothing.
 *   Same arguments as w8a8_linear without the workspace.
 *   Limit: w8a8_linear_workspace_bytes(M, K) <= W8A8_NOALLOC_MAX_BYTES
 *   (8 MiB: M * K up to about 8.3 million, e.g. 64 tokens at K = 131072 or
 *   2048 tokens at K = 4096); larger sizes return W8A8_ERROR_WORKSPACE and
 *   enqueue nothing. Each device holds its own 8 MiB array until the
 *   process ends; its address is looked up on the first call on a device
 *   (W8A8_ERROR_HIP if that fails).
 *   Every call on a device uses that device's one array: calls that may
 *   overlap on one device (different streams, or another thread's calls)
 *   race and must be serialized by the caller. Nothing in the array needs
 *   to start at zero; each call overwrites what it reads.
 */
#define W8A8_NOALLOC_MAX_BYTES (8u << 20)
w8a8_status_t w8a8_linear_noalloc(const uint16_t* x, int64_t ldx, const float* smooth,
                                  const int8_t* wq, int64_t ldw, const float* s_chan,
                                  int64_t M, int64_t N, int64_t K,
                                  uint16_t* y, int64_t ldy, hipStream_t stream);

/* ----------------------------------------------------------------------- *
 * Offline preparation (calibration and weight quantization). These run
 * once per model, not per token, but use the same arithmetic on the GPU.
 * ----------------------------------------------------------------------- */

/*
 * Per-channel absolute maximum over rows, accumulated:
 *   absmax[k] = max(absmax[k], max_r |a[r,k]|)
 * Used on calibration activations (rows = tokens; call once per batch) and
 * on weights (rows = output channels: the page's "row j of the receiving
 * layer's weight" in its K x N layout). Cited: part 1, "How the SmoothQuant
 * smoothing factor is computed".
 *   a [rows, K] bf16, lda >= K (read);  absmax [K] fp32, >= 0 (read+written;
 *   zero it before the first batch). K % 8 == 0 suffices here.
 */
w8a8_status_t w8a8_channel_absmax(const uint16_t* a, int64_t lda, int64_t rows,
                                  int64_t K, float* absmax, hipStream_t stream);

/*
 * SmoothQuant factors with migration strength 1/2:
 *   smooth[k] = sqrt(act_absmax[k] / w_absmax[k])   (binary32 division and
 *               square root, correctly rounded); 1 where either input is 0.
 * Cited: part 1, "How the SmoothQuant smoothing factor is computed" (terms
 * of the factor; the article's own run uses strength 0.8).
 *   act_absmax, w_absmax [K] fp32 (read); smooth [K] fp32 (written). Any K >= 0.
 */
w8a8_status_t w8a8_smoothing_factors(const float* act_absmax, const float* w_absmax,
                                     int64_t K, float* smooth, hipStream_t stream);

/*
 * Smooth and quantize a weight per output channel (symmetric round to nearest):
 *   w'[n,k]   = bf16_rne(float(w[n,k]) * smooth[k])    (smooth == NULL: w' = w)
 *   s_chan[n] = max_k |w'[n,k]| / 127
 *   wq[n,k]   = clamp(round(w'[n,k] / s_chan[n]), -127, 127), half away from 0
 * Cited: part 1, "The problem with naive quantization" (one scale per weight
 * channel) and "How the SmoothQuant smoothing factor is computed" (weights
 * scaled up by the factor, still bf16, before quantization).
 *   w [N, K] bf16, ldw >= K; smooth [K] or NULL (read)
 *   wq [N, K] int8, ldwq >= K; s_chan [N] fp32  (written)
 */
w8a8_status_t w8a8_quantize_weight(const uint16_t* w, int64_t ldw, const float* smooth,
                                   int64_t N, int64_t K, int8_t* wq, int64_t ldwq,
                                   float* s_chan, hipStream_t stream);

/* ----------------------------------------------------------------------- *
 * Static per-tensor activation scale. The article "INT8 Post-Training
 * Quantization for LLM Inference on NVIDIA GPUs", section "The Heart of PTQ:
 * Entropy-Based Calibration", fixes one activation scale per tensor ahead of
 * time (min-max or entropy calibration) instead of one per token at run
 * time. The run-time step then needs no reduction and the clamp binds for
 * values beyond the calibrated threshold.
 * ----------------------------------------------------------------------- */

#define W8A8_HIST_BINS 2048    /* default histogram size for entropy calibration */
#define W8A8_QUANT_LEVELS 128  /* code magnitudes 0..127; smallest candidate threshold */

/*
 * Quantization with one fixed scale S = scale[0] for every token:
 *   x'[m,k] = x[m,k] / smooth[k] (binary32 division; skipped when NULL)
 *   xq[m,k] = clamp(round(x'[m,k] / S), -127, 127), round half away from 0
 *   s_tok[m] = S for every row (so that w8a8_gemm applies it)
 * S == 0 gives all-zero codes. Cited: "1. Min-Max Calibration" (S = T / 127,
 * symmetric range) in the calibration section above.
 *   x [M, K] bf16, ldx >= K; smooth [K] or NULL; scale [1] fp32, finite,
 *   >= 0 (device memory, read)
 *   xq [M, K] int8, ldq >= K; s_tok [M] fp32 (written)
 */
w8a8_status_t w8a8_quantize_act_static(const uint16_t* x, int64_t ldx, const float* smooth,
                                       const float* scale, int64_t M, int64_t K, int8_t* xq,
                                       int64_t ldq, float* s_tok, hipStream_t stream);

/*
 * w8a8_linear with the static scale: w8a8_quantize_act_static into the
 * workspace (same layout and size as w8a8_linear's), then w8a8_gemm; in one
 * launch under the same conditions as w8a8_linear's.
 */
w8a8_status_t w8a8_linear_static(const uint16_t* x, int64_t ldx, const float* smooth,
                                 const float* scale, const int8_t* wq, int64_t ldw,
                                 const float* s_chan, int64_t M, int64_t N, int64_t K,
                                 uint16_t* y, int64_t ldy, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * Min-max calibration ("1. Min-Max Calibration"):
 *   amax[0]  = max_k act_absmax[k] / smooth[k]   (binary32 division; the
 *              largest |x'| seen, since rounding is monotone)
 *   scale[0] = amax[0] / 127
 *   act_absmax [K] fp32 from w8a8_channel_absmax over the calibration
 *   tokens; smooth [K] or NULL (read). amax, scale [1] fp32 (written). K > 0.
 */
w8a8_status_t w8a8_calibrate_minmax(const float* act_absmax, const float* smooth, int64_t K,
                                    float* amax, float* scale, hipStream_t stream);

/*
 * Histogram of |x'| for entropy calibration ("2. Entropy Calibration"):
 *   w = amax[0] / bins; bin = floor(min(|x'| / w, bins - 1)) (binary32;
 *   values at or past amax land in the last bin; w == 0 puts all in bin 0)
 *   hist[bin] += 1, accumulated across calls (zero it before the first batch).
 *   x [rows, K] bf16, ldx >= K, K % 8 == 0; smooth [K] or NULL; amax [1] fp32
 *   (e.g. from w8a8_calibrate_minmax) (read). hist [bins] uint32 (read and
 *   written). 128 <= bins <= 8192. Counts wrap past 2^32 - 1 per bin.
 */
w8a8_status_t w8a8_activation_histogram(const uint16_t* x, int64_t ldx, const float* smooth,
                                        int64_t rows, int64_t K, const float* amax, int64_t bins,
                                        uint32_t* hist, hipStream_t stream);

/*
 * Entropy calibration ("2. Entropy Calibration: Minimizing Information
 * Loss"): for every candidate threshold T_i = i * w, i = 128 .. bins,
 *   P_i = hist[0..i) with the counts past T_i added to bin i-1 (saturation),
 *   Q_i = hist[0..i) merged into 128 groups [g*i/128, (g+1)*i/128) and each
 *         group's count spread evenly over its nonzero bins,
 *   KL_i = sum over P_i > 0 of p log(p / q) (each normalized; binary64;
 *          +inf where Q_i is 0 under mass of P_i);
 * the smallest i with the least KL gives scale[0] = (i * w) / 127
 * (binary32, w = amax[0] / bins).
 *   hist [bins] uint32, amax [1] fp32 (read); scale [1] fp32 (written);
 *   kl [bins + 1] fp64 or NULL (written: KL_i at index i, NaN below 128).
 *   128 <= bins <= 8192. One workgroup: an offline step, not a hot one.
 */
w8a8_status_t w8a8_calibrate_entropy(const uint32_t* hist, int64_t bins, const float* amax,
                                     float* scale, double* kl, hipStream_t stream);

/* ----------------------------------------------------------------------- *
 * Fused producers. Part 1, section "How SmoothQuant prevents outliers in
 * activation tensors", locates the outliers in RMSNorm's weight, and "How
 * the SmoothQuant smoothing factor is computed" folds the smoothing division
 * into that weight; the ops that feed a block's linears can therefore end in
 * the quantizer and emit codes and per-token scales directly, with no bf16
 * activation written and read back.
 * ----------------------------------------------------------------------- */

/*
 * Optional residual add, RMSNorm with a folded weight, per-token quantization:
 *   if residual: h[m,k] = bf16(h[m,k] + residual[m,k])   (binary32 sum; h written)
 *   ms[m]  = sum_k h[m,k]^2 / K: the exact mean, rounded once to binary32
 *   inv[m] = 1 / sqrt(ms[m] + eps)                         (binary32 steps)
 *   y[m,k] = (h[m,k] * inv[m]) * gamma[k]                  (binary32)
 *   s_tok[m] = max_k |y[m,k]| / 127; xq = clamp(round(y / s_tok), -127, 127)
 * gamma is the norm weight divided by the next linear's smoothing factor
 * (w8a8_fold_gamma).
 *   h [M, K] bf16, ldh >= K (read; written when residual != NULL);
 *   residual [M, K] bf16 or NULL; gamma [K] fp32; eps >= 0 (read)
 *   xq [M, K] int8, ldq >= K; s_tok [M] fp32 (written). K <= 65536.
 */
w8a8_status_t w8a8_rmsnorm_quantize(uint16_t* h, int64_t ldh, const uint16_t* residual,
                                    int64_t ldr, const float* gamma, float eps, int64_t M,
                                    int64_t K, int8_t* xq, int64_t ldq, float* s_tok,
                                    hipStream_t stream);

/*
 * SiLU-gated product and per-token quantization of a gate|up row:
 *   m[m,k]  = bf16((g / (1 + exp(-g))) * u), g = gu[m,k], u = gu[m,I+k],
 *             evaluated in binary64 and rounded once
 *   x'[m,k] = m[m,k] / smooth[k] (binary32; skipped when NULL)
 *   s_tok[m] = max_k |x'[m,k]| / 127; xq = clamp(round(x' / s_tok), -127, 127)
 *   gu [M, 2I] bf16, ldgu >= 2I (read); smooth [I] or NULL (read)
 *   xq [M, I] int8, ldq >= I; s_tok [M] fp32 (written). I % 16 == 0, I <= 65536.
 */
w8a8_status_t w8a8_silu_mul_quantize(const uint16_t* gu, int64_t ldgu, const float* smooth,
                                     int64_t M, int64_t I, int8_t* xq, int64_t ldq, float* s_tok,
                                     hipStream_t stream);

/* g[k] = gamma[k] / smooth[k] (binary32 division; g = gamma when smooth is NULL). */
w8a8_status_t w8a8_fold_gamma(const float* gamma, const float* smooth, int64_t K, float* g,
                              hipStream_t stream);

/* h[m,k] = bf16(h[m,k] + r[m,k]) (binary32 sum of bf16 values). K % 8 == 0. */
w8a8_status_t w8a8_residual_add(uint16_t* h, int64_t ldh, const uint16_t* r, int64_t ldr,
                                int64_t M, int64_t K, hipStream_t stream);

/* ----------------------------------------------------------------------- *
 * GPTQ weight quantization (offline). Part 1, section "The solution: How
 * GPTQ improves on naive quantization": quantize one input column at a time
 * and push each rounding error onto the columns not yet quantized, weighted
 * by the Hessian of the calibration activations. Produces the same Wq and
 * per-output-channel scales as w8a8_quantize_weight (the scales are equal;
 * the codes differ where errors were compensated).
 * ----------------------------------------------------------------------- */

/*
 * H[i,j] += 2 sum_m x'[m,i] x'[m,j], x' = x / smooth (binary32, then binary64).
 *   x [n, K] bf16, ldx >= K; smooth [K] or NULL (read);
 *   H [K, K] fp64 row-major, dense (read and written; zero it first).
 *   K % 16 == 0, K <= 32768.
 */
w8a8_status_t w8a8_gptq_hessian(const uint16_t* x, int64_t ldx, const float* smooth, int64_t n,
                                int64_t K, double* H, hipStream_t stream);

/* Workspace for w8a8_gptq_factor: K*K + 1 doubles, 256-byte aligned size. */
size_t w8a8_gptq_factor_workspace_bytes(int64_t K);

/*
 * U, upper triangular, with U^T U = (Hd + lambda I)^-1, where Hd is H with
 * zero diagonal entries set to 1 and lambda = damp * mean(diag Hd) (damp
 * 0.01 is customary). Computed as U = J inv(chol(J (Hd + lambda I) J)) J
 * (J reverses the index order), in binary64.
 *   H [K, K] fp64 (read); U [K, K] fp64 (written); workspace as sized above.
 */
w8a8_status_t w8a8_gptq_factor(const double* H, int64_t K, double damp, double* U,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace for w8a8_gptq_quantize: N*K + 64*N doubles (256-byte aligned parts). */
size_t w8a8_gptq_quantize_workspace_bytes(int64_t N, int64_t K);

/*
 * GPTQ codes of w [N, K]: W' = bf16(w * smooth) as in w8a8_quantize_weight,
 * s_chan[n] = max_k |W'[n,k]| / 127, then for columns j = 0 .. K-1 of every
 * row: q = clamp(round(RN32(W'[n,j]) / s_chan[n]), -127, 127) (binary32,
 * half away), err = (W'[n,j] - q s_chan[n]) / U[j,j], and
 * W'[n,k] -= err * U[j,k] for k > j (binary64 product, then difference).
 *   w [N, K] bf16, ldw >= K; smooth [K] or NULL; U [K, K] fp64 (read)
 *   wq [N, K] int8, ldwq >= K; s_chan [N] fp32 (written)
 */
w8a8_status_t w8a8_gptq_quantize(const uint16_t* w, int64_t ldw, const float* smooth,
                                 const double* U, int64_t N, int64_t K, int8_t* wq, int64_t ldwq,
                                 float* s_chan, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
