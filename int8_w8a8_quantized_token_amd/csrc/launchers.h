// Host-side launchers of the gfx950 kernels. Arguments are already
// validated by the C-ABI layer (api.hip); each launcher only enqueues.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

// Per-row quantization of bf16 rows: activations (x / smooth) or weights
// (bf16(w * smooth)). Writes int8 codes and one binary32 scale per row.
enum class RowMode { kActivation = 0, kWeight = 1 };

hipError_t launch_quantize_rows(RowMode mode, const uint16_t* x, int64_t ldx,
                                const float* smooth, int64_t rows, int64_t K,
                                int8_t* q, int64_t ldq, float* scale, hipStream_t s);

hipError_t launch_channel_absmax(const uint16_t* a, int64_t lda, int64_t rows, int64_t K,
                                 float* absmax, hipStream_t s);

hipError_t launch_smoothing_factors(const float* ax, const float* aw, int64_t K,
                                    float* smooth, hipStream_t s);

// GEMM with either the bf16 dequantizing epilogue (y != nullptr) or the
// int32 accumulator epilogue (acc != nullptr).
hipError_t launch_gemm(const int8_t* xq, int64_t ldq, const float* s_tok,
                       const int8_t* wq, int64_t ldw, const float* s_chan,
                       int64_t M, int64_t N, int64_t K,
                       uint16_t* y, int64_t ldy, int32_t* acc, int64_t ldc,
                       hipStream_t s);

// The whole linear (quantize, GEMM, epilogue) in one launch for
// M <= kLinearFusedMaxM tokens, N < kLinearFusedMaxN, K % 128 == 0 and
// K <= kLinearFusedMaxK (linear_fused.hip); dynamic per-token or one static
// scale. Same results as quantize + GEMM.
constexpr int64_t kLinearFusedMaxM = 2;
constexpr int64_t kLinearFusedMaxN = 16384;
constexpr int64_t kLinearFusedMaxK = 4096;
bool linear_fused_supported(int64_t M, int64_t N, int64_t K);
hipError_t launch_linear_fused(const uint16_t* x, int64_t ldx, const float* smooth,
                               const int8_t* wq, int64_t ldw, const float* s_chan, int64_t M,
                               int64_t N, int64_t K, uint16_t* y, int64_t ldy, hipStream_t s);
hipError_t launch_linear_fused_static(const uint16_t* x, int64_t ldx, const float* smooth,
                                      const float* scale, const int8_t* wq, int64_t ldw,
                                      const float* s_chan, int64_t M, int64_t N, int64_t K,
                                      uint16_t* y, int64_t ldy, hipStream_t s);

// Static per-tensor scale: quantizer and calibration (static_scale.hip).
hipError_t launch_quantize_static(const uint16_t* x, int64_t ldx, const float* smooth,
                                  const float* scale, int64_t M, int64_t K, int8_t* q,
                                  int64_t ldq, float* s_tok, hipStream_t s);

hipError_t launch_calibrate_minmax(const float* act_absmax, const float* smooth, int64_t K,
                                   float* amax, float* scale, hipStream_t s);

hipError_t launch_abs_histogram(const uint16_t* x, int64_t ldx, const float* smooth, int64_t rows,
                                int64_t K, const float* amax, int64_t bins, uint32_t* hist,
                                hipStream_t s);

hipError_t launch_calibrate_entropy(const uint32_t* hist, int64_t bins, const float* amax,
                                    float* scale, double* kl, hipStream_t s);

// Fused producers (producers.hip).
hipError_t launch_rmsnorm_quantize(uint16_t* h, int64_t ldh, const uint16_t* residual,
                                   int64_t ldr, const float* g, float eps, int64_t M, int64_t K,
                                   int8_t* q, int64_t ldq, float* s_tok, hipStream_t s);

hipError_t launch_silu_mul_quantize(const uint16_t* gu, int64_t ldgu, const float* smooth,
                                    int64_t M, int64_t I, int8_t* q, int64_t ldq, float* s_tok,
                                    hipStream_t s);

hipError_t launch_fold_gamma(const float* gamma, const float* smooth, int64_t K, float* g,
                             hipStream_t s);

hipError_t launch_residual_add(uint16_t* h, int64_t ldh, const uint16_t* r, int64_t ldr,
                               int64_t M, int64_t K, hipStream_t s);

// GPTQ (gptq.hip).
hipError_t launch_gptq_hessian(const uint16_t* x, int64_t ldx, const float* smooth, int64_t n,
                               int64_t K, double* H, hipStream_t s);

hipError_t launch_gptq_factor(const double* H, int64_t K, double damp, double* U, double* work,
                              hipStream_t s);

hipError_t launch_gptq_quantize(const uint16_t* w, int64_t ldw, const float* smooth,
                                const double* U, int64_t N, int64_t K, int8_t* wq, int64_t ldwq,
                                float* s_chan, double* Wf, double* Err, hipStream_t s);

}  // namespace w8a8
