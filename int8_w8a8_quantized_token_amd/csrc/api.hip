// C ABI of the W8A8 INT8 linear layer: argument validation (host only, before
// any HIP call) and dispatch to the gfx950 kernel launchers.

#include <limits.h>
#include <stdint.h>

#include <mutex>

#include "../../include/w8a8.h"
#include "launchers.h"

namespace {

constexpr int64_t kMaxK = 131072;  // 128 * 128 * K stays below 2^31
constexpr int64_t kMinBins = W8A8_QUANT_LEVELS;
constexpr int64_t kMaxBins = 8192;
constexpr int64_t kMaxProducerK = 65536;   // 8 vectors of 8 per thread at 1024 threads
// Sizes of the kernels that stride over rows (calibration, histogram,
// residual add) and of vectors: below 2^31 - 65536, so that any count
// rounded up to a block and every index formed from it fit in int.
constexpr int64_t kMaxDim = (int64_t)INT32_MAX - 65535;
// Tokens and output channels of the row and GEMM kernels: one workgroup
// of up to 1024 threads per row, or output tiles of at least 192 x 256 with
// 512 threads, so at most 2^22 - 1 rows and 2^37 outputs keep every grid
// dimension within 2^32 work-items (2^37 bf16 outputs exceed HBM anyway).
constexpr int64_t kMaxRows = (int64_t(1) << 22) - 1;
constexpr int64_t kMaxOutputs = int64_t(1) << 37;

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Checks a row-major [rows, cols] operand with row stride ld (elements).
w8a8_status_t check_matrix(const void* p, int64_t ld, int64_t rows, int64_t cols, int64_t elem) {
  if (p == nullptr || ld < cols) return W8A8_ERROR_INVALID_VALUE;
  if (ld > (INT64_MAX / 4) / elem / (rows > 0 ? rows : 1)) return W8A8_ERROR_UNSUPPORTED;
  if (!aligned(p, 16) || (ld * elem) % 16 != 0) return W8A8_ERROR_MISALIGNED;
  return W8A8_SUCCESS;
}

// Output matrices need only element alignment; the kernels use vector stores
// when the base and row stride allow them.
w8a8_status_t check_out_matrix(const void* p, int64_t ld, int64_t rows, int64_t cols,
                               int64_t elem) {
  if (p == nullptr || ld < cols) return W8A8_ERROR_INVALID_VALUE;
  if (ld > (INT64_MAX / 4) / elem / (rows > 0 ? rows : 1)) return W8A8_ERROR_UNSUPPORTED;
  if (!aligned(p, (uintptr_t)elem)) return W8A8_ERROR_MISALIGNED;
  return W8A8_SUCCESS;
}

w8a8_status_t check_vector(const void* p) {
  if (p == nullptr) return W8A8_ERROR_INVALID_VALUE;
  if (!aligned(p, 4)) return W8A8_ERROR_MISALIGNED;
  return W8A8_SUCCESS;
}

// Size checks common to the row-reading entry points.
w8a8_status_t check_dims(int64_t rows, int64_t K, int64_t N = 1) {
  if (rows < 0 || K < 0 || N < 0) return W8A8_ERROR_INVALID_VALUE;
  if (K == 0) return W8A8_ERROR_INVALID_VALUE;
  if (K % 16 != 0 || K > kMaxK || rows > kMaxRows || N > kMaxRows) return W8A8_ERROR_UNSUPPORTED;
  if (rows * N > kMaxOutputs) return W8A8_ERROR_UNSUPPORTED;
  return W8A8_SUCCESS;
}

w8a8_status_t from_hip(hipError_t e) { return e == hipSuccess ? W8A8_SUCCESS : W8A8_ERROR_HIP; }

#define W8A8_TRY(expr)                      \
  do {                                      \
    const w8a8_status_t st_ = (expr);       \
    if (st_ != W8A8_SUCCESS) return st_;    \
  } while (0)

w8a8_status_t validate_gemm(const int8_t* xq, int64_t ldq, const int8_t* wq, int64_t ldw,
                            int64_t M, int64_t N, int64_t K) {
  W8A8_TRY(check_matrix(xq, ldq, M, K, 1));
  W8A8_TRY(check_matrix(wq, ldw, N, K, 1));
  return W8A8_SUCCESS;
}

}  // namespace

extern "C" {

const char* w8a8_status_string(int status) {
  switch (status) {
    case W8A8_SUCCESS: return "success";
    case W8A8_ERROR_INVALID_VALUE: return "invalid value (null pointer, negative size or leading dimension too small)";
    case W8A8_ERROR_MISALIGNED: return "misaligned pointer or row stride";
    case W8A8_ERROR_UNSUPPORTED: return "unsupported size (K must be a positive multiple of 16, at most 131072)";
    case W8A8_ERROR_WORKSPACE: return "workspace missing or too small";
    case W8A8_ERROR_HIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

int w8a8_abi_version(void) { return W8A8_ABI_VERSION; }

w8a8_status_t w8a8_quantize_act(const uint16_t* x, int64_t ldx, const float* smooth, int64_t M,
                                int64_t K, int8_t* xq, int64_t ldq, float* s_tok,
                                hipStream_t stream) {
  W8A8_TRY(check_dims(M, K));
  if (M == 0) return W8A8_SUCCESS;
  W8A8_TRY(check_matrix(x, ldx, M, K, 2));
  W8A8_TRY(check_matrix(xq, ldq, M, K, 1));
  W8A8_TRY(check_vector(s_tok));
  if (smooth) W8A8_TRY(check_vector(smooth));
  return from_hip(w8a8::launch_quantize_rows(w8a8::RowMode::kActivation, x, ldx, smooth, M, K, xq,
                                             ldq, s_tok, stream));
}

w8a8_status_t w8a8_gemm(const int8_t* xq, int64_t ldq, const float* s_tok, const int8_t* wq,
                        int64_t ldw, const float* s_chan, int64_t M, int64_t N, int64_t K,
                        uint16_t* y, int64_t ldy, hipStream_t stream) {
  W8A8_TRY(check_dims(M, K, N));
  if (M == 0 || N == 0) return W8A8_SUCCESS;
  W8A8_TRY(validate_gemm(xq, ldq, wq, ldw, M, N, K));
  W8A8_TRY(check_vector(s_tok));
  W8A8_TRY(check_vector(s_chan));
  W8A8_TRY(check_out_matrix(y, ldy, M, N, 2));
  return from_hip(w8a8::launch_gemm(xq, ldq, s_tok, wq, ldw, s_chan, M, N, K, y, ldy, nullptr, 0,
                                    stream));
}

w8a8_status_t w8a8_gemm_i32(const int8_t* xq, int64_t ldq, const int8_t* wq, int64_t ldw,
                            int64_t M, int64_t N, int64_t K, int32_t* acc, int64_t ldc,
                            hipStream_t stream) {
  W8A8_TRY(check_dims(M, K, N));
  if (M == 0 || N == 0) return W8A8_SUCCESS;
  W8A8_TRY(validate_gemm(xq, ldq, wq, ldw, M, N, K));
  W8A8_TRY(check_out_matrix(acc, ldc, M, N, 4));
  return from_hip(w8a8::launch_gemm(xq, ldq, nullptr, wq, ldw, nullptr, M, N, K, nullptr, 0, acc,
                                    ldc, stream));
}

size_t w8a8_linear_workspace_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0 || M > kMaxRows || K > kMaxK) return 0;
  return align256((size_t)M * (size_t)K) + align256((size_t)M * sizeof(float));
}

w8a8_status_t w8a8_linear(const uint16_t* x, int64_t ldx, const float* smooth, const int8_t* wq,
                          int64_t ldw, const float* s_chan, int64_t M, int64_t N, int64_t K,
                          uint16_t* y, int64_t ldy, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  W8A8_TRY(check_dims(M, K, N));
  if (M == 0 || N == 0) return W8A8_SUCCESS;
  W8A8_TRY(check_matrix(x, ldx, M, K, 2));
  W8A8_TRY(check_matrix(wq, ldw, N, K, 1));
  W8A8_TRY(check_vector(s_chan));
  if (smooth) W8A8_TRY(check_vector(smooth));
  W8A8_TRY(check_out_matrix(y, ldy, M, N, 2));
  if (workspace == nullptr || workspace_bytes < w8a8_linear_workspace_bytes(M, K))
    return W8A8_ERROR_WORKSPACE;
  if (!aligned(workspace, 256)) return W8A8_ERROR_MISALIGNED;

  // One or two tokens on a short, narrow weight: one launch that quantizes
  // inside the GEMM (same codes and scales).
  if (w8a8::linear_fused_supported(M, N, K))
    return from_hip(w8a8::launch_linear_fused(x, ldx, smooth, wq, ldw, s_chan, M, N, K, y, ldy,
                                              stream));
  int8_t* xq = static_cast<int8_t*>(workspace);
  float* s_tok = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256((size_t)M * K));
  W8A8_TRY(from_hip(w8a8::launch_quantize_rows(w8a8::RowMode::kActivation, x, ldx, smooth, M, K,
                                               xq, K, s_tok, stream)));
  return from_hip(w8a8::launch_gemm(xq, K, s_tok, wq, ldw, s_chan, M, N, K, y, ldy, nullptr, 0,
                                    stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// w8a8_linear without a caller workspace
// ---------------------------------------------------------------------------
//
// For callers that cannot allocate device memory: the workspace of
// w8a8_linear (codes and token scales) lives in one fixed device array.
// Each device holds its own copy of the array, at its own address, from the
// library's load until the process ends. In host code the array's name is
// only a stand-in, so its device address is taken once per device with
// hipGetSymbolAddress and kept; kernels receive that address.

namespace {

static __device__ __align__(256) unsigned char scratch[W8A8_NOALLOC_MAX_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];

// The current device's copy of the array (nullptr if it cannot be found).
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

w8a8_status_t w8a8_linear_noalloc(const uint16_t* x, int64_t ldx, const float* smooth,
                                  const int8_t* wq, int64_t ldw, const float* s_chan, int64_t M,
                                  int64_t N, int64_t K, uint16_t* y, int64_t ldy,
                                  hipStream_t stream) {
  W8A8_TRY(check_dims(M, K, N));
  if (M == 0 || N == 0) return W8A8_SUCCESS;
  W8A8_TRY(check_matrix(x, ldx, M, K, 2));
  W8A8_TRY(check_matrix(wq, ldw, N, K, 1));
  W8A8_TRY(check_vector(s_chan));
  if (smooth) W8A8_TRY(check_vector(smooth));
  W8A8_TRY(check_out_matrix(y, ldy, M, N, 2));
  if (w8a8_linear_workspace_bytes(M, K) > (size_t)W8A8_NOALLOC_MAX_BYTES)
    return W8A8_ERROR_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return W8A8_ERROR_HIP;
  return w8a8_linear(x, ldx, smooth, wq, ldw, s_chan, M, N, K, y, ldy, ws,
                     (size_t)W8A8_NOALLOC_MAX_BYTES, stream);
}

w8a8_status_t w8a8_quantize_act_static(const uint16_t* x, int64_t ldx, const float* smooth,
                                       const float* scale, int64_t M, int64_t K, int8_t* xq,
                                       int64_t ldq, float* s_tok, hipStream_t stream) {
  W8A8_TRY(check_dims(M, K));
  if (M == 0) return W8A8_SUCCESS;
  W8A8_TRY(check_matrix(x, ldx, M, K, 2));
  W8A8_TRY(check_matrix(xq, ldq, M, K, 1));
  W8A8_TRY(check_vector(scale));
  W8A8_TRY(check_vector(s_tok));
  if (smooth) W8A8_TRY(check_vector(smooth));
  return from_hip(w8a8::launch_quantize_static(x, ldx, smooth, scale, M, K, xq, ldq, s_tok, stream));
}

w8a8_status_t w8a8_linear_static(const uint16_t* x, int64_t ldx, const float* smooth,
                                 const float* scale, const int8_t* wq, int64_t ldw,
                                 const float* s_chan, int64_t M, int64_t N, int64_t K, uint16_t* y,
                                 int64_t ldy, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  W8A8_TRY(check_dims(M, K, N));
  if (M == 0 || N == 0) return W8A8_SUCCESS;
  W8A8_TRY(check_matrix(x, ldx, M, K, 2));
  W8A8_TRY(check_matrix(wq, ldw, N, K, 1));
  W8A8_TRY(check_vector(scale));
  W8A8_TRY(check_vector(s_chan));
  if (smooth) W8A8_TRY(check_vector(smooth));
  W8A8_TRY(check_out_matrix(y, ldy, M, N, 2));
  if (workspace == nullptr || workspace_bytes < w8a8_linear_workspace_bytes(M, K))
    return W8A8_ERROR_WORKSPACE;
  if (!aligned(workspace, 256)) return W8A8_ERROR_MISALIGNED;

  if (w8a8::linear_fused_supported(M, N, K))
    return from_hip(w8a8::launch_linear_fused_static(x, ldx, smooth, scale, wq, ldw, s_chan, M, N,
                                                     K, y, ldy, stream));
  int8_t* xq = static_cast<int8_t*>(workspace);
  float* s_tok = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256((size_t)M * K));
  W8A8_TRY(from_hip(
      w8a8::launch_quantize_static(x, ldx, smooth, scale, M, K, xq, K, s_tok, stream)));
  return from_hip(w8a8::launch_gemm(xq, K, s_tok, wq, ldw, s_chan, M, N, K, y, ldy, nullptr, 0,
                                    stream));
}

w8a8_status_t w8a8_calibrate_minmax(const float* act_absmax, const float* smooth, int64_t K,
                                    float* amax, float* scale, hipStream_t stream) {
  if (K <= 0) return W8A8_ERROR_INVALID_VALUE;
  if (K > kMaxDim) return W8A8_ERROR_UNSUPPORTED;
  W8A8_TRY(check_vector(act_absmax));
  W8A8_TRY(check_vector(amax));
  W8A8_TRY(check_vector(scale));
  if (smooth) W8A8_TRY(check_vector(smooth));
  return from_hip(w8a8::launch_calibrate_minmax(act_absmax, smooth, K, amax, scale, stream));
}

w8a8_status_t w8a8_activation_histogram(const uint16_t* x, int64_t ldx, const float* smooth,
                                        int64_t rows, int64_t K, const float* amax, int64_t bins,
                                        uint32_t* hist, hipStream_t stream) {
  if (rows < 0 || K <= 0) return W8A8_ERROR_INVALID_VALUE;
  if (K % 8 != 0 || K > kMaxDim / 8 || rows > kMaxDim || bins < kMinBins || bins > kMaxBins)
    return W8A8_ERROR_UNSUPPORTED;
  if (rows == 0) return W8A8_SUCCESS;
  W8A8_TRY(check_matrix(x, ldx, rows, K, 2));
  W8A8_TRY(check_vector(amax));
  W8A8_TRY(check_vector(hist));
  if (smooth) W8A8_TRY(check_vector(smooth));
  return from_hip(
      w8a8::launch_abs_histogram(x, ldx, smooth, rows, K, amax, bins, hist, stream));
}

w8a8_status_t w8a8_calibrate_entropy(const uint32_t* hist, int64_t bins, const float* amax,
                                     float* scale, double* kl, hipStream_t stream) {
  if (bins < kMinBins || bins > kMaxBins) return W8A8_ERROR_UNSUPPORTED;
  W8A8_TRY(check_vector(hist));
  W8A8_TRY(check_vector(amax));
  W8A8_TRY(check_vector(scale));
  if (kl && !aligned(kl, 8)) return W8A8_ERROR_MISALIGNED;
  return from_hip(w8a8::launch_calibrate_entropy(hist, bins, amax, scale, kl, stream));
}

w8a8_status_t w8a8_rmsnorm_quantize(uint16_t* h, int64_t ldh, const uint16_t* residual,
                                    int64_t ldr, const float* gamma, float eps, int64_t M,
                                    int64_t K, int8_t* xq, int64_t ldq, float* s_tok,
                                    hipStream_t stream) {
  W8A8_TRY(check_dims(M, K));
  if (K > kMaxProducerK) return W8A8_ERROR_UNSUPPORTED;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return W8A8_ERROR_INVALID_VALUE;
  if (M == 0) return W8A8_SUCCESS;
  W8A8_TRY(check_matrix(h, ldh, M, K, 2));
  if (residual) W8A8_TRY(check_matrix(residual, ldr, M, K, 2));
  W8A8_TRY(check_vector(gamma));
  W8A8_TRY(check_matrix(xq, ldq, M, K, 1));
  W8A8_TRY(check_vector(s_tok));
  return from_hip(
      w8a8::launch_rmsnorm_quantize(h, ldh, residual, ldr, gamma, eps, M, K, xq, ldq, s_tok, stream));
}

w8a8_status_t w8a8_silu_mul_quantize(const uint16_t* gu, int64_t ldgu, const float* smooth,
                                     int64_t M, int64_t I, int8_t* xq, int64_t ldq, float* s_tok,
                                     hipStream_t stream) {
  W8A8_TRY(check_dims(M, I));
  if (I > kMaxProducerK) return W8A8_ERROR_UNSUPPORTED;
  if (M == 0) return W8A8_SUCCESS;
  W8A8_TRY(check_matrix(gu, ldgu, M, 2 * I, 2));
  if (smooth) W8A8_TRY(check_vector(smooth));
  W8A8_TRY(check_matrix(xq, ldq, M, I, 1));
  W8A8_TRY(check_vector(s_tok));
  return from_hip(w8a8::launch_silu_mul_quantize(gu, ldgu, smooth, M, I, xq, ldq, s_tok, stream));
}

w8a8_status_t w8a8_fold_gamma(const float* gamma, const float* smooth, int64_t K, float* g,
                              hipStream_t stream) {
  if (K < 0) return W8A8_ERROR_INVALID_VALUE;
  if (K > kMaxDim) return W8A8_ERROR_UNSUPPORTED;
  if (K == 0) return W8A8_SUCCESS;
  W8A8_TRY(check_vector(gamma));
  W8A8_TRY(check_vector(g));
  if (smooth) W8A8_TRY(check_vector(smooth));
  return from_hip(w8a8::launch_fold_gamma(gamma, smooth, K, g, stream));
}

w8a8_status_t w8a8_residual_add(uint16_t* h, int64_t ldh, const uint16_t* r, int64_t ldr,
                                int64_t M, int64_t K, hipStream_t stream) {
  if (M < 0 || K <= 0) return W8A8_ERROR_INVALID_VALUE;
  if (K % 8 != 0 || K > kMaxDim / 8 || M > kMaxDim) return W8A8_ERROR_UNSUPPORTED;
  if (M == 0) return W8A8_SUCCESS;
  W8A8_TRY(check_matrix(h, ldh, M, K, 2));
  W8A8_TRY(check_matrix(r, ldr, M, K, 2));
  return from_hip(w8a8::launch_residual_add(h, ldh, r, ldr, M, K, stream));
}

// GPTQ -------------------------------------------------------------------

constexpr int64_t kGptqMaxK = 32768;   // K x K binary64 factor: 8 GiB at the limit
constexpr int64_t kGptqMaxN = int64_t(1) << 19;   // column-update grid: N / 16 rows of blocks
constexpr int64_t kGptqPanel = 64;

w8a8_status_t w8a8_gptq_hessian(const uint16_t* x, int64_t ldx, const float* smooth, int64_t n,
                                int64_t K, double* H, hipStream_t stream) {
  W8A8_TRY(check_dims(n, K));
  if (K > kGptqMaxK) return W8A8_ERROR_UNSUPPORTED;
  if (n == 0) return W8A8_SUCCESS;
  W8A8_TRY(check_matrix(x, ldx, n, K, 2));
  if (smooth) W8A8_TRY(check_vector(smooth));
  if (H == nullptr) return W8A8_ERROR_INVALID_VALUE;
  if (!aligned(H, 8)) return W8A8_ERROR_MISALIGNED;
  return from_hip(w8a8::launch_gptq_hessian(x, ldx, smooth, n, K, H, stream));
}

size_t w8a8_gptq_factor_workspace_bytes(int64_t K) {
  if (K <= 0 || K > kGptqMaxK) return 0;
  return align256((size_t)(K * K + 1) * sizeof(double));
}

w8a8_status_t w8a8_gptq_factor(const double* H, int64_t K, double damp, double* U,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (K <= 0 || H == nullptr || U == nullptr || !(damp >= 0.0) || damp > 1.0e6)
    return W8A8_ERROR_INVALID_VALUE;
  if (K > kGptqMaxK) return W8A8_ERROR_UNSUPPORTED;
  if (!aligned(H, 8) || !aligned(U, 8)) return W8A8_ERROR_MISALIGNED;
  if (workspace == nullptr || workspace_bytes < w8a8_gptq_factor_workspace_bytes(K))
    return W8A8_ERROR_WORKSPACE;
  if (!aligned(workspace, 256)) return W8A8_ERROR_MISALIGNED;
  return from_hip(
      w8a8::launch_gptq_factor(H, K, damp, U, static_cast<double*>(workspace), stream));
}

size_t w8a8_gptq_quantize_workspace_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || K > kGptqMaxK || N > kGptqMaxN) return 0;
  return align256((size_t)N * (size_t)K * sizeof(double)) +
         align256((size_t)N * kGptqPanel * sizeof(double));
}

w8a8_status_t w8a8_gptq_quantize(const uint16_t* w, int64_t ldw, const float* smooth,
                                 const double* U, int64_t N, int64_t K, int8_t* wq, int64_t ldwq,
                                 float* s_chan, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  W8A8_TRY(check_dims(N, K));
  if (K > kGptqMaxK || N > kGptqMaxN) return W8A8_ERROR_UNSUPPORTED;
  if (N == 0) return W8A8_SUCCESS;
  W8A8_TRY(check_matrix(w, ldw, N, K, 2));
  W8A8_TRY(check_matrix(wq, ldwq, N, K, 1));
  W8A8_TRY(check_vector(s_chan));
  if (smooth) W8A8_TRY(check_vector(smooth));
  if (U == nullptr) return W8A8_ERROR_INVALID_VALUE;
  if (!aligned(U, 8)) return W8A8_ERROR_MISALIGNED;
  if (workspace == nullptr || workspace_bytes < w8a8_gptq_quantize_workspace_bytes(N, K))
    return W8A8_ERROR_WORKSPACE;
  if (!aligned(workspace, 256)) return W8A8_ERROR_MISALIGNED;
  double* Wf = static_cast<double*>(workspace);
  double* Err = reinterpret_cast<double*>(static_cast<char*>(workspace) +
                                          align256((size_t)N * (size_t)K * sizeof(double)));
  return from_hip(w8a8::launch_gptq_quantize(w, ldw, smooth, U, N, K, wq, ldwq, s_chan, Wf, Err,
                                             stream));
}

w8a8_status_t w8a8_channel_absmax(const uint16_t* a, int64_t lda, int64_t rows, int64_t K,
                                  float* absmax, hipStream_t stream) {
  if (rows < 0 || K <= 0) return W8A8_ERROR_INVALID_VALUE;
  if (K % 8 != 0 || K > kMaxDim / 8 || rows > kMaxDim) return W8A8_ERROR_UNSUPPORTED;
  if (rows == 0) return W8A8_SUCCESS;
  W8A8_TRY(check_matrix(a, lda, rows, K, 2));
  W8A8_TRY(check_vector(absmax));
  return from_hip(w8a8::launch_channel_absmax(a, lda, rows, K, absmax, stream));
}

w8a8_status_t w8a8_smoothing_factors(const float* act_absmax, const float* w_absmax, int64_t K,
                                     float* smooth, hipStream_t stream) {
  if (K < 0) return W8A8_ERROR_INVALID_VALUE;
  if (K > kMaxDim) return W8A8_ERROR_UNSUPPORTED;
  if (K == 0) return W8A8_SUCCESS;
  W8A8_TRY(check_vector(act_absmax));
  W8A8_TRY(check_vector(w_absmax));
  W8A8_TRY(check_vector(smooth));
  return from_hip(w8a8::launch_smoothing_factors(act_absmax, w_absmax, K, smooth, stream));
}

w8a8_status_t w8a8_quantize_weight(const uint16_t* w, int64_t ldw, const float* smooth, int64_t N,
                                   int64_t K, int8_t* wq, int64_t ldwq, float* s_chan,
                                   hipStream_t stream) {
  W8A8_TRY(check_dims(N, K));
  if (N == 0) return W8A8_SUCCESS;
  W8A8_TRY(check_matrix(w, ldw, N, K, 2));
  W8A8_TRY(check_matrix(wq, ldwq, N, K, 1));
  W8A8_TRY(check_vector(s_chan));
  if (smooth) W8A8_TRY(check_vector(smooth));
  return from_hip(w8a8::launch_quantize_rows(w8a8::RowMode::kWeight, w, ldw, smooth, N, K, wq,
                                             ldwq, s_chan, stream));
}

}  // extern "C"
