// Host-only driver of the C ABI's argument checks, for a build with the
// address and undefined-behaviour sanitizers (tests/test_sanitizers.py).
// api.hip is compiled for the host alone; every kernel launcher below is a
// stub that aborts, and every call made here must be refused (or be an
// empty call) by the host-side validation before any launcher or HIP call.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../include/w8a8.h"
#include "../int8_w8a8_quantized_token_amd/csrc/launchers.h"

namespace w8a8 {

[[noreturn]] static void launched(const char* what) {
  fprintf(stderr, "a kernel launcher was reached: %s\n", what);
  abort();
}

hipError_t launch_quantize_rows(RowMode, const uint16_t*, int64_t, const float*, int64_t, int64_t,
                                int8_t*, int64_t, float*, hipStream_t) {
  launched("quantize_rows");
}
hipError_t launch_channel_absmax(const uint16_t*, int64_t, int64_t, int64_t, float*, hipStream_t) {
  launched("channel_absmax");
}
hipError_t launch_smoothing_factors(const float*, const float*, int64_t, float*, hipStream_t) {
  launched("smoothing_factors");
}
hipError_t launch_gemm(const int8_t*, int64_t, const float*, const int8_t*, int64_t, const float*,
                       int64_t, int64_t, int64_t, uint16_t*, int64_t, int32_t*, int64_t,
                       hipStream_t) {
  launched("gemm");
}
bool linear_fused_supported(int64_t, int64_t, int64_t) { launched("linear_fused_supported"); }
hipError_t launch_linear_fused(const uint16_t*, int64_t, const float*, const int8_t*, int64_t,
                               const float*, int64_t, int64_t, int64_t, uint16_t*, int64_t,
                               hipStream_t) {
  launched("linear_fused");
}
hipError_t launch_linear_fused_static(const uint16_t*, int64_t, const float*, const float*,
                                      const int8_t*, int64_t, const float*, int64_t, int64_t,
                                      int64_t, uint16_t*, int64_t, hipStream_t) {
  launched("linear_fused_static");
}
hipError_t launch_quantize_static(const uint16_t*, int64_t, const float*, const float*, int64_t,
                                  int64_t, int8_t*, int64_t, float*, hipStream_t) {
  launched("quantize_static");
}
hipError_t launch_calibrate_minmax(const float*, const float*, int64_t, float*, float*,
                                   hipStream_t) {
  launched("calibrate_minmax");
}
hipError_t launch_abs_histogram(const uint16_t*, int64_t, const float*, int64_t, int64_t,
                                const float*, int64_t, uint32_t*, hipStream_t) {
  launched("abs_histogram");
}
hipError_t launch_calibrate_entropy(const uint32_t*, int64_t, const float*, float*, double*,
                                    hipStream_t) {
  launched("calibrate_entropy");
}
hipError_t launch_rmsnorm_quantize(uint16_t*, int64_t, const uint16_t*, int64_t, const float*,
                                   float, int64_t, int64_t, int8_t*, int64_t, float*,
                                   hipStream_t) {
  launched("rmsnorm_quantize");
}
hipError_t launch_silu_mul_quantize(const uint16_t*, int64_t, const float*, int64_t, int64_t,
                                    int8_t*, int64_t, float*, hipStream_t) {
  launched("silu_mul_quantize");
}
hipError_t launch_fold_gamma(const float*, const float*, int64_t, float*, hipStream_t) {
  launched("fold_gamma");
}
hipError_t launch_residual_add(uint16_t*, int64_t, const uint16_t*, int64_t, int64_t, int64_t,
                               hipStream_t) {
  launched("residual_add");
}
hipError_t launch_gptq_hessian(const uint16_t*, int64_t, const float*, int64_t, int64_t, double*,
                               hipStream_t) {
  launched("gptq_hessian");
}
hipError_t launch_gptq_factor(const double*, int64_t, double, double*, double*, hipStream_t) {
  launched("gptq_factor");
}
hipError_t launch_gptq_quantize(const uint16_t*, int64_t, const float*, const double*, int64_t,
                                int64_t, int8_t*, int64_t, float*, double*, double*,
                                hipStream_t) {
  launched("gptq_quantize");
}

}  // namespace w8a8

static int failures = 0;

#define EXPECT(call, want)                                                                  \
  do {                                                                                      \
    const int got_ = (int)(call);                                                           \
    if (got_ != (int)(want)) {                                                              \
      fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_,     \
              (int)(want));                                                                 \
      ++failures;                                                                           \
    }                                                                                       \
  } while (0)

int main() {
  // fake, never dereferenced addresses: A aligned, MIS 8-byte aligned only
  char* const A = reinterpret_cast<char*>(0x10000);
  char* const MIS = A + 8;
  const int64_t BIG = INT64_MAX, I32 = INT32_MAX, ROWS = (int64_t(1) << 22) - 1;
  auto u16 = [](char* p) { return reinterpret_cast<uint16_t*>(p); };
  auto i8 = [](char* p) { return reinterpret_cast<int8_t*>(p); };
  auto f32 = [](char* p) { return reinterpret_cast<float*>(p); };
  auto f64 = [](char* p) { return reinterpret_cast<double*>(p); };
  auto i32 = [](char* p) { return reinterpret_cast<int32_t*>(p); };
  auto u32 = [](char* p) { return reinterpret_cast<uint32_t*>(p); };
  const w8a8_status_t OK = W8A8_SUCCESS, INV = W8A8_ERROR_INVALID_VALUE,
                      MISAL = W8A8_ERROR_MISALIGNED, UNS = W8A8_ERROR_UNSUPPORTED,
                      WS = W8A8_ERROR_WORKSPACE;

  // status strings and sizes at the extremes
  for (int s = -3; s < 9; ++s)
    if (w8a8_status_string(s) == nullptr) ++failures;
  EXPECT(w8a8_abi_version(), W8A8_ABI_VERSION);
  EXPECT(w8a8_linear_workspace_bytes(-1, 16) == 0, 1);
  EXPECT(w8a8_linear_workspace_bytes(BIG, BIG) == 0, 1);
  EXPECT(w8a8_linear_workspace_bytes(ROWS, 131072) > 0, 1);
  EXPECT(w8a8_linear_workspace_bytes(ROWS + 1, 131072) == 0, 1);
  EXPECT(w8a8_gptq_quantize_workspace_bytes(1 << 19, 16) > 0, 1);
  EXPECT(w8a8_gptq_quantize_workspace_bytes((1 << 19) + 1, 16) == 0, 1);
  EXPECT(w8a8_gptq_factor_workspace_bytes(-5) == 0, 1);
  EXPECT(w8a8_gptq_factor_workspace_bytes(BIG) == 0, 1);
  EXPECT(w8a8_gptq_quantize_workspace_bytes(BIG, BIG) == 0, 1);

  // quantizer
  EXPECT(w8a8_quantize_act(nullptr, 4096, nullptr, 16, 4096, i8(A), 4096, f32(A), 0), INV);
  EXPECT(w8a8_quantize_act(u16(A), 4096, nullptr, -1, 4096, i8(A), 4096, f32(A), 0), INV);
  EXPECT(w8a8_quantize_act(u16(A), 4096, nullptr, 16, 24, i8(A), 24, f32(A), 0), UNS);
  EXPECT(w8a8_quantize_act(u16(A), BIG, nullptr, I32, 4096, i8(A), 4096, f32(A), 0), UNS);
  EXPECT(w8a8_quantize_act(u16(A), 4096, nullptr, BIG, 4096, i8(A), 4096, f32(A), 0), UNS);
  EXPECT(w8a8_quantize_act(u16(MIS), 4096, nullptr, 16, 4096, i8(A), 4096, f32(A), 0), MISAL);
  EXPECT(w8a8_quantize_act(nullptr, 4096, nullptr, 0, 4096, nullptr, 4096, nullptr, 0), OK);

  // GEMMs
  EXPECT(w8a8_gemm(i8(A), 4096, f32(A), i8(A), 4096, f32(A), 16, BIG, 4096, u16(A), 4096, 0), UNS);
  EXPECT(w8a8_gemm(i8(A), 4096, f32(A), i8(A), BIG, f32(A), I32, I32, 4096, u16(A), I32, 0), UNS);
  EXPECT(w8a8_gemm(i8(A), 4096, f32(A), i8(A), 4096, f32(A), 16, 4096, 4096, u16(A + 1), 4096, 0),
         MISAL);
  EXPECT(w8a8_gemm(i8(A), 4096, f32(A), i8(A), 4096, f32(A), 16, 4096, 4096, u16(A), BIG, 0), UNS);
  EXPECT(w8a8_gemm(nullptr, 4096, nullptr, nullptr, 4096, nullptr, 0, 4096, 4096, nullptr, 4096, 0),
         OK);
  EXPECT(w8a8_gemm_i32(i8(A), 64, i8(A), 64, 4, 10, 64, i32(A + 2), 10, 0), MISAL);
  EXPECT(w8a8_gemm_i32(i8(A), 64, i8(A), 64, 4, 8, 64, i32(A), 6, 0), INV);
  EXPECT(w8a8_gemm_i32(i8(A), 64, i8(A), 64, I32, I32, 64, i32(A), BIG, 0), UNS);
  EXPECT(w8a8_gemm(i8(A), 16, f32(A), i8(A), 16, f32(A), 1, ROWS + 1, 16, u16(A), ROWS + 1, 0),
         UNS);                                             // N past the channel bound
  EXPECT(w8a8_gemm(i8(A), 16, f32(A), i8(A), 16, f32(A), ROWS, ROWS, 16, u16(A), ROWS, 0),
         UNS);                                             // M * N past 2^37 outputs
  EXPECT(w8a8_quantize_act(u16(A), 16, nullptr, ROWS + 1, 16, i8(A), 16, f32(A), 0), UNS);

  // linears
  EXPECT(w8a8_linear(u16(A), 4096, nullptr, i8(A), 4096, f32(A), 16, 4096, 4096, u16(A), 4096,
                     nullptr, 0, 0), WS);
  EXPECT(w8a8_linear(u16(A), 131072, nullptr, i8(A), 131072, f32(A), I32, I32, 131072, u16(A), I32,
                     A, 1, 0), UNS);                       // y's rows overflow the size bound
  EXPECT(w8a8_linear(u16(A), 4096, nullptr, i8(A), 4096, f32(A), 16, 4096, 131072, u16(A), 4096,
                     A, 1 << 20, 0), INV);                 // ld < K
  EXPECT(w8a8_linear(u16(A), 4096, nullptr, i8(A), 4096, f32(A), 16, 4096, 4096, u16(A), 4096,
                     A + 16, 1 << 20, 0), MISAL);
  EXPECT(w8a8_linear_static(u16(A), 4096, nullptr, nullptr, i8(A), 4096, f32(A), 16, 4096, 4096,
                            u16(A), 4096, A, 1 << 20, 0), INV);
  EXPECT(w8a8_linear_noalloc(u16(A), 4096, nullptr, i8(A), 4096, f32(A), 2048, 4096, 4096, u16(A),
                             4096, 0), WS);
  EXPECT(w8a8_linear_noalloc(u16(A), 131072, nullptr, i8(A), 131072, f32(A), ROWS, 16,
                             131072, u16(A), 16, 0), WS);
  EXPECT(w8a8_linear_noalloc(u16(A), 131072, nullptr, i8(A), 131072, f32(A), ROWS + 1, 16,
                             131072, u16(A), 16, 0), UNS);  // M past the row bound
  EXPECT(w8a8_linear_noalloc(nullptr, 4096, nullptr, i8(A), 4096, f32(A), 16, 4096, 4096, u16(A),
                             4096, 0), INV);

  // offline preparation and calibration
  EXPECT(w8a8_channel_absmax(u16(A), BIG, I32, 4096, f32(A), 0), UNS);
  EXPECT(w8a8_smoothing_factors(f32(A), f32(A), BIG, f32(A), 0), UNS);
  EXPECT(w8a8_quantize_weight(u16(A), 4096, nullptr, 16, 4104, i8(A), 4104, f32(A), 0), UNS);
  EXPECT(w8a8_quantize_act_static(u16(A), 4096, nullptr, f32(A + 2), 16, 4096, i8(A), 4096, f32(A),
                                  0), MISAL);
  EXPECT(w8a8_calibrate_minmax(f32(A), nullptr, BIG, f32(A), f32(A), 0), UNS);
  EXPECT(w8a8_calibrate_minmax(f32(A), nullptr, -1, f32(A), f32(A), 0), INV);
  EXPECT(w8a8_activation_histogram(u16(A), 4096, nullptr, 16, 4096, f32(A), BIG, u32(A), 0), UNS);
  EXPECT(w8a8_activation_histogram(u16(A), 4096, nullptr, BIG, 4096, f32(A), 2048, u32(A), 0), UNS);
  EXPECT(w8a8_calibrate_entropy(u32(A), BIG, f32(A), f32(A), nullptr, 0), UNS);
  EXPECT(w8a8_calibrate_entropy(u32(A), -5, f32(A), f32(A), nullptr, 0), UNS);

  // producers
  EXPECT(w8a8_rmsnorm_quantize(u16(A), 4096, nullptr, 4096, f32(A), 1e-5f, BIG, 4096, i8(A), 4096,
                               f32(A), 0), UNS);
  EXPECT(w8a8_rmsnorm_quantize(u16(A), 4096, nullptr, 4096, f32(A), -1.0f, 16, 4096, i8(A), 4096,
                               f32(A), 0), INV);
  EXPECT(w8a8_silu_mul_quantize(u16(A), BIG, nullptr, 16, 4096, i8(A), 4096, f32(A), 0), UNS);
  EXPECT(w8a8_silu_mul_quantize(u16(A), 8192, nullptr, 16, BIG, i8(A), 4096, f32(A), 0), UNS);
  EXPECT(w8a8_fold_gamma(f32(A), nullptr, BIG, f32(A), 0), UNS);
  EXPECT(w8a8_residual_add(u16(A), BIG, u16(A), 4096, I32, 4096, 0), UNS);

  // GPTQ
  EXPECT(w8a8_gptq_hessian(u16(A), 4096, nullptr, 16, 40000, f64(A), 0), UNS);
  EXPECT(w8a8_gptq_hessian(u16(A), BIG, nullptr, BIG, 4096, f64(A), 0), UNS);
  EXPECT(w8a8_gptq_factor(f64(A), BIG, 0.01, f64(A), A, 1 << 20, 0), UNS);
  EXPECT(w8a8_gptq_factor(f64(A), 64, 0.01, f64(A), nullptr, 0, 0), WS);
  EXPECT(w8a8_gptq_quantize(u16(A), 64, nullptr, f64(A), BIG, 64, i8(A), 64, f32(A), A, 1 << 20,
                            0), UNS);

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi host checks ok\n");
  return 0;
}
