// Operand loads and the dequantizing epilogue shared by the GEMM kernels.
//   y[m,n] = bf16_rne((float(acc) * s_tok[m]) * s_chan[n])
#pragma once

#include "device_common.h"

namespace w8a8 {

__device__ __forceinline__ v4i ldg16(const int8_t* p) {
  return *reinterpret_cast<const v4i*>(p);
}

__device__ __forceinline__ float dequant(int acc, float st, float sc) {
  return ((float)acc * st) * sc;
}

// Writes 4 consecutive outputs of row m starting at column n (n % 4 == 0):
// int32 accumulators, or bf16((float(acc) * st) * sc[e]).
// vec: the output rows allow one 8-byte (bf16) or 16-byte (int32) store
// per group of 4 (checked on the host: base and row stride aligned).
template <bool I32OUT>
__device__ __forceinline__ void store4(uint16_t* __restrict__ y, int64_t ldy,
                                       int32_t* __restrict__ c, int64_t ldc, int m, int n, int N,
                                       bool vec, float st, const float (&sc)[4], int a0, int a1,
                                       int a2, int a3) {
  if constexpr (I32OUT) {
    int32_t* p = c + (int64_t)m * ldc + n;
    if (vec && n + 3 < N) {
      *reinterpret_cast<v4i*>(p) = v4i{a0, a1, a2, a3};
    } else {
      const int a[4] = {a0, a1, a2, a3};
      for (int e = 0; e < 4 && n + e < N; ++e) p[e] = a[e];
    }
  } else {
    uint16_t* p = y + (int64_t)m * ldy + n;
    const uint32_t b0 = f32_to_bf16_rne(dequant(a0, st, sc[0]));
    const uint32_t b1 = f32_to_bf16_rne(dequant(a1, st, sc[1]));
    const uint32_t b2 = f32_to_bf16_rne(dequant(a2, st, sc[2]));
    const uint32_t b3 = f32_to_bf16_rne(dequant(a3, st, sc[3]));
    if (vec && n + 3 < N) {
      *reinterpret_cast<uint2*>(p) = uint2{b0 | (b1 << 16), b2 | (b3 << 16)};
    } else {
      const uint32_t b[4] = {b0, b1, b2, b3};
      for (int e = 0; e < 4 && n + e < N; ++e) p[e] = (uint16_t)b[e];
    }
  }
}

// Loads the 4 channel scales of outputs n..n+3 (clamped to valid indices;
// values for columns past N are never stored).
__device__ __forceinline__ void load_chan4(const float* __restrict__ s_chan, int n, int N,
                                           float (&sc)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) sc[e] = s_chan[min(n + e, N - 1)];
}

}  // namespace w8a8
