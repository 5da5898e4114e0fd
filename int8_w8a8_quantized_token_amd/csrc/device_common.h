// Device helpers shared by the gfx950 kernels of the W8A8 linear layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;     // CDNA wavefront width
constexpr float kQMax = 127.0f;

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_lo(uint32_t two) { return __uint_as_float(two << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t two) { return __uint_as_float(two & 0xFFFF0000u); }

// float -> bf16 bit pattern, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// The int8 code of a quotient: round half away from zero, clamp to
// [-127, 127]. roundf is C's round (ties away from zero).
__device__ __forceinline__ int int8_code(float v) {
  float r = roundf(v);
  r = fminf(fmaxf(r, -kQMax), kQMax);
  return (int)r;
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) |
         ((uint32_t)(c & 0xFF) << 16) | ((uint32_t)(d & 0xFF) << 24);
}

// Max over a wavefront (all 64 lanes end with the result).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

}  // namespace w8a8
