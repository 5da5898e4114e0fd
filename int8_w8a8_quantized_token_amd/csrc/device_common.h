// Device helpers shared by the gfx950 kernels of the W8A8 linear layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;     // CDNA wavefront width
constexpr float kQMax = 127.0f;
constexpr int kQuantLevels = 128;   // code magnitudes 0..127

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_lo(uint32_t two) { return __uint_as_float(two << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t two) { return __uint_as_float(two & 0xFFFF0000u); }

// float -> bf16 bit pattern, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// binary64 -> bf16 bit pattern, one rounding to nearest even (finite inputs).
// Round to odd into binary32 first (truncate, then set the last bit when the
// truncation was inexact), then to nearest even into bf16: with 16 spare
// bits in between this equals the direct rounding (Boldo and Melquiond,
// "Emulation of FMA and correctly rounded sums: proved algorithms using
// rounding to odd").
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double m) {
  const float f = __double2float_rz(m);
  uint32_t u = __float_as_uint(f);
  if ((double)f != m) u |= 1u;
  return f32_to_bf16_rne(__uint_as_float(u));
}

// The int8 code of a quotient: round half away from zero, clamp to
// [-127, 127]. roundf is C's round (ties away from zero).
__device__ __forceinline__ int int8_code(float v) {
  float r = roundf(v);
  r = fminf(fmaxf(r, -kQMax), kQMax);
  return (int)r;
}

// ---------------------------------------------------------------------------
// Division-free form of the quantizer's code step. Where it applies it
// returns what the division gives (IEEE binary32, round to nearest even,
// denormals kept); elsewhere the callers divide.
// tests/exhaustive/quantize_fastpath_check.c checks it on the host.
// ---------------------------------------------------------------------------

// Codes: the int8 code of v / S (round half away from zero, clamp) from
// t = RN(v R), R = RN(1 / S), S in [2^-100, 2^100]. t lies within
// 3 * 2^-24 * |v / S| + 2^-148 of RN(v / S), which is below 2^-15 while
// |v / S| <= 128.0001. So when n = rint(t) satisfies |t - n| < 1/2 - 2^-15,
// the quotient lies strictly within 1/2 of n and rounds to n under any tie
// rule; |t| >= 128 means a clamped code. ok is false for the rest (about 6
// values in 10^5), which divide.
constexpr float kTieGuard = 0x1p-15f;

__device__ __forceinline__ bool code_fast_ok(float S) { return S >= 0x1p-100f && S <= 0x1p100f; }

__device__ __forceinline__ float code_fast(float v, float R, bool& ok) {
  const float t = v * R;
  const float n = __builtin_rintf(t);
  ok = fabsf(t - n) < 0.5f - kTieGuard || fabsf(t) >= 128.0f;
  return fminf(fmaxf(n, -kQMax), kQMax);
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) |
         ((uint32_t)(c & 0xFF) << 16) | ((uint32_t)(d & 0xFF) << 24);
}

// Codes of 8 values under one row scale S, packed little-endian (value e in
// byte e). R = RN(1 / S) and fast = code_fast_ok(S); values the fast form
// leaves open (all of them when fast is false) are divided. S == 0 gives 0.
__device__ __forceinline__ uint2 codes8(const float (&v)[8], float S, float R, bool fast) {
  int c[8];
  if (S == 0.0f) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = 0;
  } else {
    uint32_t slow = fast ? 0u : 0xFFu;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bool ok;
      c[e] = (int)code_fast(v[e], R, ok);
      slow |= ok ? 0u : (1u << e);
    }
    if (slow != 0u) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (slow & (1u << e)) c[e] = int8_code(v[e] / S);
    }
  }
  return uint2{pack4_i8(c[0], c[1], c[2], c[3]), pack4_i8(c[4], c[5], c[6], c[7])};
}

// One DPP move of a binary32 value within rows of 16 lanes (ctrl constant).
#define W8A8_DPP_F32(x, ctrl) \
  __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), (ctrl), 0xF, 0xF, false))

// Max over a wavefront; every lane ends with the result. All 64 lanes must be
// active. Within each row of 16 lanes: max with the neighbour (quad_perm
// [1,0,3,2]), with the other pair (quad_perm [2,3,0,1]), with the mirrored
// half row (row_half_mirror) and with the mirrored row (row_mirror); then the
// four row maxima through scalar reads. No LDS traffic, unlike a butterfly
// of cross-lane shuffles (ds_bpermute), whose six LDS round trips sat on the
// critical path of every row reduction.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, W8A8_DPP_F32(v, 0xB1));
  v = fmaxf(v, W8A8_DPP_F32(v, 0x4E));
  v = fmaxf(v, W8A8_DPP_F32(v, 0x141));
  v = fmaxf(v, W8A8_DPP_F32(v, 0x140));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

}  // namespace w8a8
