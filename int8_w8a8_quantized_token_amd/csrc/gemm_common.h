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


// ---------------------------------------------------------------------------
// Direct global -> LDS loads and their waits.
// ---------------------------------------------------------------------------

// s_waitcnt with vmcnt = n and the other counters left alone (gfx9 encoding).
#define W8A8_WAIT_VM(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | ((((n) >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8))

// s_waitcnt lgkmcnt(0) with the other counters left alone.
#define W8A8_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt((0xF) | (3 << 14) | (0x7 << 4))

__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// Instruction classes of __builtin_amdgcn_sched_group_barrier's mask.
constexpr int kSchedMfma = 0x008;     // MFMA / WMMA
constexpr int kSchedDsRead = 0x100;   // LDS reads

// One global_load_lds_dwordx4: each lane's 16 bytes at gptr land in LDS at
// lds_base + 16 * lane (lds_base is wave-uniform). Issued as inline asm so
// that the compiler's wait-count pass does not treat it as a pending LDS
// write (it would otherwise drain every outstanding DMA before the next LDS
// read); the kernel's explicit vmcnt waits order it instead. No output
// registers; the address is read at issue.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p);
}

// LDS rows of 128 bytes = 8 chunks of 16: row r's chunk c sits at slot
// c ^ swz8(r), swz8(r) = (r & 7) ^ ((r >> 3) & 1). The 8 rows one 8-lane group
// reads, and the 8 even / 8 odd rows of a 16-lane group, land in distinct
// banks; swz8 depends on the low 4 row bits only.
__device__ __forceinline__ int lds_swz8(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// Stage rotation of the LDS-staged decode kernels for weight rows a
// multiple of 4 KB apart: workgroup b starts its K walk at stage
// (b * kMidRotation) mod (K / 128).
constexpr int kMidRotation = 9;

// Waits until at most n * per DMA instructions of this wave are outstanding
// (n < 4; s_waitcnt takes an immediate).
template <int PER>
__device__ __forceinline__ void wait_stages(int n) {
  if (n >= 3) W8A8_WAIT_VM(3 * PER);
  else if (n == 2) W8A8_WAIT_VM(2 * PER);
  else if (n == 1) W8A8_WAIT_VM(PER);
  else W8A8_WAIT_VM(0);
  asm volatile("" ::: "memory");     // LDS reads stay below the wait
}

}  // namespace w8a8
