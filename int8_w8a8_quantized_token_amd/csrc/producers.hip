// Fused producers on gfx950: the ops that feed a Llama block's linears end in
// the per-token quantizer, so they emit int8 codes and scales directly
// instead of a bf16 tensor that a separate quantize pass would read again.
//
// The Red Hat article "Understanding W8A8 INT8 LLM quantization: Half the
// size, better performance, same accuracy" places the activation outliers in
// RMSNorm's weight (section "How SmoothQuant prevents outliers in activation
// tensors") and folds the SmoothQuant division into that weight (section
// "How the SmoothQuant smoothing factor is computed"). So:
//   * add + RMSNorm + quantize: h = bf16(h + r) (optional, written back as the
//     new residual stream); ms = sum(h^2) / K, the exact mean rounded once
//     to binary32;
//     inv = 1 / sqrt(ms + eps); y = (h * inv) * g with g = gamma / s; then
//     S = max|y| / 127 and codes;
//   * SiLU-gated product + quantize: m = bf16((g / (1 + exp(-g))) * u), the
//     real value rounded once (a binary32 evaluation with a proven error
//     bound where that decides the rounding, binary64 elsewhere), from the
//     bf16 gate and up halves of a row; x' = m / s; codes.
//
// The sum of squares is exact per term (a bf16 square fits binary64) and is
// accumulated in double-double; the binary32 rounding of the mean is then
// decided exactly (mean_square_rn32), so it does not depend on the order of
// the sum.

#include "device_common.h"
#include "launchers.h"

namespace w8a8 {

// ---------------------------------------------------------------------------
// double-double accumulation
// ---------------------------------------------------------------------------

struct DD {
  double hi, lo;
};

// s + e = a + b exactly (Knuth's two-sum; needs no contraction).
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  const double bp = s - a;
  e = (a - (s - bp)) + (b - bp);
}

__device__ __forceinline__ DD dd_add(DD x, DD y) {
  double s, e;
  two_sum(x.hi, y.hi, s, e);
  e += x.lo + y.lo;
  DD r;
  two_sum(s, e, r.hi, r.lo);
  return r;
}

__device__ __forceinline__ DD dd_add(DD x, double v) {
  double s, e;
  two_sum(x.hi, v, s, e);
  DD r;
  r.hi = s;
  r.lo = x.lo + e;
  return r;
}

__device__ __forceinline__ DD dd_shfl_xor(DD x, int off) {
  DD r;
  r.hi = __shfl_xor(x.hi, off, kWave);
  r.lo = __shfl_xor(x.lo, off, kWave);
  return r;
}

// Block-wide double-double sum (normalized: |lo| <= ulp(hi) / 2); every
// thread gets the same value.
template <int BS>
__device__ __forceinline__ DD block_sum_dd(DD v, DD* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = dd_add(v, dd_shfl_xor(v, off));
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[wave] = v;
  __syncthreads();
  DD t = red[0];
#pragma unroll
  for (int w = 1; w < BS / kWave; ++w) t = dd_add(t, red[w]);
  return t;
}

template <int BS>
__device__ __forceinline__ float block_max_f(float v, float* red) {
  v = wave_max(v);
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < BS / kWave; ++w) r = fmaxf(r, red[w]);
  return r;
}

// Codes of 8 values of one row (as in the per-token quantizer).
__device__ __forceinline__ void store_codes8(int8_t* __restrict__ qr, int vi, const float (&v)[8],
                                             float S, float R, bool fast) {
  *reinterpret_cast<uint2*>(qr + (int64_t)vi * 8) = codes8(v, S, R, fast);
}

__device__ __forceinline__ void unpack8(uint4 raw, float (&v)[8]) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = bf16_lo(w[e]);
    v[2 * e + 1] = bf16_hi(w[e]);
  }
}

__device__ __forceinline__ uint4 pack8_bf16(const float (&v)[8]) {
  uint4 r;
  r.x = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
  r.y = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
  r.z = f32_to_bf16_rne(v[4]) | (f32_to_bf16_rne(v[5]) << 16);
  r.w = f32_to_bf16_rne(v[6]) | (f32_to_bf16_rne(v[7]) << 16);
  return r;
}

// ---------------------------------------------------------------------------
// the mean of squares, rounded once to binary32
// ---------------------------------------------------------------------------
//
// The row's sum of squares S arrives as a normalized double-double hi + lo.
// Every term is nonnegative, the two-sum steps are exact and only the low
// words' additions round (a thread adds at most 64 terms, then about 22
// double-double additions combine the threads), so hi + lo is within 2^-90
// of S, relatively. Its quotient by K, rounded to binary32, is therefore
// RN32(S / K) or a binary32 neighbour of it; which one depends on the sign of
// S - K t for the two midpoints t around that candidate. K t is exact in
// binary64 (a midpoint has 25 significant bits, K < 2^17). Where
// hi + lo - K t lies farther from 0 than 2^-70 hi, its sign is the sign of
// S - K t; otherwise (the mean within 2^-70 of a midpoint, which real data
// essentially never meets) the workgroup compares S and K t exactly.

// Number of bins of exact_square_sum_cmp: a bf16 value with biased exponent E
// is m 2^(e) with integer significand m < 256 and e = max(E, 1) - 134, so its
// square is m^2 4^(max(E, 1) - 1) 2^-266 and finite squares fall into bins
// 0 .. 253; bin 254 takes E = 255 (inf, NaN), whose rows have no defined
// result but must not index past the array.
constexpr int kSqBins = 255;
constexpr int kLimbs = 18;           // 32-bit limbs of S 2^266 < 2^539 (< 2^541 with bin 254)

struct SqScratch {
  unsigned long long bins[kSqBins];  // sum of m^2 per exponent (< 65536 * 2^16)
  uint32_t s[kLimbs], t[kLimbs];     // S 2^266 and T 2^266, little-endian
  int result;
};

// sign(S - T) for S the exact sum of squares of the row's values and T > 0 a
// binary64 value with T 2^266 an integer. The values are read back from the
// row in memory (bf16, nvec vectors of 8); each thread reads the vectors it
// wrote itself. Called by every thread of the workgroup.
template <int BS>
__device__ __forceinline__ int exact_square_sum_cmp(const uint16_t* row, int nvec,
                                                 double T, SqScratch* sc) {
  const int tid = threadIdx.x;
  for (int k = tid; k < kSqBins; k += BS) sc->bins[k] = 0ull;
  for (int k = tid; k < kLimbs; k += BS) { sc->s[k] = 0u; sc->t[k] = 0u; }
  __syncthreads();
#pragma unroll 1
  for (int vi = tid; vi < nvec; vi += BS) {
    const uint4 raw = *reinterpret_cast<const uint4*>(row + (int64_t)vi * 8);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t b = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      const uint32_t E = (b >> 7) & 0xFFu, f = b & 0x7Fu;
      const uint32_t m = E ? (f | 0x80u) : f;
      if (m) atomicAdd(&sc->bins[E ? E - 1 : 0], (unsigned long long)(m * m));
    }
  }
  __syncthreads();
  if (tid == 0) {
    // S 2^266 = sum_k bins[k] 4^k
    for (int k = 0; k < kSqBins; ++k) {
      unsigned long long add = sc->bins[k] << ((2 * k) & 31);   // < 2^63
      for (int j = (2 * k) >> 5; add != 0ull && j < kLimbs; ++j) {
        const unsigned long long cur = (unsigned long long)sc->s[j] + (add & 0xFFFFFFFFull);
        sc->s[j] = (uint32_t)cur;
        add = (add >> 32) + (cur >> 32);
      }
    }
    // T 2^266 = mant 2^(ex + 266) for the normal binary64 T = mant 2^ex
    const unsigned long long tb = (unsigned long long)__double_as_longlong(T);
    const unsigned long long mant = (tb & 0xFFFFFFFFFFFFFull) | 0x10000000000000ull;
    const int sh = (int)((tb >> 52) & 0x7FF) - 1075 + 266;            // >= 0 here
    const int w = sh >> 5, b = sh & 31;
    const unsigned long long lo = mant << b;                           // low 64 bits
    const unsigned long long hi = b ? mant >> (64 - b) : 0ull;         // bits 64 and up
    if (w < kLimbs) sc->t[w] = (uint32_t)lo;
    if (w + 1 < kLimbs) sc->t[w + 1] = (uint32_t)(lo >> 32);
    if (w + 2 < kLimbs) sc->t[w + 2] = (uint32_t)hi;
    int r = 0;
    for (int j = kLimbs - 1; j >= 0 && r == 0; --j)
      r = sc->s[j] > sc->t[j] ? 1 : (sc->s[j] < sc->t[j] ? -1 : 0);
    sc->result = r;
  }
  __syncthreads();
  const int r = sc->result;
  __syncthreads();
  return r;
}

// sign(S - T) from the double-double sum, 2 where it is too close to tell.
__device__ __forceinline__ int square_sum_cmp_fast(DD ss, double T) {
  double d, e;
  two_sum(ss.hi, -T, d, e);
  const double r = d + (e + ss.lo);
  const double bound = ss.hi * 0x1p-70;
  return r > bound ? 1 : (r < -bound ? -1 : 2);
}

// RN32(S / K) where S / K may lie near a binary32 midpoint, from q, an
// approximation of S / K whose binary32 rounding is RN32(S / K) or a
// neighbour of it: the two midpoints around that candidate, compared with S as
// described above.
template <int BS>
__device__ __forceinline__ float mean_square_rn32_near(DD ss, double q, int K,
                                                    const uint16_t* row, int nvec,
                                                    SqScratch* sc) {
  const float c = (float)q;
  const uint32_t cb = __float_as_uint(c);
  // the midpoints below and above c; past the largest finite value the
  // overflow threshold 2^128 - 2^103 takes the place of a midpoint
  const double cd = cb == 0x7F800000u ? 0x1p128 : (double)c;
  const double tl = cb != 0u ? ((double)__uint_as_float(cb - 1u) + cd) * 0.5 : 0.0;
  const double nd = cb == 0x7F7FFFFFu ? 0x1p128 : (double)__uint_as_float(cb + 1u);
  const double tu = cb != 0x7F800000u ? (cd + nd) * 0.5 : 0.0;
  int sl = cb != 0u ? square_sum_cmp_fast(ss, tl * (double)K) : 1;
  int su = cb != 0x7F800000u ? square_sum_cmp_fast(ss, tu * (double)K) : -1;
  if (sl == 2 || su == 2) {
    const int ex = exact_square_sum_cmp<BS>(row, nvec, (sl == 2 ? tl : tu) * (double)K, sc);
    if (sl == 2) sl = ex;
    else su = ex;
  }
  if (sl < 0 || (sl == 0 && (cb & 1u))) return __uint_as_float(cb - 1u);
  if (su > 0 || (su == 0 && (cb & 1u))) return __uint_as_float(cb + 1u);
  return c;
}

// Whether the binary32 rounding of q = (hi + lo) * RN(1 / K) is RN32(S / K),
// ties to even, for S the exact sum of squares of the row. q is within 3.01
// units in its last place of S / K (2^-90 from the double-double, one
// rounding each for hi + lo, 1 / K and the product). For q in the normal
// binary32 range its 29 bits below binary32 precision say where q lies
// between two binary32 values; unless they are within 8 units of the halfway
// pattern, S / K lies on the same side of the midpoint as q and rounds to
// RN32(q). The rest (about 2^-25 of rows, plus rows whose mean is not a
// normal binary32 value) take the comparison with the midpoints.
__device__ __forceinline__ bool mean_square_clear(DD ss, double q) {
  const uint32_t low = (uint32_t)(__double_as_longlong(q) & 0x1FFFFFFFll);
  // evaluated without branches (bitwise, not short-circuit)
  return (ss.hi == 0.0) |                                 // every square is 0
         ((q >= 0x1p-126) & (q < 0x1p127) & ((low < 0x10000000u - 8u) | (low > 0x10000000u + 8u)));
}

// RN32(S / K), ties to even: q's binary32 rounding where mean_square_clear
// says so, else the comparison with the midpoints. Every thread sees the same
// ss, so the branch is uniform; the rare case is laid out after the kernel's
// common path.
template <int BS>
__device__ __forceinline__ float mean_square_rn32(DD ss, double q, int K, const uint16_t* row,
                                                  int nvec, SqScratch* sc) {
  float ms = (float)q;
  if (__builtin_expect(!mean_square_clear(ss, q), 0))
    ms = mean_square_rn32_near<BS>(ss, q, K, row, nvec, sc);
  return ms;
}

// ---------------------------------------------------------------------------
// residual add + RMSNorm + quantize: one BS-thread workgroup per row, the row
// in registers (NV vectors of 8 per thread)
// ---------------------------------------------------------------------------

template <int BS, int NV, bool ADD>
__global__ __launch_bounds__(BS) void rmsnorm_quantize_kernel(
    uint16_t* __restrict__ h, int64_t ldh, const uint16_t* __restrict__ res, int64_t ldr,
    const float* __restrict__ g, float eps, int K, double inv_k, int8_t* __restrict__ q, int64_t ldq,
    float* __restrict__ s_tok) {
  __shared__ DD red_dd[BS / kWave];
  __shared__ float red_f[BS / kWave];
  __shared__ SqScratch sq;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nvec = K / 8;
  uint16_t* hr = h + row * ldh;

  // Every load a thread needs (its h, residual and factor vectors) goes out
  // before any arithmetic: one memory round trip per row, not one per vector
  // plus one for the factors after the reduction. Vectors past the row end
  // load the row's last vector (K >= 16) and are then left out. At 1024
  // threads (128 registers a lane) with 8 vectors a thread the early factors
  // would not fit beside the row, so those read them after the reduction.
  constexpr bool kEarlyG = !(BS == 1024 && NV == 8);
  uint4 hraw[NV], rraw[NV];
  float gv[kEarlyG ? NV : 1][8];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vl = min(tid + i * BS, nvec - 1);
    hraw[i] = *reinterpret_cast<const uint4*>(hr + (int64_t)vl * 8);
    if constexpr (ADD) rraw[i] = *reinterpret_cast<const uint4*>(res + row * ldr + (int64_t)vl * 8);
    if constexpr (kEarlyG) {
#pragma unroll
      for (int e = 0; e < 8; ++e) gv[i][e] = g[vl * 8 + e];
    }
  }

  float v[NV][8];
  DD acc = {0.0, 0.0};
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vi = tid + i * BS;
    if (vi < nvec) {
      unpack8(hraw[i], v[i]);
      if constexpr (ADD) {
        float r[8];
        unpack8(rraw[i], r);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[i][e] = __uint_as_float(f32_to_bf16_rne(v[i][e] + r[e]) << 16);
        *reinterpret_cast<uint4*>(hr + (int64_t)vi * 8) = pack8_bf16(v[i]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double x = (double)v[i][e];
        acc = dd_add(acc, x * x);
      }
    }
  }
  const DD ss = block_sum_dd<BS>(acc, red_dd);
  const float ms = mean_square_rn32<BS>(ss, (ss.hi + ss.lo) * inv_k, K, hr, nvec, &sq);
  const float inv = 1.0f / sqrtf(ms + eps);

  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vi = tid + i * BS;
    if (vi < nvec) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float gi;
        if constexpr (kEarlyG) gi = gv[i][e];
        else gi = g[vi * 8 + e];
        v[i][e] = (v[i][e] * inv) * gi;
        amax = fmaxf(amax, fabsf(v[i][e]));
      }
    }
  }
  amax = block_max_f<BS>(amax, red_f);
  const float S = amax / kQMax;
  if (tid == 0) s_tok[row] = S;
  const bool fast = code_fast_ok(S);
  const float R = fast ? 1.0f / S : 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vi = tid + i * BS;
    if (vi < nvec) store_codes8(q + row * ldq, vi, v[i], S, R, fast);
  }
}

// ---------------------------------------------------------------------------
// SiLU-gated product + quantize
// ---------------------------------------------------------------------------

// e^x for |x| <= 80 in binary32: x = n ln 2 + r with a two-part ln 2 (fused
// multiply-adds), e^r by its Taylor polynomial to degree 7 (|r| <= ln2 / 2,
// remainder below 2^-26.5 relative), then the exact scaling by 2^n. Relative
// error below 3 * 2^-24.
__device__ __forceinline__ float exp_bounded(float x) {
  const float n = __builtin_rintf(x * 0x1.715476p+0f);   // log2(e)
  float r = fmaf(-n, 0x1.62e43p-1f, x);                  // ln 2, high part
  r = fmaf(-n, -0x1.05c61p-29f, r);                      // ln 2, low part
  float p = 0x1.a01a02p-13f;                             // 1/7!
  p = fmaf(p, r, 0x1.6c16c2p-10f);                       // 1/6!
  p = fmaf(p, r, 0x1.111112p-7f);                        // 1/5!
  p = fmaf(p, r, 0x1.555556p-5f);                        // 1/4!
  p = fmaf(p, r, 0x1.555556p-3f);                        // 1/3!
  p = fmaf(p, r, 0.5f);
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  return ldexpf(p, (int)n);
}

// bf16(g / (1 + e^-g) * u) from a binary32 evaluation, when that is certain.
// The quotient is g times the hardware reciprocal of 1 + e, which the ISA
// documents as within 1 ulp (so one of the two binary32 neighbours of the
// exact reciprocal). For |g| <= 80 the binary32 value is then within 9 ulps
// of the real one (relative errors: exp 3 * 2^-24, 1 + e 2^-24, the
// reciprocal 2 * 2^-24, the two products 2^-24 each), so its bf16 rounding
// is the real value's whenever its low 16 bits are more than 16 away from
// 0x8000, the rounding boundary, and it is a normal number of moderate size;
// a zero gate or up value gives an exact zero. ok = false for everything
// else. tests/exhaustive/silu_fastpath_check.c runs this decision for every
// pair of finite bf16 inputs and every reciprocal the 1-ulp bound allows.
__device__ __forceinline__ float silu_mul_fast(float g, float u, bool& ok) {
  const float q = g * __builtin_amdgcn_rcpf(1.0f + exp_bounded(-g));
  const float m = q * u;
  const float a = fabsf(m);
  const int lo = (int)(__float_as_uint(m) & 0xFFFFu);
  // bitwise, not short-circuit: the compiler would branch per value
  const bool clear = (lo > 0x8000 + 16) | (lo < 0x8000 - 16);
  ok = (fabsf(g) <= 80.0f) &
       ((g == 0.0f) | (u == 0.0f) | ((a >= 0x1p-120f) & (a < 0x1p120f) & clear));
  return __uint_as_float(f32_to_bf16_rne(m) << 16);
}

// The same value evaluated in binary64 and rounded once to bf16.
__device__ __forceinline__ float silu_mul_f64(float g, float u) {
  const double gd = (double)g;
  const double m = (gd / (1.0 + exp(-gd))) * (double)u;
  return __uint_as_float((uint32_t)f64_to_bf16_rne(m) << 16);
}

template <int BS, int NV, bool SMOOTH>
__global__ __launch_bounds__(BS) void silu_mul_quantize_kernel(
    const uint16_t* __restrict__ gu, int64_t ldgu, const float* __restrict__ smooth, int I,
    int8_t* __restrict__ q, int64_t ldq, float* __restrict__ s_tok) {
  __shared__ float red_f[BS / kWave];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nvec = I / 8;
  const uint16_t* gr = gu + row * ldgu;

  float v[NV][8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vi = tid + i * BS;
    if (vi < nvec) {
      float gv[8], uv[8];
      unpack8(*reinterpret_cast<const uint4*>(gr + (int64_t)vi * 8), gv);
      unpack8(*reinterpret_cast<const uint4*>(gr + I + (int64_t)vi * 8), uv);
      float mv[8];
      uint32_t slow = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bool ok;
        mv[e] = silu_mul_fast(gv[e], uv[e], ok);
        slow |= ok ? 0u : (1u << e);
      }
      // The undecided values in binary64, one per lane per pass, so that a
      // wave runs the slow path about once however its lanes' values fall.
      while (slow != 0u) {
        const int idx = __builtin_ctz(slow);
        float gs = gv[0], us = uv[0];
#pragma unroll
        for (int e = 1; e < 8; ++e)
          if (idx == e) { gs = gv[e]; us = uv[e]; }
        const float r = silu_mul_f64(gs, us);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (idx == e) mv[e] = r;
        slow &= slow - 1u;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float mf = mv[e];
        if constexpr (SMOOTH) mf = mf / smooth[vi * 8 + e];
        v[i][e] = mf;
        amax = fmaxf(amax, fabsf(mf));
      }
    }
  }
  amax = block_max_f<BS>(amax, red_f);
  const float S = amax / kQMax;
  if (tid == 0) s_tok[row] = S;
  const bool fast = code_fast_ok(S);
  const float R = fast ? 1.0f / S : 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vi = tid + i * BS;
    if (vi < nvec) store_codes8(q + row * ldq, vi, v[i], S, R, fast);
  }
}

// ---------------------------------------------------------------------------
// small elementwise helpers: gamma / s, and h = bf16(h + r)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void fold_gamma_kernel(const float* __restrict__ gamma,
                                                         const float* __restrict__ smooth,
                                                         int64_t K, float* __restrict__ g) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k < K) g[k] = smooth ? gamma[k] / smooth[k] : gamma[k];
}

__global__ __launch_bounds__(256) void residual_add_kernel(uint16_t* __restrict__ h, int64_t ldh,
                                                           const uint16_t* __restrict__ r,
                                                           int64_t ldr, int64_t M, int K) {
  const int vi = blockIdx.x * 256 + threadIdx.x;
  if (vi >= K / 8) return;
  for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
    float a[8], b[8];
    unpack8(*reinterpret_cast<const uint4*>(h + m * ldh + (int64_t)vi * 8), a);
    unpack8(*reinterpret_cast<const uint4*>(r + m * ldr + (int64_t)vi * 8), b);
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = a[e] + b[e];
    *reinterpret_cast<uint4*>(h + m * ldh + (int64_t)vi * 8) = pack8_bf16(a);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

// Threads per row: 1024 for few rows (decode), otherwise 256 (512 for rows
// longer than 8192 channels), raised until 8 vectors per thread cover the row.
static int producer_threads(int64_t rows, int64_t K) {
  int bs = rows <= 512 ? 1024 : (K > 8192 ? 512 : 256);
  while (bs < 1024 && (K / 8 + bs - 1) / bs > 8) bs *= 2;
  return bs;
}

template <int BS, bool ADD>
static hipError_t launch_rmsnorm_bs(uint16_t* h, int64_t ldh, const uint16_t* r, int64_t ldr,
                                    const float* g, float eps, int64_t M, int64_t K, int8_t* q,
                                    int64_t ldq, float* s_tok, hipStream_t s) {
  const int64_t per = (K / 8 + BS - 1) / BS;
  const double inv_k = 1.0 / (double)K;                 // correctly rounded
#define W8A8_RMS(NVV)                                                                             \
  hipLaunchKernelGGL((rmsnorm_quantize_kernel<BS, NVV, ADD>), dim3((unsigned)M), dim3(BS), 0, s, \
                     h, ldh, r, ldr, g, eps, (int)K, inv_k, q, ldq, s_tok)
  if (per <= 1) W8A8_RMS(1);
  else if (per <= 2) W8A8_RMS(2);
  else if (per <= 4) W8A8_RMS(4);
  else W8A8_RMS(8);
#undef W8A8_RMS
  return hipGetLastError();
}

template <bool ADD>
static hipError_t launch_rmsnorm_add(uint16_t* h, int64_t ldh, const uint16_t* r, int64_t ldr,
                                     const float* g, float eps, int64_t M, int64_t K, int8_t* q,
                                     int64_t ldq, float* s_tok, hipStream_t s) {
  switch (producer_threads(M, K)) {
    case 256: return launch_rmsnorm_bs<256, ADD>(h, ldh, r, ldr, g, eps, M, K, q, ldq, s_tok, s);
    case 512: return launch_rmsnorm_bs<512, ADD>(h, ldh, r, ldr, g, eps, M, K, q, ldq, s_tok, s);
    default: return launch_rmsnorm_bs<1024, ADD>(h, ldh, r, ldr, g, eps, M, K, q, ldq, s_tok, s);
  }
}

hipError_t launch_rmsnorm_quantize(uint16_t* h, int64_t ldh, const uint16_t* residual,
                                   int64_t ldr, const float* g, float eps, int64_t M, int64_t K,
                                   int8_t* q, int64_t ldq, float* s_tok, hipStream_t s) {
  return residual ? launch_rmsnorm_add<true>(h, ldh, residual, ldr, g, eps, M, K, q, ldq, s_tok, s)
                  : launch_rmsnorm_add<false>(h, ldh, residual, ldr, g, eps, M, K, q, ldq, s_tok, s);
}

template <int BS, bool SMOOTH>
static hipError_t launch_silu_bs(const uint16_t* gu, int64_t ldgu, const float* smooth, int64_t M,
                                 int64_t I, int8_t* q, int64_t ldq, float* s_tok, hipStream_t s) {
  const int64_t per = (I / 8 + BS - 1) / BS;
#define W8A8_SILU(NVV)                                                                          \
  hipLaunchKernelGGL((silu_mul_quantize_kernel<BS, NVV, SMOOTH>), dim3((unsigned)M), dim3(BS), \
                     0, s, gu, ldgu, smooth, (int)I, q, ldq, s_tok)
  if (per <= 1) W8A8_SILU(1);
  else if (per <= 2) W8A8_SILU(2);
  else if (per <= 4) W8A8_SILU(4);
  else W8A8_SILU(8);
#undef W8A8_SILU
  return hipGetLastError();
}

template <bool SMOOTH>
static hipError_t launch_silu_sm(const uint16_t* gu, int64_t ldgu, const float* smooth, int64_t M,
                                 int64_t I, int8_t* q, int64_t ldq, float* s_tok, hipStream_t s) {
  switch (producer_threads(M, I)) {
    case 256: return launch_silu_bs<256, SMOOTH>(gu, ldgu, smooth, M, I, q, ldq, s_tok, s);
    case 512: return launch_silu_bs<512, SMOOTH>(gu, ldgu, smooth, M, I, q, ldq, s_tok, s);
    default: return launch_silu_bs<1024, SMOOTH>(gu, ldgu, smooth, M, I, q, ldq, s_tok, s);
  }
}

hipError_t launch_silu_mul_quantize(const uint16_t* gu, int64_t ldgu, const float* smooth,
                                    int64_t M, int64_t I, int8_t* q, int64_t ldq, float* s_tok,
                                    hipStream_t s) {
  return smooth ? launch_silu_sm<true>(gu, ldgu, smooth, M, I, q, ldq, s_tok, s)
                : launch_silu_sm<false>(gu, ldgu, smooth, M, I, q, ldq, s_tok, s);
}

hipError_t launch_fold_gamma(const float* gamma, const float* smooth, int64_t K, float* g,
                             hipStream_t s) {
  hipLaunchKernelGGL(fold_gamma_kernel, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, s, gamma,
                     smooth, K, g);
  return hipGetLastError();
}

hipError_t launch_residual_add(uint16_t* h, int64_t ldh, const uint16_t* r, int64_t ldr,
                               int64_t M, int64_t K, hipStream_t s) {
  const dim3 grid((unsigned)((K / 8 + 255) / 256), (unsigned)(M < 65535 ? M : 65535));
  hipLaunchKernelGGL(residual_add_kernel, grid, dim3(256), 0, s, h, ldh, r, ldr, M, (int)K);
  return hipGetLastError();
}

}  // namespace w8a8
