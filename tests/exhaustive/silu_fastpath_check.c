/*
 * Exhaustive check of the binary32 fast path of the SiLU-gated product used
 * by the gfx950 MLP producer.
 *
 * The product of a bf16 gate g and a bf16 up value u is
 *     m = bf16(g / (1 + e^-g) * u),
 * the real value rounded once to bf16 (the binary64 evaluation of the
 * formula rounds to the same bf16 except within about 2^-50 of a bf16
 * rounding boundary). The kernel first evaluates it in binary32:
 *     e = exp_bounded(-g)      Cody-Waite reduction with a two-part ln 2,
 *                              degree-7 Taylor polynomial (Horner, fma),
 *                              scaling by 2^n
 *     d = RN(1 + e),  c = rcp(d),  q = RN(g * c),  m32 = RN(q * u)
 * where rcp is the hardware reciprocal, documented as within 1 ulp of 1/d:
 * this program tries every binary32 value within 1 ulp of the exact 1/d
 * (the two neighbours, or the exact value and its two neighbours). For
 * |g| <= 80 the relative error of m32 is below 9 * 2^-24, so m32 lies
 * within 9 binary32 ulps of the real value. The kernel accepts
 * bf16_rne(m32) when the low 16 bits of m32 are more than 16 away from
 * 0x8000 (the bf16 rounding boundary), |m32| is in [2^-120, 2^120) and
 * |g| <= 80, or when g or u is zero (an exact zero). Everything else is
 * evaluated in binary64.
 *
 * This program runs that decision for every pair of finite bf16 values
 * (g, u), 2^32 minus the non-finite ones, and every admissible reciprocal,
 * and compares every accepted result with the binary64 evaluation (C's exp)
 * rounded exactly to bf16. It prints the number of mismatches (expected 0)
 * and the share of pairs the fast path takes (with the reciprocal rounded
 * to nearest). Build with -ffp-contract=off so that each binary32 step is
 * the one the device performs.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static uint64_t dbits(double d) { uint64_t u; memcpy(&u, &d, 8); return u; }

/* e^x for |x| <= 80: x = n ln2 + r, |r| <= ln2 / 2 + tiny; e^r by its Taylor
 * polynomial to degree 7 (remainder < 2^-26.5 relative); 2^n exactly. */
static float exp_bounded(float x) {
  const float n = rintf(x * 0x1.715476p+0f);        /* log2(e) */
  float r = fmaf(-n, 0x1.62e43p-1f, x);             /* ln 2, high part */
  r = fmaf(-n, -0x1.05c61p-29f, r);                 /* ln 2, low part */
  float p = 0x1.a01a02p-13f;                        /* 1/7! */
  p = fmaf(p, r, 0x1.6c16c2p-10f);                  /* 1/6! */
  p = fmaf(p, r, 0x1.111112p-7f);                   /* 1/5! */
  p = fmaf(p, r, 0x1.555556p-5f);                   /* 1/4! */
  p = fmaf(p, r, 0x1.555556p-3f);                   /* 1/3! */
  p = fmaf(p, r, 0.5f);
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  return ldexpf(p, (int)n);
}

static uint32_t bf16_rne_f32(float f) {
  const uint32_t u = to_bits(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

/* bf16 rounding (nearest even) of a binary64 value whose magnitude is in
 * the normal bf16 range [2^-126, 2^128): drop 45 of the 52 fraction bits. */
static uint32_t bf16_rne_f64_normal(double v) {
  const uint64_t b = dbits(v);
  const uint64_t sign = b >> 63;
  uint64_t mag = b & 0x7FFFFFFFFFFFFFFFull;
  mag += 0x0FFFFFFFFFFFull + ((mag >> 45) & 1u);
  mag &= ~((1ull << 45) - 1);
  const int e = (int)(mag >> 52) - 1023;
  if (e + 127 >= 255) return (uint32_t)(sign << 15) | 0x7F80u;
  const uint32_t fb = ((uint32_t)(e + 127) << 23) | (uint32_t)((mag >> 29) & 0x7FFFFF);
  return (uint32_t)(sign << 15) | (fb >> 16);
}

#define NC 3
static float qf[NC][65536];  /* q = g * c for each admissible reciprocal c of 1 + e^-g, or NaN */
static double s64[65536];    /* binary64 g / (1 + exp(-g)) per gate pattern */
static float uf[65536];
static double ud[65536];
static int finite_pat[65536];

int main(void) {
  for (uint32_t p = 0; p < 65536; ++p) {
    const float v = from_bits(p << 16);
    finite_pat[p] = isfinite(v);
    uf[p] = v;
    ud[p] = (double)v;
    const double g = (double)v;
    s64[p] = g / (1.0 + exp(-g));
    for (int c = 0; c < NC; ++c) qf[c][p] = NAN;
    if (fabsf(v) <= 80.0f) {
      const float d = 1.0f + exp_bounded(-v);
      const double r = 1.0 / (double)d;         /* exact to 2^-53, never a binary32 midpoint */
      const float f = (float)r;
      float cand[NC];
      int n = 0;
      if ((double)f == r) {                     /* exact: it and both neighbours */
        cand[n++] = f;
        cand[n++] = nextafterf(f, 0.0f);
        cand[n++] = nextafterf(f, 2.0f);
      } else {                                  /* the two neighbours of r */
        cand[n++] = f;
        cand[n++] = (double)f < r ? nextafterf(f, 2.0f) : nextafterf(f, 0.0f);
      }
      for (int c = 0; c < n; ++c) qf[c][p] = v * cand[c];
    }
  }
  long long mismatches = 0, accepted = 0, total = 0, in_range = 0, in_range_ok = 0;
#pragma omp parallel for schedule(dynamic, 64) \
    reduction(+ : mismatches, accepted, total, in_range, in_range_ok)
  for (int gp = 0; gp < 65536; ++gp) {
    if (!finite_pat[gp]) continue;
    const float g = uf[gp];
    for (int up = 0; up < 65536; ++up) {
      if (!finite_pat[up]) continue;
      ++total;
      const float u = uf[up];
      for (int c = 0; c < NC; ++c) {
        const float q = qf[c][gp];
        if (isnan(q)) continue;                   /* |g| > 80 or no such candidate */
        const float m = q * u;
        int ok;
        if (g == 0.0f || u == 0.0f) {
          ok = 1;
        } else {
          const float a = fabsf(m);
          const int lo = (int)(to_bits(m) & 0xFFFFu);
          const int dist = lo > 0x8000 ? lo - 0x8000 : 0x8000 - lo;
          const int range = a >= 0x1p-120f && a < 0x1p120f;
          ok = range && dist > 16;
          if (c == 0) {                           /* shares for the nearest reciprocal */
            in_range += range;
            in_range_ok += ok;
          }
        }
        if (!ok) continue;
        if (c == 0) ++accepted;
        const uint32_t fast = bf16_rne_f32(m);
        const double m64 = s64[gp] * ud[up];
        uint32_t want;
        if (m64 == 0.0) {
          want = signbit(m64) ? 0x8000u : 0u;
        } else {
          want = bf16_rne_f64_normal(m64);
        }
        if (fast != want) {
          if (mismatches < 10)
            printf("mismatch: g=%a u=%a c=%d fast=%04x want=%04x m32=%a m64=%a\n", (double)g,
                   (double)u, c, fast, want, (double)m, m64);
          ++mismatches;
        }
      }
    }
  }
  printf("%lld finite pairs, fast path taken for %lld (%.4f%%); of the %lld nonzero pairs with "
         "|g| <= 80 and |m| in [2^-120, 2^120), %.4f%%; %lld mismatches\n",
         total, accepted, 100.0 * (double)accepted / (double)total, in_range,
         100.0 * (double)in_range_ok / (double)in_range, mismatches);
  return mismatches != 0;
}
