/*
 * Check of the division-free rounding step used by the gfx950 quantizers.
 *
 * The code of a value v under scale S is roundf(RN(v / S)) (round half away
 * from zero), clamped to [-127, 127]. With R = RN(1 / S) the kernels compute
 * t = RN(v * R) and n = rint(t), and accept n when |t - n| < 1/2 - d,
 * d = 2^-15; otherwise they divide. Whenever |t| >= 128 the code is +-127.
 * The argument: for S in [2^-100, 2^100] and |v / S| <= 128.0001,
 * |t - RN(v / S)| <= 3 * 2^-24 * 128.0001 + 2^-148 < d, so the quotient lies
 * strictly inside (n - 1/2, n + 1/2) and rounds to n under any tie rule;
 * for |t| >= 128 the quotient exceeds 127.5 in magnitude. This program
 * exercises that claim where it is tightest: quotients within a few ulps of
 * every half-integer k + 1/2 (k = 0..127), for 2^14 pseudo-random scale
 * significands over several exponents, plus uniformly random quotients, and
 * the clamp region (|v / S| up to 2^20, static scales). It counts accepted
 * fast codes that differ from the division (expected 0) and prints how often
 * the fast path was taken.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static int clamp_code(float r) { return (int)fminf(fmaxf(r, -127.0f), 127.0f); }

/* returns the fast code, or 1000 when the fast path declines */
static int fast_code(float v, float R) {
  const float t = v * R;
  const float n = rintf(t);               /* round half even (default mode) */
  const int ok = fabsf(t - n) < 0.5f - 0x1p-15f || fabsf(t) >= 128.0f;
  return ok ? clamp_code(n) : 1000;
}

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next32(void) {             /* splitmix64 */
  uint64_t z = (state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return (uint32_t)((z ^ (z >> 31)) >> 32);
}

int main(void) {
  static const int exps[] = {-100, -60, -20, -7, 0, 5, 30, 99};
  long long bad = 0, fast = 0, total = 0;
  for (int ie = 0; ie < 8; ++ie) {
    for (int si = 0; si < 16384; ++si) {
      const uint32_t ms = next32() & 0x7FFFFFu;
      const float S = ldexpf(from_bits(0x3F800000u | ms), exps[ie]);
      const volatile float one = 1.0f;
      const float R = one / S;
      for (int k = 0; k < 128; ++k) {
        /* v near (k + 1/2) * S: walk the neighbouring binary32 values */
        const float c = (float)((k + 0.5) * (double)S);
        for (int d = -6; d <= 6; ++d) {
          for (int sg = 0; sg < 2; ++sg) {
            float v = from_bits(to_bits(c) + d);
            if (sg) v = -v;
            const int want = clamp_code(roundf(v / S));
            const int got = fast_code(v, R);
            total++;
            if (got != 1000) {
              fast++;
              if (got != want) {
                if (bad < 5) printf("mismatch v=%a S=%a got %d want %d\n", v, S, got, want);
                bad++;
              }
            }
          }
        }
      }
      for (int j = 0; j < 64; ++j) {     /* uniform quotients, then the clamp region */
        const float q = (j < 48) ? ((float)(next32() >> 8) / 16777216.0f) * 255.0f - 127.5f
                                 : ldexpf((float)(next32() >> 8) / 16777216.0f, (int)(next32() % 21));
        const float v = q * S;
        const int want = clamp_code(roundf(v / S));
        const int got = fast_code(v, R);
        total++;
        if (got != 1000) {
          fast++;
          if (got != want) {
            if (bad < 5) printf("mismatch v=%a S=%a got %d want %d\n", v, S, got, want);
            bad++;
          }
        }
      }
    }
  }
  printf("checked %lld values, fast path %lld (%.2f%%), %lld mismatches\n", total, fast,
         100.0 * fast / total, bad);
  return bad == 0 ? 0 : 1;
}
