/* Checks, with IEEE fp32 arithmetic on the host, the identity the encode and
 * fit kernels use to normalize a weight w by its row scale s (an fp16 value):
 *   y = RN(1/s), q0 = RN(w * y), rem = fma(-q0, s, w), q = RN(rem * y + q0)
 *   =>  q == RN(w / s)
 * (Markstein's correction step with a correctly rounded reciprocal).
 * Mode 0: every fp32 significand of w against every fp16 significand of s,
 *         both in [1, 2) (the identity is scale-invariant away from the
 *         subnormal range and overflow).
 * Mode 1: the edges of the range the kernels use it in, |w| in [2^-100, 2^100]
 *         with s at the fp16 extremes (subnormal 2^-24 .. 65504), on a strided
 *         subset of significands, both signs.
 * Prints "pairs <n> mismatches <m>". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static long long check(float w, float s, long long *bad) {
  const float y = 1.0f / s;
  const float q0 = w * y;
  const float rem = fmaf(-q0, s, w);
  const float q = fmaf(rem, y, q0);
  const float ref = w / s;
  if (to_bits(q) != to_bits(ref)) {
    if (*bad < 4) printf("mismatch w=%a s=%a q=%a ref=%a\n", w, s, q, ref);
    ++*bad;
  }
  return 1;
}

int main(int argc, char **argv) {
  const int mode = argc > 1 ? atoi(argv[1]) : 0;
  long long pairs = 0, bad = 0;
  if (mode == 0) {
#pragma omp parallel for reduction(+ : pairs, bad) schedule(dynamic)
    for (int ms = 0; ms < 1024; ++ms) {
      const float s = 1.0f + (float)ms / 1024.0f;
      long long b = 0, n = 0;
      for (uint32_t mw = 0; mw < (1u << 23); ++mw) n += check(from_bits(0x3F800000u | mw), s, &b);
      pairs += n;
      bad += b;
    }
  } else {
    /* fp16 scales: normal ones at the extreme and some middle exponents (every
     * 7th significand) and subnormal ones m * 2^-24 (every 3rd m) */
    float sv[2048];
    int ns = 0;
    const int ex[] = {-14, -3, 0, 7, 15};
    for (size_t i = 0; i < sizeof ex / sizeof ex[0]; ++i)
      for (int ms = 0; ms < 1024; ms += 7) sv[ns++] = ldexpf(1.0f + (float)ms / 1024.0f, ex[i]);
    for (int m = 1; m < 1024; m += 3) sv[ns++] = ldexpf((float)m, -24);
    const float wexp[] = {0x1p-100f, 0x1p-60f, 0x1p-1f, 0x1p+40f, 0x1p+99f};
#pragma omp parallel for reduction(+ : pairs, bad) schedule(dynamic)
    for (int i = 0; i < ns; ++i) {
      long long b = 0, n = 0;
      for (size_t k = 0; k < sizeof wexp / sizeof wexp[0]; ++k)
        for (uint32_t mw = 0; mw < (1u << 23); mw += 4099) {
          const float w = wexp[k] * from_bits(0x3F800000u | mw);
          n += check(w, sv[i], &b);
          n += check(-w, sv[i], &b);
        }
      pairs += n;
      bad += b;
    }
  }
  printf("pairs %lld mismatches %lld\n", pairs, bad);
  return bad != 0;
}
