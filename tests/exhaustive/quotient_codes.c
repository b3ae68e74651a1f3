// Exhaustive check of the quantizer's quotient (test infrastructure, host only).
//
// The GPU quantizer forms x / s without a division per element (Markstein's correction of a
// reciprocal product, Muller et al., Handbook of Floating-Point Arithmetic, division by FMA):
//   y = RN(1 / s) once per row, q = RN(x y), r = fma(-q, s, x), q' = fma(r, y, q),
// with x and s both taken times 2^64 in rows whose amax is below 2^-60. This program checks,
// for every positive bf16 amax whose scale s = RN(amax / 448) is a normal fp32 and every bf16
// x with 0 <= x <= amax (the sign is symmetric), that q' and the correctly rounded quotient
// RN(x / s) round to the same OCP E4M3 code (round to nearest, ties to even). Negative x are
// the mirror image (every rounding here is symmetric), except x = -0, for which the chain
// gives +0: the quantizer copies the sign of x onto q', and the -0 case is checked at the end.
// Exit status 0 iff there is no mismatch. Build without contraction:
// gcc -O2 -ffp-contract=off ... -lm.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
// magnitude code of a non-negative float v <= 464
static int e4m3(float v) {
  if (v < 0x1p-6f) {                       // subnormal codes m * 2^-9, m = 0..8 (8 = 2^-6)
    const double t = (double)v * 512.0;    // exact
    double m = floor(t);
    const double fr = t - m;
    if (fr > 0.5 || (fr == 0.5 && fmod(m, 2.0) == 1.0)) m += 1.0;
    return (int)m;                          // 8 -> 0x08, the smallest normal
  }
  const uint32_t u = u_of(v);
  int e = (int)(u >> 23) - 127;            // v = 1.m * 2^e, e >= -6
  uint32_t man = u & 0x7FFFFF;
  uint32_t keep = man >> 20, rest = man & 0xFFFFF;
  if (rest > 0x80000 || (rest == 0x80000 && (keep & 1))) { keep += 1; if (keep == 8) { keep = 0; e += 1; } }
  int code = ((e + 7) << 3) | (int)keep;
  return code > 0x7E ? 0x7F : code;        // 0x7F would be NaN: flags overflow
}
int main(void) {
  long long pairs = 0, bad = 0, badbits = 0;
  for (uint32_t A = 1; A < 0x7F80; ++A) {
    const float amax = f_of(A << 16);
    const float s = amax / 448.0f;
    if (s < 1.17549435e-38f) continue;
    // rows with a tiny amax work on x 2^64 and s 2^64 (same quotient, no subnormal residuals)
    const float k = amax < 0x1p-60f ? 0x1p64f : 1.0f;
    const float ss = s * k;
    const float y = 1.0f / ss;
    for (uint32_t X = 0; X <= A; ++X) {
      const float x = f_of(X << 16);
      const float f = x / s;
      const float xs = x * k;
      const float q = xs * y;
      const float r = fmaf(-q, ss, xs);
      const float q2 = fmaf(r, y, q);
      ++pairs;
      if (u_of(q2) != u_of(f)) ++badbits;
      if (e4m3(q2) != e4m3(f)) {
        if (bad < 10) printf("code mismatch amax=%a x=%a: div %a fast %a\n", amax, x, f, q2);
        ++bad;
      }
    }
  }
  // x = -0 with any normal scale: the sign-corrected chain must give -0 (code 0x80)
  for (uint32_t A = 0x0080; A < 0x7F80; A += 0x0101) {
    const float s = f_of(A << 16) / 448.0f;
    if (s < 1.17549435e-38f) continue;
    const float y = 1.0f / s, x = -0.0f;
    const float q = x * y;
    const float q2 = copysignf(fmaf(fmaf(-q, s, x), y, q), x);
    if (u_of(q2) != 0x80000000u) {
      printf("-0 gives %a\n", q2);
      ++bad;
    }
  }
  printf("pairs %lld, code mismatches %lld (quotient bit mismatches %lld)\n", pairs, bad,
         badbits);
  return bad != 0;
}
