/*
 * CPU model of the quantiser kernel's quotients (tests/test_fast_quotient.py).
 *
 * The kernel encodes each element as E2M1_RNE(fl(x / s)) with s the block's
 * decoded scale times the tensor scale.  Its 16 quotients share s, so it
 * computes rs = RN(1/s) once and, per element,
 *     q = clamp(RN(x * rs), -8, 8),  y = copysign(RN(q + RN(x - q s) rs), x)
 * (two FMAs: Markstein's correction), for s in [2^-100, 2^125], and a true
 * division otherwise.  This program evaluates that sequence with the C
 * library's fmaf on many (x, s) pairs and checks, against the IEEE quotient,
 * that the E2M1 code is always the same and that y is bit-identical whenever
 * 2^-3 <= |x / s| < 8.  Pairs: random quotients over a wide exponent range,
 * x a few ulps either side of s times every E2M1 decision point with extreme
 * mantissas of s, BF16-valued x, signed zeros and quotients past 8 (up to
 * overflow).  Exit status 0 iff no pair differs.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
static uint64_t st = 0x9E3779B97F4A7C15ull;
static inline uint64_t rnd(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }
static inline float bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static inline uint32_t ubits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static long long bad = 0, tot = 0, badbits = 0;
/* E2M1 code, nearest even, saturating, sign from the sign bit (as the oracle). */
static int e2m1(float y) {
  float a = fabsf(y); int c;
  if (a <= 0.25f) c = 0; else if (a < 0.75f) c = 1; else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3; else if (a <= 2.5f) c = 4; else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6; else c = 7;
  return c | (signbit(y) ? 8 : 0);
}
static long long slow = 0;
static void check(float x, float s) {
  volatile float ref = x / s;
  if (!(s >= 0x1p-100f && s <= 0x1p125f)) { slow++; return; }  /* the kernel divides there */
  float r = 1.0f / s;
  float q = x * r;
  float qc = fminf(fmaxf(q, -8.0f), 8.0f);
  float e = fmaf(-qc, s, x);
  float q1 = copysignf(fmaf(e, r, qc), x);
  tot++;
  if (fabsf(ref) >= 0x1p-3f && fabsf(ref) < 8.0f && ubits(q1) != ubits(ref)) badbits++;
  if (e2m1(q1) != e2m1(ref)) {
    if (bad < 10) printf("code mismatch x=%a s=%a ref=%a got=%a\n", x, s, ref, q1);
    bad++;
  }
}
int main(int argc, char** argv) {
  long long n = argc > 1 ? atoll(argv[1]) : 100000000LL;
  /* 1. random s of any normal exponent in a band, random x with |x/s| in [2^-30, 8] */
  for (long long i = 0; i < n; ++i) {
    uint32_t se = 27 + (uint32_t)(rnd() % 165);           /* s exponent field 27..191 */
    float s = bits((se << 23) | (uint32_t)(rnd() & 0x7FFFFF));
    int qe = -30 + (int)(rnd() % 34);                       /* quotient exponent -30..3 */
    float xm = bits((127u << 23) | (uint32_t)(rnd() & 0x7FFFFF));  /* [1,2) */
    float x = ldexpf(xm, qe) * s;                           /* near-arbitrary x */
    x = bits(ubits(x) ^ (uint32_t)(rnd() & 7));             /* perturb low bits */
    if (rnd() & 1) x = -x;
    check(x, s);
  }
  /* 2. s with extreme mantissas (all ones, all zeros, one bit) and x on E2M1 decision points */
  const float t[] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f, 6.0f, 0.5f, 1.0f};
  for (uint32_t se = 100; se < 160; ++se) {
    const uint32_t mants[] = {0x7FFFFF, 0, 1, 0x400000, 0x7FFFFE, 0x3FFFFF, 0x555555, 0x2AAAAA};
    for (int mi = 0; mi < 8; ++mi) {
      float s = bits((se << 23) | mants[mi]);
      for (int ti = 0; ti < 10; ++ti) {
        float c = t[ti] * s;  /* x near t * s */
        uint32_t cu = ubits(c);
        for (int d = -2000; d <= 2000; ++d) { check(bits(cu + d), s); check(-bits(cu + d), s); }
      }
    }
  }
  /* 3. BF16 x (8-bit mantissa) against random s: the common input */
  for (long long i = 0; i < n; ++i) {
    float s = bits(((uint32_t)(90 + rnd() % 60) << 23) | (uint32_t)(rnd() & 0x7FFFFF));
    float x = bits((uint32_t)(rnd() & 0xFFFF0000u));
    if (!isfinite(x) || !isfinite(x / s)) continue;
    check(x, s);
  }
  /* 4. zeros, huge quotients (static scale far too small), quotients near 8 */
  for (long long i = 0; i < n / 10; ++i) {
    float s = bits(((uint32_t)(2 + rnd() % 250) << 23) | (uint32_t)(rnd() & 0x7FFFFF));
    if (!(s >= 0x1p-125f && s <= 0x1p125f)) continue;
    float x;
    switch (rnd() % 4) {
      case 0: x = (rnd() & 1) ? -0.0f : 0.0f; break;
      case 1: x = bits(((uint32_t)(1 + rnd() % 254) << 23) | (uint32_t)(rnd() & 0x7FFFFF)); break;
      case 2: x = s * bits(((uint32_t)(127 + rnd() % 6) << 23) | (uint32_t)(rnd() & 0x7FFFFF)); break;
      default: x = bits((uint32_t)(rnd() & 0x7F7FFFFFu)); break;
    }
    if (rnd() & 1) x = -x;
    if (!isfinite(x)) continue;
    check(x, s);
  }
  printf("checked %lld pairs (%lld outside the fast range): %lld code mismatches, %lld bit mismatches with 2^-3 <= |x/s| < 8\n", tot, slow, bad, badbits);
  return bad != 0 || badbits != 0;
}
