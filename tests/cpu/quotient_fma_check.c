/* Checks, on the host, the identity the GPU row quantizer relies on: for a float32 scale
 * s >= 2^-64 and |a| <= 127 * s, the reciprocal y = RN(1/s) with one fused multiply-add
 * correction, q = RN(q0 + RN(a - s*q0) * y) with q0 = RN(a*y), equals the correctly rounded
 * quotient RN(a/s) (Markstein's theorem for division with an FMA) whenever no intermediate
 * underflows (|a| >= 2^-100 suffices: the remainder a - s*q0 then lies on a representable
 * grid), and in every case rounds to the same int8 code rint(RN(a/s)) clamped to
 * [-127, 127].  Cases: every bfloat16 value against many scales, float32 values within a few
 * ulps of half-integer multiples of the scale, and uniform float32 values.
 * Prints "<cases> <code mismatches> <quotient mismatches with |a| >= 2^-100>". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t state = 88172645463325252ull;
static uint64_t next_u64(void) {
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return state;
}
static double uniform01(void) { return (next_u64() >> 11) * (1.0 / 9007199254740992.0); }
static float from_bits(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static float clamp127(float v) { return v > 127.0f ? 127.0f : (v < -127.0f ? -127.0f : v); }

static long cases = 0, code_bad = 0, quot_bad = 0;

static void check(float a, float s) {
  volatile float exact = a / s; /* IEEE division, correctly rounded */
  const float y = 1.0f / s;
  const float q0 = a * y;
  const float r = fmaf(-s, q0, a);
  const float q = fmaf(r, y, q0);
  cases++;
  if (clamp127(rintf(exact)) != clamp127(rintf(q))) code_bad++;
  if (q != exact && fabsf(a) >= 0x1p-100f) quot_bad++;
}

int main(int argc, char** argv) {
  const long scale_draws = argc > 1 ? atol(argv[1]) : 400;
  const long near_draws = argc > 2 ? atol(argv[2]) : 40000;
  const long random_draws = argc > 3 ? atol(argv[3]) : 4000000;
  for (long t = 0; t < scale_draws; t++) {
    const float amax = (float)exp(uniform01() * 60.0 - 30.0);
    const float s = amax / 127.0f;
    if (!(s >= 0x1p-64f)) continue;
    for (uint32_t b = 0; b < 0x10000u; b++) {
      const float a = from_bits(b << 16);
      if (isfinite(a) && fabsf(a) <= amax) check(a, s);
    }
  }
  for (long t = 0; t < near_draws; t++) {
    const float amax = (float)exp(uniform01() * 40.0 - 20.0);
    const float s = amax / 127.0f;
    for (int j = 0; j < 64; j++) {
      const int n = (int)(next_u64() % 255) - 127;
      float a = (float)((n + 0.5) * (double)s);
      const int d = (int)(next_u64() % 9) - 4;
      for (int u = 0; u < abs(d); u++) a = nextafterf(a, d > 0 ? INFINITY : -INFINITY);
      if (fabsf(a) <= amax) check(a, s);
    }
  }
  for (long t = 0; t < random_draws; t++) {
    const float amax = (float)exp(uniform01() * 40.0 - 20.0);
    const float s = amax / 127.0f;
    check((float)((uniform01() * 2.0 - 1.0) * amax), s);
  }
  printf("%ld %ld %ld\n", cases, code_bad, quot_bad);
  return 0;
}
