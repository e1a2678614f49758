/* Checks the FP8 step's quotient sequence against IEEE fp32 division.
 *
 * q0 = RN(a * r), e = fma(b, q0, -a), q1 = fma(-e, r, q0) with r = RN(1/b).
 * For numerators with `mbits` fraction bits (7: bfloat16, 10: float16) at
 * exponent `aexp`, and every divisor significand in [lo, hi) (step `step`) at
 * exponent `bexp`, counts results that differ from a / b (sign included).
 * Usage: quotient_check mbits aexp bexp lo hi step
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(int argc, char** argv) {
  if (argc != 7) return 2;
  const int mbits = atoi(argv[1]), aexp = atoi(argv[2]), bexp = atoi(argv[3]);
  const long lo = atol(argv[4]), hi = atol(argv[5]), step = atol(argv[6]);
  long bad = 0, total = 0;
  for (long bm = lo; bm < hi; bm += step) {
    const float b = f_of(((uint32_t)(bexp + 127) << 23) | (uint32_t)bm);
    const float r = 1.0f / b;
    for (int am = 0; am < (1 << mbits); ++am) {
      for (int s = 0; s < 2; ++s) {
        const float a = f_of(((uint32_t)s << 31) | ((uint32_t)(aexp + 127) << 23) | ((uint32_t)am << (23 - mbits)));
        const float q0 = a * r;
        const float e = fmaf(b, q0, -a);
        const float q1 = fmaf(-e, r, q0);
        ++total;
        if (u_of(q1) != u_of(a / b)) ++bad;
      }
    }
  }
  printf("%ld %ld\n", total, bad);
  return 0;
}
