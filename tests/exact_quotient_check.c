/* CPU check of the quantisers' exact-quotient rule (fp8_codec.h, exact_quotient):
 * for a group scale s = RN(amax / 448) with y = RN(1 / s), every element's
 * q = RN(q0 - RN(s q0 - x) y), q0 = RN(x y), must encode to the E4M3 code of
 * the correctly rounded quotient RN(x / s) that the method specifies (the tech
 * note's q = round(x / s), read as the binary32 quotient rounded to E4M3).
 *
 * Domain: every positive finite bf16 amax with s >= 2^-100 (smaller scales
 * take the division itself) and every bf16 x with |x| <= amax, both signs,
 * plus the all-zero group (amax = 0, y = 0). Two quotients give the same E4M3
 * code when their bits are equal, or when both are below 2^-11 in magnitude
 * with the same sign (E4M3's smallest subnormal is 2^-9: both round to a
 * signed zero). Exit status 0 when every pair agrees; prints the counts.
 * Arguments: [stride] -- test every stride-th amax (1 = all, the default).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bf(uint32_t b) { uint32_t u = b << 16; float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* volatile temporaries: each operation rounded once, in this order, as on the GPU */
static float exact_quotient(float x, float s, float y) {
  volatile float q0 = x * y;
  volatile float nx = -x;
  volatile float e = fmaf(s, q0, nx);
  volatile float ne = -e;
  volatile float q = fmaf(ne, y, q0);
  return q;
}

static int same_code(float q, float ref) {
  return bits(q) == bits(ref) || (fabsf(q) < 0x1p-11f && fabsf(ref) < 0x1p-11f && signbit(q) == signbit(ref));
}

int main(int argc, char** argv) {
  const int stride = argc > 1 ? atoi(argv[1]) : 1;
  long long pairs = 0, bad = 0, bit_diff = 0;
  /* the all-zero group */
  for (int sg = 0; sg < 2; ++sg) {
    const float x = sg ? -0.0f : 0.0f, q = exact_quotient(x, 0.0f, 0.0f);
    pairs++;
    if (bits(q) != bits(x)) { bad++; printf("all-zero group: x=%g gives %g\n", x, q); }
  }
#pragma omp parallel for schedule(dynamic, 16) reduction(+ : pairs, bad, bit_diff)
  for (uint32_t ab = 1; ab < 0x7F80; ab += stride) {
    const float amax = bf(ab);
    const float s = amax / 448.0f;
    if (s < 0x1p-100f) continue;
    const float y = 1.0f / s;
    for (uint32_t xb = 0; xb <= ab; ++xb) {
      for (int sg = 0; sg < 2; ++sg) {
        const float x = bf(xb | (sg ? 0x8000u : 0u));
        volatile float ref = x / s;
        const float q = exact_quotient(x, s, y);
        pairs++;
        if (bits(q) != bits(ref)) bit_diff++;
        if (!same_code(q, ref)) {
          bad++;
          if (bad < 5) printf("mismatch: amax=%a x=%a RN(x/s)=%a q=%a\n", amax, x, (float)ref, q);
        }
      }
    }
  }
  printf("pairs %lld, code mismatches %lld, quotient-bit differences below 2^-11 %lld\n", pairs, bad, bit_diff);
  return bad != 0;
}
