/* The quantizers divide by a row's scale s as RN(q0 + (v - q0 s) y), with
 * y = RN(1 / s), q0 = RN(v y) and the remainder formed by an FMA. This checks
 * that the result equals the IEEE quotient RN(v / s) for v within 3 ulps of
 * every code boundary (n + 1/2) s, n in [-128, 127], and every STRIDE-th
 * significand of s in [1, 2) (the identity is scale-free while the
 * intermediates stay normal). Prints "mismatches <count> of <cases>". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(int argc, char** argv) {
  const long stride = argc > 1 ? atol(argv[1]) : 1;
  long bad = 0, cases = 0;
#pragma omp parallel for reduction(+ : bad, cases) schedule(dynamic, 1024)
  for (long m = 0; m < (1L << 23); m += stride) {
    const float s = f_of((127u << 23) | (uint32_t)m);
    volatile float one = 1.0f;
    const float y = one / s;
    for (int n = -128; n <= 127; ++n) {
      const float t = (float)((double)(n + 0.5) * (double)s);
      for (int d = -3; d <= 3; ++d) {
        const float v = f_of(u_of(t) + (uint32_t)d);
        volatile float exact = v / s;
        volatile float q0 = v * y;
        volatile float e = fmaf(-q0, s, v);
        const float q = fmaf(e, y, q0);
        ++cases;
        if (u_of(exact) != u_of(q)) ++bad;
      }
    }
  }
  printf("mismatches %ld of %ld\n", bad, cases);
  return 0;
}
