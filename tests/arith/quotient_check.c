/* Exhaustive check of the corrected float32 quotient used by the HIP
 * quantizers: with r = RN(1/m), q0 = RN(x r), e = RN(m q0 - x) (one FMA),
 * q = RN(q0 - e r) (one FMA) equals the IEEE quotient RN(x / m) bit for bit,
 * signed zeros included, for every float32 significand of x in the binades
 * given on the command line (both signs), for the eight E4M3 significands
 * m = 1 + k/8 and for m = 6. Exit status 0 iff no mismatch. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(int argc, char** argv) {
  float ms[9];
  for (int k = 0; k < 8; ++k) ms[k] = 1.0f + (float)k / 8.0f;
  ms[8] = 6.0f;
  long bad = 0;
  for (int mi = 0; mi < 9; ++mi) {
    const volatile float m = ms[mi];
    const float r = 1.0f / m;
    printf("m=%g r=0x%08x\n", (double)m, u_of(r));
    for (int a = 1; a < argc; ++a) {
      const int e = atoi(argv[a]);
      for (uint32_t sg = 0; sg < 2; ++sg)
        for (uint32_t f = 0; f < (1u << 23); ++f) {
          const float x = f_of((sg << 31) | ((uint32_t)(e + 127) << 23) | f);
          const float q0 = x * r;
          const float err = fmaf(m, q0, -x);
          const float q = fmaf(err, -r, q0);
          if (u_of(q) != u_of(x / m)) ++bad;
        }
    }
    for (uint32_t sg = 0; sg < 2; ++sg) {
      const float x = f_of(sg << 31);
      const float q0 = x * r, q = fmaf(fmaf(m, q0, -x), -r, q0);
      if (u_of(q) != u_of(x / m)) ++bad;
    }
  }
  printf("mismatches %ld\n", bad);
  return bad != 0;
}
