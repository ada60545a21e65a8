/* Host check of the reciprocal division the E4M3 quantization kernels use (Sol-Attn2 draft,
   "FP8 quantization": X8 = E4M3(X / s), s = max|X| / 448).  For every positive finite bf16
   max m with s = RN(m / 448) >= 2^-60 (every STRIDE-th one) and every bf16 x with |x| <= m,
   q = RN(x r) with r = RN(1 / s), corrected by Markstein's step RN(q + RN(x - q s) r), must
   equal the IEEE quotient RN(x / s) bit for bit wherever either is at least 2^-12, and stay
   below 2^-11 where the IEEE quotient is below 2^-12 (both then give the E4M3 code 0).
   Prints the number of violations; exit status 0 when there are none. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bf16(uint32_t h) {
  uint32_t u = h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

int main(int argc, char** argv) {
  const uint32_t stride = argc > 1 ? (uint32_t)atoi(argv[1]) : 1;
  long bad = 0, total = 0;
  for (uint32_t mh = 1; mh < 0x7f80; mh += stride) {
    const float m = bf16(mh);
    const float s = m / 448.0f;
    if (!(s >= 0x1p-60f)) continue;
    const float r = 1.0f / s;
    for (uint32_t h = 0; h < 65536; ++h) {
      const float x = bf16(h);
      if (isnan(x) || fabsf(x) > m) continue;
      const float ieee = x / s;
      const float q = x * r;
#ifdef PLAIN_PRODUCT
      const float mk = q;   /* no correction: must fail (the check is not vacuous) */
#else
      const float mk = fmaf(fmaf(-q, s, x), r, q);
#endif
      ++total;
      const int differ = memcmp(&ieee, &mk, 4) != 0;
      if ((differ && (fabsf(ieee) >= 0x1p-12f || fabsf(mk) >= 0x1p-12f)) ||
          (fabsf(ieee) < 0x1p-12f && fabsf(mk) >= 0x1p-11f)) {
        if (bad < 5) printf("x=%a s=%a ieee=%a reciprocal=%a\n", x, s, ieee, mk);
        ++bad;
      }
    }
  }
  printf("checked %ld quotients, %ld violations\n", total, bad);
  return bad != 0;
}
