/* Exhaustive check, over every float32 bit pattern, that the kernels' int8
 * quantiser  trunc(c + copysign(0.5 - 2^-25, c)),  c = clamp(v, -127, 127),
 * equals saturate(round-half-away-from-zero(v)) computed exactly in double.
 * Built with -O2 -ffp-contract=off (SSE float arithmetic rounds to nearest
 * even, like the GPU's default mode). Exit status 0 when every value agrees. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static int q8_kernel(float v) {
  float c = fminf(fmaxf(v, -127.f), 127.f);
  volatile float s = c + copysignf(0.49999997f, c);
  return (int)s; /* truncation toward zero */
}

static int q8_exact(float v) {
  double x = (double)v;
  double m = fabs(x), f = floor(m);
  double r = f + ((m - f) >= 0.5 ? 1.0 : 0.0);
  if (r > 127.0) r = 127.0;
  return x < 0 ? -(int)r : (int)r;
}

int main(void) {
  uint64_t bad = 0, checked = 0;
  for (uint64_t u = 0; u <= 0xFFFFFFFFull; ++u) {
    uint32_t bits = (uint32_t)u;
    float v;
    memcpy(&v, &bits, 4);
    if (isnan(v)) continue;
    ++checked;
    if (q8_kernel(v) != q8_exact(v)) {
      if (bad < 10) printf("mismatch bits=%08x v=%.9g kernel=%d exact=%d\n", bits, v, q8_kernel(v), q8_exact(v));
      ++bad;
    }
  }
  printf("checked %llu values, %llu mismatches\n", (unsigned long long)checked, (unsigned long long)bad);
  return bad != 0;
}
