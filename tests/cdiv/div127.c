/* The decode kernels form fp32(s / 127) as q0 = s * fp32(1/127) corrected
 * once by its fused remainder: fmaf(fmaf(-q0, 127, s), fp32(1/127), q0).
 * This program compares that with the correctly rounded quotient s / 127.0f
 * for every finite fp32 bit pattern whose index is a multiple of STRIDE
 * (argument 1, default 1) and prints the number of patterns that differ
 * other than in the sign of a zero result. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int main(int argc, char **argv) {
  const int64_t stride = argc > 1 ? atoll(argv[1]) : 1;
  const float c = 1.0f / 127.0f;
  long long bad = 0, tested = 0;
#pragma omp parallel for reduction(+ : bad, tested) schedule(static)
  for (int64_t u = 0; u < (1LL << 32); u += stride) {
    const uint32_t bits = (uint32_t)u;
    float x;
    memcpy(&x, &bits, 4);
    if (!isfinite(x)) continue;
    const float ref = x / 127.0f;
    const float q0 = x * c;
    const float got = fmaf(fmaf(-q0, 127.0f, x), c, q0);
    ++tested;
    if (memcmp(&ref, &got, 4) != 0 && !(ref == 0.0f && got == 0.0f)) ++bad;
  }
  printf("%lld %lld\n", tested, bad);
  return 0;
}
