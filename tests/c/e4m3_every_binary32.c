/*
 * Pin of the oracle's e4m3 encoder on every one of the 2^32 binary32 inputs:
 * it must agree with a second encoder written independently from the format
 * (round half to even on the dropped mantissa bits in the normal range,
 * multiples of 2^-9 rounded half to even below 2^-6, saturation at 448, sign
 * kept, NaN to 0x7F|sign) -- the same method as the bit-level encoder of
 * tests/test_oracle_e4m3.py, in C for speed.  Test code: it links the
 * oracle's library.  Prints one line; exit 0 when nothing differs.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

uint8_t oracle_e4m3_encode(double v);

static uint8_t bitlevel_encode(uint32_t u) {
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return (uint8_t)(sign | 0x7Fu); /* NaN */
  if (a >= 0x43E00000u) return (uint8_t)(sign | 0x7Eu); /* |x| >= 448, inf */
  if (a < 0x3C800000u) {                                /* |x| < 2^-6: multiples of 2^-9 */
    float x;
    memcpy(&x, &a, 4);
    return (uint8_t)(sign | (uint32_t)rintf(x * 512.0f)); /* exact product, half to even */
  }
  const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u); /* keep 3 mantissa bits, half to even */
  return (uint8_t)(sign | ((r >> 20) - (120u << 3)));
}

int main(void) {
  long long mismatches = 0;
  long long first = -1;
#pragma omp parallel for schedule(static) reduction(+ : mismatches)
  for (long long i = 0; i < (1LL << 32); ++i) {
    const uint32_t u = (uint32_t)i;
    float f;
    memcpy(&f, &u, 4);
    if (oracle_e4m3_encode((double)f) != bitlevel_encode(u)) {
      ++mismatches;
#pragma omp critical
      if (first < 0 || i < first) first = i;
    }
  }
  printf("e4m3 encode, every binary32 input: %lld inputs, %lld mismatches", 1LL << 32, mismatches);
  if (mismatches) printf(" (first 0x%08llx)", first);
  printf("\n");
  return mismatches ? 1 : 0;
}
