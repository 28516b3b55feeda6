/* Exhaustive check of the quantizers' division for BF16 dividends.
 *
 * The GPU quantizers compute y = RN32(x / s) for a BF16 value x and a group scale s from
 * r = RN32(1 / s) as q0 = RN32(x * r), e = RN32(q0 * s - x), y = RN32(q0 - e * r) (fused
 * multiply-adds).  This program compares that y with the correctly rounded quotient,
 * found by integer division, for every BF16 significand (x in [1, 2), 128 values) and
 * every FP32 significand of s (s in [1, 2), 2^23 values).  Both sides scale exactly with
 * the exponents of x and s while nothing leaves the normal range, so these pairs cover
 * every such quotient.  It also runs the negated dividend, which must give the negated
 * quotient.  Prints the number of mismatches; exit status 0 iff there are none.
 *
 * Build: gcc -O2 -ffp-contract=off [-fopenmp] division_exhaustive.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static uint32_t bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

/* RN32(xm * 2^-7 / (sm * 2^-23)), ties to even, by integer division. */
static float exact_quotient(uint64_t xm, uint64_t sm) {
  const uint64_t num = xm << 41;
  const uint64_t q = num / sm, rem = num % sm; /* q in (2^24, 2^26) */
  const int len = 64 - __builtin_clzll(q);
  const int sh = len - 24;
  uint64_t keep = q >> sh;
  const uint64_t low = q & ((1ull << sh) - 1), half = 1ull << (sh - 1);
  if (low > half || (low == half && (rem != 0 || (keep & 1)))) keep++;
  return ldexpf((float)keep, sh - 25);
}

static float one_correction(float x, float s, float r) {
  const float q0 = x * r;
  const float en = fmaf(q0, s, -x);
  return fmaf(-en, r, q0);
}

int main(void) {
  unsigned long long mismatches = 0, checked = 0;
#pragma omp parallel for reduction(+ : mismatches, checked) schedule(dynamic, 4096)
  for (long sm = 1l << 23; sm < (1l << 24); ++sm) {
    const float s = ldexpf((float)sm, -23);
    const float r = 1.0f / s;
    for (uint64_t xm = 128; xm < 256; ++xm) {
      const float x = ldexpf((float)xm, -7);
      const float want = exact_quotient(xm, (uint64_t)sm);
      checked += 2;
      if (bits(one_correction(x, s, r)) != bits(want)) mismatches++;
      if (bits(one_correction(-x, s, r)) != bits(-want)) mismatches++;
    }
  }
  printf("%llu mismatches in %llu quotients\n", mismatches, checked);
  return mismatches != 0;
}
