/* Host sweep of the corrected quotient the kernels use for fl32(x / s):
 *   r = fl32(1 / s),  q0 = fl32(x r),  e = fma(-q0, s, x),  q = fma(e, r, q0)
 * (one residual correction of the product with the correctly rounded reciprocal; Markstein's method as in
 * Muller et al., Handbook of Floating-Point Arithmetic, division chapter), against the IEEE quotient x / s
 * of this host, bit for bit.  Scaling x or s by a power of two scales both results exactly while everything
 * stays normal, so one binade of numerator mantissas (all 2^23 of them) against a set of divisor mantissas
 * covers those binades; the exponent pairs probe the ends of the range.
 *
 * Method 1 is the other form the kernels use where the numerator is held in fp64: the fp64 product of x with
 * fl64(1 / s), rounded once to fp32.  It must equal the IEEE quotient wherever that is a normal number, and lie
 * within one step of it below.  Method 2, the plain product fl32(x fl32(1 / s)), is the contrast: it is not the
 * quotient.
 *
 * usage: sweep <n_divisors> <x_exponent> <s_exponent> [method]   (exponents of normal numbers, -126..127;
 *        method 0: corrected product (default), 1: fp64 product, 2: fp32 product)
 *        -> prints "checked mismatches" over the finite quotients
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* divisor mantissa i: a few special patterns (1.0, all ones, 1.5, all ones but the last, the last bit), then
 * SplitMix64 values */
static uint32_t divisor_mantissa(int i) {
  switch (i) {
    case 0: return 0;
    case 1: return 0x7FFFFFu;
    case 2: return 0x400000u;
    case 3: return 0x7FFFFEu;
    case 4: return 1u;
    default: {
      uint64_t z = (uint64_t)i * 0x9E3779B97F4A7C15ull;
      z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
      z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
      return (uint32_t)((z ^ (z >> 31)) & 0x7FFFFFu);
    }
  }
}

int main(int argc, char** argv) {
  if (argc != 4 && argc != 5) return 2;
  const int nd = atoi(argv[1]), ex = atoi(argv[2]), es = atoi(argv[3]), method = argc == 5 ? atoi(argv[4]) : 0;
  if (ex < -126 || ex > 127 || es < -126 || es > 127 || method < 0 || method > 2) return 2;
  long long checked = 0, bad = 0;
#pragma omp parallel for reduction(+ : checked, bad) schedule(dynamic)
  for (int i = 0; i < nd; ++i) {
    const float s = f_of(((uint32_t)(127 + es) << 23) | divisor_mantissa(i));
    const float r = 1.0f / s;
    const double r64 = 1.0 / (double)s;
    for (uint32_t m = 0; m < (1u << 23); ++m) {
      const float x = f_of(((uint32_t)(127 + ex) << 23) | m);
      const float want = x / s;
      if (!isfinite(want)) continue;
      float q;
      if (method == 1) {
        q = (float)((double)x * r64);
      } else if (method == 2) {
        q = x * r;
      } else {
        const float q0 = x * r;
        const float e = fmaf(-q0, s, x);
        q = fmaf(e, r, q0);
      }
      ++checked;
      if (method == 1 && fabsf(want) < 0x1p-126f) {
        /* a subnormal quotient: within one step (same sign) */
        const uint32_t a = u_of(q), b = u_of(want);
        bad += (a > b ? a - b : b - a) > 1;
      } else {
        bad += u_of(q) != u_of(want);
      }
    }
  }
  printf("%lld %lld\n", checked, bad);
  return 0;
}
