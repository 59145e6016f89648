/*
 * Brute-force pin for the oracle's E2M1 rounding: for every fp32 magnitude
 * pattern in a range, find the nearest E2M1 magnitude by direct search over
 * the eight grid values (0, 0.5, 1, 1.5, 2, 3, 4, 6; OCP MX v1.0 FP4 E2M1),
 * breaking an exact tie toward the even code, and compare with the function
 * under test.  Near every tie both distances are exact in fp64.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

typedef int (*index_fn)(double);

static int nearest_even(double m) {
  static const double g[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  int best = 0;
  double bd = fabs(m - g[0]);
  for (int i = 1; i < 8; ++i) {
    const double dd = fabs(m - g[i]);
    if (dd < bd || (dd == bd && (i % 2) == 0)) { best = i; bd = dd; }
  }
  return best;
}

/* Checks bit patterns lo, lo+stride, ... < hi (as positive fp32). Returns mismatches; first one in *first_bad. */
int64_t e2m1_compare_range(index_fn fn, uint32_t lo, uint32_t hi, uint32_t stride, uint32_t* first_bad) {
  int64_t bad = 0;
  for (uint64_t b = lo; b < hi; b += stride) {
    const uint32_t bits = (uint32_t)b;
    float f;
    memcpy(&f, &bits, 4);
    if (!isfinite(f)) continue;
    const double m = (double)f;
    if (fn(m) != nearest_even(m)) {
      if (bad == 0 && first_bad) *first_bad = bits;
      ++bad;
    }
  }
  return bad;
}

int e2m1_nearest_even(double m) { return nearest_even(m); }
