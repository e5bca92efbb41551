// plsh_binning.h -- the random-binning predicate and block search, shared by
// the host sampler and the GPU kernels so that both derive identical blocks.
//
// "Positional LSH: Binary Block Matrix Approximation for Attention with Linear
// Biases", Methodology §1: a hash h partitions the integer positions into
// contiguous bins; M(h)_ij = 1 when i and j share a bin.  Random binning
// (Rahimi-Recht) with pitch delta and offset u puts position x in bin
// floor((x + u) / delta).  The predicate is evaluated in IEEE binary64 exactly
// as written (rounded add, correctly rounded divide, floor); every step is
// monotone in x, so the bins of consecutive positions never decrease and each
// bin is a contiguous run of positions.
//
// Bin values stay doubles: for tiny pitches they exceed the int64 range.
#pragma once

#include <math.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define PLSH_HD __host__ __device__ __forceinline__
#else
#define PLSH_HD inline
#endif

namespace plsh {

PLSH_HD double bin_of(int32_t x, double delta, double u) {
  return floor(((double)x + u) / delta);
}

// The same bin without the division wherever that is provably safe.  With
// a = fl(x + u), Q = a / delta exact, D = fl(Q) the correctly rounded
// quotient and q = fl(a * rinv), rinv = fl(1 / delta): each of the three
// roundings errs by at most 2^-53 relative, so |q - D| <= 3.02 * 2^-53 |q|.
// If no integer lies within that distance of q, D and q have the same floor
// f.  The test: r = q - f (exact by Sterbenz's lemma), accepted when
// |r - 1/2| < 1/2 - 2^-50 |q|, i.e. r farther than 2^-50 |q| from 0 and 1.
// The two remaining roundings (of r - 1/2 and of the bound) err by at most
// 2^-54 together, which leaves a margin above 3.02 * 2^-53 |q| for
// |q| >= 1/10; below that f = 0 and 0 <= D < 1 anyway.  q == 0 gives
// |r - 1/2| == 1/2, |q| >= 2^49 a bound <= 0, inf and NaN a NaN: all rejected,
// so the defining division decides.  The bound is one fused multiply-add:
// its product is a power-of-two scaling, exact, so it rounds once, as the
// scaling followed by the subtraction would (one instruction fewer).
PLSH_HD double bin_of_r(int32_t x, double delta, double u, double rinv) {
  const double a = (double)x + u;
  const double q = a * rinv;
  const double f = floor(q);
  if (fabs((q - f) - 0.5) < fma(-fabs(q), 0x1p-50, 0.5)) return f;
  return floor(a / delta);
}

// The first position y in [lo, hi] with y == hi or bin(y) >= m, given that
// bin(lo - 1) < m when lo > 0 (bins never decrease, so every y' in [lo, y)
// has bin(y') < m).  The block of x starts at first_at_least(bin(x), 0, x)
// and ends before first_at_least(bin(x) + 1, x + 1, n).  The arithmetic guess
// ceil(m delta - u) is settled with the exact predicate, so the answer never
// depends on how the guess was rounded; a bisection finishes any case the
// local steps do not.  The two probes of a step are independent, so their
// arithmetic overlaps.
PLSH_HD int32_t first_at_least(double m, int32_t lo, int32_t hi, double delta, double u, double rinv) {
  const double c = ceil(m * delta - u);
  // (a NaN guess, possible only for parameters the callers reject, skips to
  // the bisection instead of converting NaN to an integer)
  const bool guess = c == c;
  int32_t y = !guess || c <= (double)lo ? lo : (c >= (double)hi ? hi : (int32_t)c);
  for (int it = 0; it < (guess ? 4 : 0); ++it) {
    const double bl = bin_of_r(y > lo ? y - 1 : lo, delta, u, rinv);
    const double by = bin_of_r(y < hi ? y : lo, delta, u, rinv);
    if (y > lo && bl >= m) { --y; continue; }
    if (y < hi && by < m) { ++y; continue; }
    return y;
  }
  int32_t a = lo, b = hi;  // answer in [a, b]: bin(a - 1) < m, and b == hi or bin(b) >= m
  while (a < b) {
    const int32_t mid = a + ((b - a) >> 1);
    if (bin_of_r(mid, delta, u, rinv) >= m) b = mid; else a = mid + 1;
  }
  return a;
}

// First position of the block that holds x (b = bin(x)).
PLSH_HD int32_t block_lo(int32_t x, double delta, double u, double b, double rinv) {
  return first_at_least(b, 0, x, delta, u, rinv);
}

// One past the last position of the block that holds x (b = bin(x)): the
// first y in (x, n] with y == n or bin(y) > b.
PLSH_HD int32_t block_hi(int32_t x, int32_t n, double delta, double u, double b, double rinv) {
  return first_at_least(b + 1.0, x + 1, n, delta, u, rinv);
}

}  // namespace plsh
