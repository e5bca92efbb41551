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

// First position of the block that holds x: the smallest y in [0, x] with
// bin(y) == bin(x) == b.  The arithmetic guess is settled with the exact
// predicate, so the answer never depends on how the guess was rounded; a
// bisection (bin is non-decreasing) finishes any case the local steps do not.
// Both probes of a step are independent, so their divisions overlap.
PLSH_HD int32_t block_lo(int32_t x, double delta, double u, double b) {
  double c = ceil(b * delta - u);
  int32_t y = (c <= 0.0) ? 0 : (c >= (double)x ? x : (int32_t)c);
  for (int it = 0; it < 4; ++it) {
    const double bl = bin_of(y > 0 ? y - 1 : 0, delta, u);
    const double by = bin_of(y, delta, u);
    if (y > 0 && bl >= b) { --y; continue; }
    if (by < b) { ++y; continue; }
    return y;
  }
  int32_t lo = 0, hi = x;  // bin(x) == b, so the answer lies in [0, x]
  while (lo < hi) {
    int32_t mid = lo + ((hi - lo) >> 1);
    if (bin_of(mid, delta, u) >= b) hi = mid; else lo = mid + 1;
  }
  return lo;
}

// One past the last position of the block that holds x: the smallest y in
// (x, n] with y == n or bin(y) > b, b = bin(x).
PLSH_HD int32_t block_hi(int32_t x, int32_t n, double delta, double u, double b) {
  double c = ceil((b + 1.0) * delta - u);
  int32_t y = (c <= (double)(x + 1)) ? x + 1 : (c >= (double)n ? n : (int32_t)c);
  for (int it = 0; it < 4; ++it) {
    const double bl = bin_of(y - 1, delta, u);
    const double by = bin_of(y, delta, u);
    if (y > x + 1 && bl > b) { --y; continue; }
    if (y < n && by <= b) { ++y; continue; }
    return y;
  }
  int32_t lo = x + 1, hi = n;
  while (lo < hi) {
    int32_t mid = lo + ((hi - lo) >> 1);
    if (bin_of(mid, delta, u) > b) hi = mid; else lo = mid + 1;
  }
  return lo;
}

}  // namespace plsh
