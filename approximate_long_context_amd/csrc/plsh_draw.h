// plsh_draw.h -- the hash draws (pitch delta and offset u of every head and
// sample), shared by the host sampler and the device sampler so that both
// produce the same bits.
//
// "Positional LSH: Binary Block Matrix Approximation for Attention with Linear
// Biases", Methodology §1 (random binning: pitch delta, offset u uniform in
// [0, delta)) and §2 (the pitch follows Gamma(2, sigma) so that the collision
// probability is the Laplacian kernel exp(-|i - j| / sigma)).
//
// Draws: SplitMix64 (Steele, Lea & Flood 2014) read as a counter-based
// generator, one stream position per (head, sample, draw); the Erlang-2 pitch
// as the sum of two exponentials, delta = -sigma (ln U1 + ln U2), U1, U2 in
// (0, 1); u = delta U3, U3 in [0, 1).
//
// ln is computed from IEEE double +, -, *, / alone (each correctly rounded on
// the host and on the GPU), in a fixed order, with contraction into fused
// multiply-adds switched off (every file that includes this header is
// compiled with -ffp-contract=off; the pragma below states it for clang):
// x = m 2^e with m in [sqrt(1/2), sqrt(2)), taken
// from the bits; f = (m - 1) / (m + 1); ln m = 2 atanh f = 2 f + 2 f (f^2 p),
// p = sum_{k=1..12} f^(2k-2) / (2k + 1) by Horner from the last term; ln x =
// (e ln2_hi + ln m) + e ln2_lo with ln2_hi = ln 2 to 32 significant bits (e
// ln2_hi is exact).  |f| <= 0.172: the series is exact to well below an ulp.
#pragma once

#include <stdint.h>
#include <string.h>

#if defined(__HIPCC__)
#define PLSH_DRAW_HD __host__ __device__ __forceinline__
#else
#define PLSH_DRAW_HD inline
#endif

#if defined(__clang__)
#define PLSH_NO_FMA_CONTRACT _Pragma("clang fp contract(off)")
#else
#define PLSH_NO_FMA_CONTRACT
#endif

namespace plsh {
namespace draw {

PLSH_DRAW_HD uint64_t splitmix64_at(uint64_t seed, uint64_t i) {
  uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

PLSH_DRAW_HD double unit_open(uint64_t z) { return ((double)(z >> 11) + 0.5) * 0x1p-53; }
PLSH_DRAW_HD double unit_halfopen(uint64_t z) { return (double)(z >> 11) * 0x1p-53; }

// The scales both samplers accept.  A pitch is sigma times e = -(ln U1 +
// ln U2), and with U1, U2 in [2^-54, 1 - 2^-54] e lies in [2^-53, 75]: for
// sigma in [kSigmaMin, kSigmaMax] every pitch is a finite normal double, its
// bins of positions below 2^31 stay finite, and u = delta U3 < delta.
constexpr double kSigmaMin = 1e-280;
constexpr double kSigmaMax = 1e300;
PLSH_DRAW_HD bool sigma_in_range(double sigma) { return sigma >= kSigmaMin && sigma <= kSigmaMax; }

// one stream position per (head, sample, draw j < 4), independent of s
PLSH_DRAW_HD uint64_t draw_index(uint64_t head, uint64_t sample, uint64_t j) {
  return ((head << 32) | sample) * 4 + j;
}

// ln x for a normal double x > 0 (the draws pass U in (0, 1)).
PLSH_DRAW_HD double series_ln(double x) {
  PLSH_NO_FMA_CONTRACT
  uint64_t bits;
  memcpy(&bits, &x, 8);
  int e = (int)((bits >> 52) & 0x7FF) - 1023;
  bits = (bits & 0x000FFFFFFFFFFFFFull) | 0x3FF0000000000000ull;  // m in [1, 2)
  double m;
  memcpy(&m, &bits, 8);
  if (m >= 0x1.6a09e667f3bcdp+0) {  // sqrt(2), rounded
    m = m * 0.5;
    e += 1;
  }
  const double f = (m - 1.0) / (m + 1.0);
  const double f2 = f * f;
  double p = 1.0 / 25.0;
  p = 1.0 / 23.0 + f2 * p;
  p = 1.0 / 21.0 + f2 * p;
  p = 1.0 / 19.0 + f2 * p;
  p = 1.0 / 17.0 + f2 * p;
  p = 1.0 / 15.0 + f2 * p;
  p = 1.0 / 13.0 + f2 * p;
  p = 1.0 / 11.0 + f2 * p;
  p = 1.0 / 9.0 + f2 * p;
  p = 1.0 / 7.0 + f2 * p;
  p = 1.0 / 5.0 + f2 * p;
  p = 1.0 / 3.0 + f2 * p;
  const double tf = 2.0 * f;
  const double lnm = tf + tf * (f2 * p);
  const double de = (double)e;
  return (de * 0x1.62e42ffp-1 + lnm) + de * -0x1.718432a1b0e26p-35;
}

// (delta, u) of sample k of head h with scale sigma.
PLSH_DRAW_HD void hash_params(uint64_t seed, uint64_t h, uint64_t k, double sigma, double *delta, double *u) {
  PLSH_NO_FMA_CONTRACT
  const double u1 = unit_open(splitmix64_at(seed, draw_index(h, k, 0)));
  const double u2 = unit_open(splitmix64_at(seed, draw_index(h, k, 1)));
  const double u3 = unit_halfopen(splitmix64_at(seed, draw_index(h, k, 2)));
  const double d = -sigma * (series_ln(u1) + series_ln(u2));
  *delta = d;
  *u = d * u3;
}

}  // namespace draw
}  // namespace plsh
