// plsh_host.cpp -- host half of libplsh: hash sampler, table validator, work
// counter and the thread-local error string.  Needs no GPU.
//
// "Positional LSH: Binary Block Matrix Approximation for Attention with Linear
// Biases": Methodology §1 (random binning of integer positions into contiguous
// bins), §2 (Gamma law of the bins; M~ = mean of s i.i.d. masks), §3 (cost of
// the reduction to s short-context attentions).

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "plsh_binning.h"
#include "plsh_draw.h"
#include "plsh_internal.h"

namespace plsh {

namespace {
thread_local std::string g_last_error;
}

plsh_status fail(plsh_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

void clear_error() { g_last_error.clear(); }

namespace {

// Block starts of one hash: 0, each bin change, n.  Walks block by block.
void hash_starts(int32_t n, double delta, double u, std::vector<int32_t> &out) {
  out.push_back(0);
  const double rinv = 1.0 / delta;
  int32_t x = 0;
  while (x < n) {
    int32_t y = block_hi(x, n, delta, u, bin_of_r(x, delta, u, rinv), rinv);
    out.push_back(y);
    x = y;
  }
}

bool finite_pos(double v) { return isfinite(v) && v > 0.0; }

}  // namespace
}  // namespace plsh

using namespace plsh;

extern "C" plsh_status plsh_sample_tables(uint64_t seed, int32_t n, int32_t heads,
                                          const double *sigma, int32_t s, double *params,
                                          int32_t *offsets, int32_t *starts,
                                          int64_t starts_capacity, int64_t *starts_needed) {
  clear_error();
  if (!sigma || !params || !offsets || !starts_needed)
    return fail(PLSH_ERR_ARG, "plsh_sample_tables: null pointer argument");
  if (n < 1 || heads < 1 || s < 1)
    return fail(PLSH_ERR_ARG, "plsh_sample_tables: need n >= 1, heads >= 1, s >= 1 (got %d, %d, %d)",
                n, heads, s);
  if (starts && starts_capacity < 0)
    return fail(PLSH_ERR_ARG, "plsh_sample_tables: negative starts_capacity");
  for (int32_t h = 0; h < heads; ++h)
    if (!draw::sigma_in_range(sigma[h]))
      return fail(PLSH_ERR_ARG, "plsh_sample_tables: sigma[%d] = %g outside [%g, %g]", h, sigma[h],
                  draw::kSigmaMin, draw::kSigmaMax);

  const int64_t rows = (int64_t)heads * s;
  std::vector<int32_t> all;
  std::vector<int32_t> one;
  offsets[0] = 0;
  for (int32_t h = 0; h < heads; ++h) {
    const double sg = sigma[h];
    for (int32_t k = 0; k < s; ++k) {
      double delta, u;  // Erlang-2 = Gamma(2, sigma) pitch, offset in [0, delta)
      draw::hash_params(seed, (uint64_t)h, (uint64_t)k, sg, &delta, &u);
      const int64_t r = (int64_t)h * s + k;
      // (holds for every sigma in range; checked so that no draw can reach
      // the scan otherwise)
      if (!(isnormal(delta) && delta > 0.0 && u >= 0.0 && u < delta))
        return fail(PLSH_ERR_ARG, "plsh_sample_tables: sigma[%d] drew an unusable pitch %g (sample %d)", h,
                    delta, k);
      params[2 * r] = delta;
      params[2 * r + 1] = u;
      one.clear();
      hash_starts(n, delta, u, one);
      if ((int64_t)all.size() + (int64_t)one.size() > (int64_t)INT32_MAX)
        return fail(PLSH_ERR_CAPACITY, "plsh_sample_tables: table exceeds 2^31 entries");
      all.insert(all.end(), one.begin(), one.end());
      offsets[r + 1] = (int32_t)all.size();
    }
  }
  (void)rows;
  *starts_needed = (int64_t)all.size();
  if (!starts) return PLSH_OK;
  if (starts_capacity < (int64_t)all.size())
    return fail(PLSH_ERR_CAPACITY, "plsh_sample_tables: starts needs %lld entries, capacity %lld",
                (long long)all.size(), (long long)starts_capacity);
  memcpy(starts, all.data(), all.size() * sizeof(int32_t));
  return PLSH_OK;
}

extern "C" plsh_status plsh_build_tables(int32_t n, int32_t heads, int32_t s, const double *params,
                                         int32_t *offsets, int32_t *starts, int64_t starts_capacity,
                                         int64_t *starts_needed) {
  clear_error();
  if (!params || !offsets || !starts_needed) return fail(PLSH_ERR_ARG, "plsh_build_tables: null pointer argument");
  if (n < 1 || heads < 1 || s < 1)
    return fail(PLSH_ERR_ARG, "plsh_build_tables: need n >= 1, heads >= 1, s >= 1 (got %d, %d, %d)", n, heads, s);
  if (starts && starts_capacity < 0) return fail(PLSH_ERR_ARG, "plsh_build_tables: negative starts_capacity");
  const int64_t rows = (int64_t)heads * s;
  for (int64_t r = 0; r < rows; ++r) {
    const double delta = params[2 * r], u = params[2 * r + 1];
    if (!finite_pos(delta) || !isnormal(delta) || !(u >= 0.0) || !(u < delta) ||
        !isfinite(((double)n + u) / delta))
      return fail(PLSH_ERR_ARG,
                  "plsh_build_tables: row %lld: need delta > 0 finite and normal, 0 <= u < delta, and finite "
                  "bins (n + u) / delta", (long long)r);
  }
  std::vector<int32_t> all, one;
  offsets[0] = 0;
  for (int64_t r = 0; r < rows; ++r) {
    one.clear();
    hash_starts(n, params[2 * r], params[2 * r + 1], one);
    if ((int64_t)all.size() + (int64_t)one.size() > (int64_t)INT32_MAX)
      return fail(PLSH_ERR_CAPACITY, "plsh_build_tables: table exceeds 2^31 entries");
    all.insert(all.end(), one.begin(), one.end());
    offsets[r + 1] = (int32_t)all.size();
  }
  *starts_needed = (int64_t)all.size();
  if (!starts) return PLSH_OK;
  if (starts_capacity < (int64_t)all.size())
    return fail(PLSH_ERR_CAPACITY, "plsh_build_tables: starts needs %lld entries, capacity %lld",
                (long long)all.size(), (long long)starts_capacity);
  memcpy(starts, all.data(), all.size() * sizeof(int32_t));
  return PLSH_OK;
}

extern "C" plsh_status plsh_validate_tables(const plsh_tables *t) {
  clear_error();
  if (!t || !t->params || !t->offsets || !t->starts)
    return fail(PLSH_ERR_ARG, "plsh_validate_tables: null pointer argument");
  if (t->n < 1 || t->heads < 1 || t->s < 1)
    return fail(PLSH_ERR_TABLE, "plsh_validate_tables: need n, heads, s >= 1");
  const int64_t rows = (int64_t)t->heads * t->s;
  if (t->offsets[0] != 0) return fail(PLSH_ERR_TABLE, "plsh_validate_tables: offsets[0] != 0");
  std::vector<int32_t> want;
  for (int64_t r = 0; r < rows; ++r) {
    const double delta = t->params[2 * r], u = t->params[2 * r + 1];
    if (!finite_pos(delta) || !(u >= 0.0) || !(u < delta))
      return fail(PLSH_ERR_TABLE, "plsh_validate_tables: row %lld: need delta > 0 finite and 0 <= u < delta",
                  (long long)r);
    const int32_t a = t->offsets[r], b = t->offsets[r + 1];
    if (b < a + 2)
      return fail(PLSH_ERR_TABLE, "plsh_validate_tables: row %lld: offsets not increasing by >= 2",
                  (long long)r);
    const int32_t *st = t->starts + a;
    if (st[0] != 0) return fail(PLSH_ERR_TABLE, "plsh_validate_tables: row %lld: first start != 0", (long long)r);
    if (st[b - a - 1] != t->n)
      return fail(PLSH_ERR_TABLE, "plsh_validate_tables: row %lld: last entry != n", (long long)r);
    for (int32_t i = 1; i < b - a; ++i)
      if (st[i] <= st[i - 1])
        return fail(PLSH_ERR_TABLE, "plsh_validate_tables: row %lld: starts not strictly increasing at %d",
                    (long long)r, i);
    want.clear();
    hash_starts(t->n, delta, u, want);
    if ((int64_t)want.size() != (int64_t)(b - a) || !std::equal(want.begin(), want.end(), st))
      return fail(PLSH_ERR_TABLE, "plsh_validate_tables: row %lld: starts differ from the bins of (delta, u)",
                  (long long)r);
  }
  return PLSH_OK;
}

extern "C" plsh_status plsh_count_work(const plsh_tables *t, int32_t causal, int64_t *pairs_alg,
                                       int64_t *pairs_distinct) {
  clear_error();
  if (!t || !t->offsets || !t->starts || !pairs_alg || !pairs_distinct)
    return fail(PLSH_ERR_ARG, "plsh_count_work: null pointer argument");
  if (t->n < 1 || t->heads < 1 || t->s < 1)
    return fail(PLSH_ERR_TABLE, "plsh_count_work: need n, heads, s >= 1");
  const int32_t n = t->n;
  int64_t alg = 0, distinct = 0;
  std::vector<int32_t> ulo(n), uhi(n);
  for (int32_t h = 0; h < t->heads; ++h) {
    std::fill(ulo.begin(), ulo.end(), n);
    std::fill(uhi.begin(), uhi.end(), 0);
    for (int32_t k = 0; k < t->s; ++k) {
      const int64_t r = (int64_t)h * t->s + k;
      const int32_t a = t->offsets[r], b = t->offsets[r + 1];
      for (int32_t e = a; e + 1 < b; ++e) {
        const int32_t lo = t->starts[e], hi = t->starts[e + 1];
        if (lo < 0 || hi > n || hi <= lo)
          return fail(PLSH_ERR_TABLE, "plsh_count_work: malformed row %lld", (long long)r);
        const int64_t L = hi - lo;
        alg += causal ? L * (L + 1) / 2 : L * L;
        for (int32_t x = lo; x < hi; ++x) {
          ulo[x] = std::min(ulo[x], lo);
          uhi[x] = std::max(uhi[x], hi);
        }
      }
    }
    for (int32_t x = 0; x < n; ++x)
      distinct += causal ? (int64_t)(x - ulo[x] + 1) : (int64_t)(uhi[x] - ulo[x]);
  }
  *pairs_alg = alg;
  *pairs_distinct = distinct;
  return PLSH_OK;
}

extern "C" const char *plsh_last_error(void) { return g_last_error.c_str(); }
