// Driver for the host half of libplsh (plsh_host.cpp) built with
// AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py.  It calls every host entry point: the hash
// sampler and its two-call protocol (Methodology §1 random binning, §2 Gamma
// pitch), the table builder on near-integer quotients, the validator on good
// and corrupted tables, the work counts (Methodology §3 cost), and the error
// paths.  Exits 0 when every check holds; the sanitizers abort on any
// invalid access or undefined behaviour.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "../include/plsh.h"

static int failures = 0;
#define CHECK(c)                                                          \
  do {                                                                    \
    if (!(c)) {                                                           \
      fprintf(stderr, "check failed at line %d: %s (%s)\n", __LINE__, #c, \
              plsh_last_error());                                         \
      ++failures;                                                         \
    }                                                                     \
  } while (0)

struct Table {
  int32_t n, heads, s;
  std::vector<double> params;
  std::vector<int32_t> offsets, starts;
  plsh_tables view() const {
    return plsh_tables{n, heads, s, params.data(), offsets.data(), starts.data()};
  }
};

static Table sample(uint64_t seed, int32_t n, const std::vector<double> &sigma, int32_t s) {
  Table t{n, (int32_t)sigma.size(), s, {}, {}, {}};
  t.params.resize((size_t)t.heads * s * 2);
  t.offsets.resize((size_t)t.heads * s + 1);
  int64_t need = -1;
  CHECK(plsh_sample_tables(seed, n, t.heads, sigma.data(), s, t.params.data(), t.offsets.data(), nullptr, 0,
                           &need) == PLSH_OK);
  CHECK(need == t.offsets.back());
  if (need > 1) {  // a buffer one entry short is refused
    std::vector<int32_t> small((size_t)need - 1);
    CHECK(plsh_sample_tables(seed, n, t.heads, sigma.data(), s, t.params.data(), t.offsets.data(), small.data(),
                             (int64_t)small.size(), &need) == PLSH_ERR_CAPACITY);
  }
  t.starts.resize((size_t)need);
  CHECK(plsh_sample_tables(seed, n, t.heads, sigma.data(), s, t.params.data(), t.offsets.data(), t.starts.data(),
                           need, &need) == PLSH_OK);
  return t;
}

int main() {
  const int32_t n = 3001;
  const std::vector<double> sig = {1e-3, 0.7, 1.19, 4.0, 64.0, 1e12};
  Table t = sample(123456789ull, n, sig, 11);
  plsh_tables v = t.view();
  CHECK(plsh_validate_tables(&v) == PLSH_OK);
  for (size_t r = 0; r + 1 < t.offsets.size(); ++r) {
    CHECK(t.starts[(size_t)t.offsets[r]] == 0);
    CHECK(t.starts[(size_t)t.offsets[r + 1] - 1] == n);
  }
  int64_t alg = -1, distinct = -1;
  CHECK(plsh_count_work(&v, 0, &alg, &distinct) == PLSH_OK && alg >= distinct && distinct >= n);
  CHECK(plsh_count_work(&v, 1, &alg, &distinct) == PLSH_OK && alg >= distinct && distinct >= n);
  // range ends of sigma, n = 1, the largest s
  Table e = sample(~0ull, 1, {1e-280, 1e300}, 255);
  plsh_tables ev = e.view();
  CHECK(plsh_validate_tables(&ev) == PLSH_OK);
  // corrupted tables are refused
  {
    Table c = t;
    c.starts[1] = c.starts[0];
    plsh_tables cv = c.view();
    CHECK(plsh_validate_tables(&cv) == PLSH_ERR_TABLE);
    Table d = t;
    d.params[1] = d.params[0] * 2.0;
    plsh_tables dv = d.view();
    CHECK(plsh_validate_tables(&dv) == PLSH_ERR_TABLE);
    Table f = t;
    f.offsets[3] = f.offsets[2] - 1;
    plsh_tables fv = f.view();
    CHECK(plsh_validate_tables(&fv) == PLSH_ERR_TABLE);
  }
  // the builder on exact and near-integer quotients
  {
    std::vector<double> prm;
    for (double d0 : {3.0, 7.0, 10.0, 2.5, 1.0 / 3.0, 1e-3}) {
      for (double dl : {d0, nextafter(d0, 0.0), nextafter(d0, 1e9)}) {
        for (double u : {0.0, dl / 2.0, nextafter(dl, 0.0)}) {
          prm.push_back(dl);
          prm.push_back(u);
        }
      }
    }
    const int32_t rows = (int32_t)(prm.size() / 2);
    std::vector<int32_t> off((size_t)rows + 1);
    int64_t need = -1;
    CHECK(plsh_build_tables(4000, rows, 1, prm.data(), off.data(), nullptr, 0, &need) == PLSH_OK);
    std::vector<int32_t> st((size_t)need);
    CHECK(plsh_build_tables(4000, rows, 1, prm.data(), off.data(), st.data(), need, &need) == PLSH_OK);
    plsh_tables bv{4000, rows, 1, prm.data(), off.data(), st.data()};
    CHECK(plsh_validate_tables(&bv) == PLSH_OK);
    double bad[2] = {2.5e-308, 0.0};
    CHECK(plsh_build_tables(100, 1, 1, bad, off.data(), nullptr, 0, &need) == PLSH_ERR_ARG);
  }
  // error paths
  int64_t need = 0;
  double prm[8];
  int32_t off[5];
  const double good[1] = {4.0}, huge[1] = {1e308}, tiny[1] = {1e-310}, nan1[1] = {NAN};
  CHECK(plsh_sample_tables(0, 10, 1, huge, 2, prm, off, nullptr, 0, &need) == PLSH_ERR_ARG);
  CHECK(plsh_sample_tables(0, 10, 1, tiny, 2, prm, off, nullptr, 0, &need) == PLSH_ERR_ARG);
  CHECK(plsh_sample_tables(0, 10, 1, nan1, 2, prm, off, nullptr, 0, &need) == PLSH_ERR_ARG);
  CHECK(plsh_sample_tables(0, 0, 1, good, 2, prm, off, nullptr, 0, &need) == PLSH_ERR_ARG);
  CHECK(plsh_sample_tables(0, 10, 1, nullptr, 2, prm, off, nullptr, 0, &need) == PLSH_ERR_ARG);
  CHECK(plsh_validate_tables(nullptr) != PLSH_OK);
  CHECK(plsh_count_work(nullptr, 0, nullptr, nullptr) != PLSH_OK);
  CHECK(strlen(plsh_last_error()) > 0);
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("host checks passed\n");
  return 0;
}
