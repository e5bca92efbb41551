// plsh_sample.hip -- the hash sampler on the GPU.
//
// "Positional LSH: Binary Block Matrix Approximation for Attention with Linear
// Biases", Methodology §1 (random binning: pitch delta, offset u) and §2
// (Gamma(2, sigma) pitch).  One thread per (head, sample) draws (delta, u)
// with the host sampler's code (plsh_draw.h): the same generator positions
// and the same sequence of IEEE double operations.  This file is compiled
// with floating-point contraction off, so that no multiply and add are fused
// into one rounding.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "plsh_draw.h"
#include "plsh_hip_status.h"
#include "plsh_internal.h"

namespace plsh {
namespace dev {

constexpr int kMaxSampleHeads = 128;

struct SampleArgs {
  uint64_t seed;
  int32_t heads, s;
  double sigma[kMaxSampleHeads];
};

__global__ __launch_bounds__(256) void sample_params_kernel(SampleArgs a, double *params) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= (int64_t)a.heads * a.s) return;
  const int h = (int)(r / a.s), k = (int)(r % a.s);
  double delta, u;
  draw::hash_params(a.seed, (uint64_t)h, (uint64_t)k, a.sigma[h], &delta, &u);
  *(double2 *)(params + 2 * r) = make_double2(delta, u);
}

}  // namespace dev
}  // namespace plsh

using namespace plsh;

extern "C" plsh_status plsh_sample_params_device(uint64_t seed, int32_t heads, const double *sigma, int32_t s,
                                                 double *params, plsh_stream_t stream) {
  static const char *who = "plsh_sample_params_device";
  clear_error();
  if (!sigma || !params) return fail(PLSH_ERR_ARG, "%s: null pointer argument", who);
  if (heads < 1 || s < 1) return fail(PLSH_ERR_ARG, "%s: need heads, s >= 1 (got %d, %d)", who, heads, s);
  if (heads > dev::kMaxSampleHeads)
    return fail(PLSH_ERR_UNSUPPORTED, "%s: heads = %d exceeds %d", who, heads, dev::kMaxSampleHeads);
  if (s > kMaxSamples) return fail(PLSH_ERR_UNSUPPORTED, "%s: s = %d exceeds %d", who, s, kMaxSamples);
  for (int32_t h = 0; h < heads; ++h)
    if (!draw::sigma_in_range(sigma[h]))
      return fail(PLSH_ERR_ARG, "%s: sigma[%d] = %g outside [%g, %g]", who, h, sigma[h], draw::kSigmaMin,
                  draw::kSigmaMax);
  if ((uintptr_t)params & 15u) return fail(PLSH_ERR_ARG, "%s: params must be 16-byte aligned", who);
  plsh_status st = have_device(who);
  if (st != PLSH_OK) return st;
  dev::SampleArgs a;
  a.seed = seed;
  a.heads = heads;
  a.s = s;
  for (int i = 0; i < dev::kMaxSampleHeads; ++i) a.sigma[i] = i < heads ? sigma[i] : 1.0;
  const int64_t rows = (int64_t)heads * s;
  hipLaunchKernelGGL(dev::sample_params_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, a, params);
  return launch_check(who);
}
