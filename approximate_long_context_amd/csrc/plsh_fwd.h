// plsh_fwd.h -- host entry of the estimator's forward kernel with 32-row
// waves (plsh_fwd.hip), called by the ABI functions in plsh_attention.hip.
#pragma once

#include <hip/hip_runtime.h>

#include <utility>

#include "plsh_internal.h"

namespace plsh {

// One forward call of the estimator over block-edge records already in `ws`
// (the pre-pass of the same call, same causal flag).
struct FwdCall {
  const void *q, *k, *v;
  void *out;
  float *save_lse2;  // optional: lse2 [batch][heads][ceil32(n)] beside out
  const void *ws;    // the records of every (head, 32-row group)
  const double *sigma;  // host [heads]: orders the work heaviest first
  int32_t batch, n, heads, kv_heads, d, s;
  bool causal;
};

// Workgroups of up to four query heads of one GQA group share their K/V
// stages when every head of the set has sigma at or below this scale.
constexpr double kSharedKvSigma = 16.0;

plsh_status launch_fwd(const FwdCall &c, hipStream_t st, std::pair<hipEvent_t, hipEvent_t> *timer,
                       const char *who);

}  // namespace plsh
