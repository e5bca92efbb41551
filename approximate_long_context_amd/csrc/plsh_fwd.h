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
// stages when every head of the set has sigma at or below this scale.  A
// shared stream covers the union of the heads' key ranges for the same 32
// rows; four consecutive row groups of one head add about three stages to
// their range instead, which dominates short ranges and not long ones.
// Measured on the 16k causal workload (32/8 heads, sigma 1.19 .. 256):
// kernel 0.131 ms at 16, 0.127 at 64, 0.134 at 256; with every head at
// sigma = 32, 0.137 ms at 16 and 0.116 at 64; with every head at 256,
// 0.359 ms unshared and 0.401 shared.
constexpr double kSharedKvSigma = 64.0;

plsh_status launch_fwd(const FwdCall &c, hipStream_t st, std::pair<hipEvent_t, hipEvent_t> *timer,
                       const char *who);

}  // namespace plsh
