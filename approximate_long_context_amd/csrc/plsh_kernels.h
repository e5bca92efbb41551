// plsh_kernels.h -- what the kernel translation units share with the host
// dispatch (plsh_attention.hip): the argument blocks of the pre-pass, the
// 16-row MFMA kernels and the exact-ALiBi comparator, the kernel timer's
// launch helper, and one launch function per kernel family.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "plsh_device.h"
#include "plsh_internal.h"

namespace plsh {
namespace dev {

struct AttnArgs {
  const void *q;
  const void *k;
  const void *v;
  void *out;
  const double *params;
  int32_t batch, n, heads, kv_heads, s;
  int32_t groups;  // query-row tiles per (batch, head)
  int32_t pstride;  // rows of params between consecutive heads (s for a whole table)
  // when o32 is set, the MFMA kernel writes fp32 O ([batch, heads, n, d]) and
  // the row's natural-log sum lse = ln sum_j c_ij exp(q_i.k_j) ([batch, heads,
  // n]) instead of bf16 out
  float *o32;
  float *lse;
  // backward: the upstream gradient dO ([batch, heads, n, d], the dtype of
  // q), each row's normaliser in log2 units lse2 = log2 sum_j c_ij 2^(q_i.k_j
  // log2 e), and D_i = dO_i . O_i, both [batch, heads, ns] with ns = n rounded
  // up to a multiple of 32 (rows n .. ns - 1 hold 0); the dQ and dK/dV
  // kernels read them (lse2, dvec).
  const void *dout;
  const float *lse2;
  const float *dvec;
  float *stat_dvec;
  // when set, the forward kernel writes lse2 ([batch, heads, ns], rows
  // n .. ns - 1 hold 0) beside out: the statistic a later backward reads
  float *save_lse2;
  // the dQ kernel forms D = dO . O from this forward output ([batch, heads,
  // n, d], bf16) itself and writes it to stat_dvec (rows n .. ns - 1: 0) for
  // the dK/dV kernel
  const void *saved_out;
  int32_t order[kMaxHeadsArg];  // head processed in slot i, heaviest sigma first
};

// Exact ALiBi attention (plsh_exact.hip).
struct ExactArgs {
  const void *q;
  const void *k;
  const void *v;
  void *out;
  int32_t batch, n, heads, kv_heads;
  int32_t groups;                 // query-row tiles per (batch, head)
  float slope2[kMaxHeadsArg];     // log2(e) / sigma_h
};

}  // namespace dev

// The event pair for the next timed attention launch, or nullptr when the
// kernel timer is off (plsh_attention.hip).
std::pair<hipEvent_t, hipEvent_t> *timer_slot();

// kernel launch, stamping the timer's events when tm is set
template <typename... Args, typename... P>
void launch_k(void (*kern)(Args...), dim3 grid, dim3 block, size_t shm, hipStream_t st,
              std::pair<hipEvent_t, hipEvent_t> *tm, P... p) {
  if (tm) hipExtLaunchKernelGGL(kern, grid, block, (uint32_t)shm, st, tm->first, tm->second, 0u, p...);
  else hipLaunchKernelGGL(kern, grid, block, shm, st, p...);
}

// plsh_prepass.hip: the block-edge records (non-causal with ws_causal set:
// both record sets in one pass), the VALU kernel, the interval dump.
plsh_status launch_edges(const dev::AttnArgs &a, bool causal, hipStream_t st, const char *who, void *ws,
                         void *ws_causal = nullptr);
plsh_status launch_valu(const dev::AttnArgs &a, int d, plsh_dtype dtype, int causal, hipStream_t st,
                        const char *who);
plsh_status launch_debug_intervals(const plsh_tables *bt, int32_t *lohi, hipStream_t st, const char *who);

// plsh_mfma16.hip: one 16-row MFMA kernel over records ws (mode 0: the
// estimator, 1: backward dQ, 2: backward dK/dV into dk, dv, 3: the per-sample
// walk), and the log-sum-exp combine of the unfused form.
plsh_status launch_attn(const dev::AttnArgs &a, int d, int causal, hipStream_t st, const char *who, int mode,
                        const void *ws, void *dk = nullptr, void *dv = nullptr);
plsh_status launch_combine(const float *o32, const float *lse, int s, int64_t rows, int d, void *out,
                           hipStream_t st, const char *who);

// plsh_exact.hip
plsh_status launch_exact(const dev::ExactArgs &a, int d, int causal, hipStream_t st, const char *who);

}  // namespace plsh
