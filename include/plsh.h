/*
 * plsh.h -- C ABI of the Positional-LSH ALiBi attention library (libplsh.so).
 *
 * Method: "Positional LSH: Binary Block Matrix Approximation for Attention
 * with Linear Biases" (Wolfson & Wagner), technical-summary pages.
 *   Methodology §1: the ALiBi bias L*_ij = exp(-|i-j|/sigma) is a Laplacian
 *     kernel on positions; random binning of integer positions gives hashes h
 *     whose 0/1 same-bin masks M(h) are contiguous block-diagonal and satisfy
 *     L* = E_h[M(h)].
 *   Methodology §2 (Theorem 2.1): M~ = (1/s) sum_k M(h_k) approximates L*;
 *     blocks stay short (b_max ~ sigma log log n); the bins follow a Gamma law.
 *   Methodology §3 (Theorem 2.2): ALiBi attention reduces to s randomized
 *     short-context attentions without positional bias, in near-linear time.
 *
 * The estimator computed here is the ratio of sums
 *   T~ = D~^-1 (A o M~ o C) V,  D~ = diag((A o M~ o C) 1),  A = exp(Q K^T),
 * with C the optional causal mask and logits q.k taken with scale 1.
 *
 * Conventions shared by every entry point:
 *   - Every call returns a plsh_status; nothing throws across the ABI, and
 *     plsh_last_error() describes a non-OK status.  PLSH_ERR_ARG,
 *     PLSH_ERR_TABLE, PLSH_ERR_UNSUPPORTED and PLSH_ERR_CAPACITY come from the
 *     argument checks, before any device work is enqueued.  PLSH_ERR_HIP can
 *     come after part of a call's work is on the stream (a launch that fails
 *     after the block-edge pre-pass, or after some of the unfused form's
 *     per-sample passes): the outputs are then undefined, and the work
 *     already enqueued still runs and reads the buffers.
 *   - Host pointers are read during the call only; the library keeps no
 *     reference to any caller buffer after it returns (device work enqueued on
 *     `stream` reads device buffers until it completes: they must stay alive
 *     until then).
 *   - Device memory: plsh_alibi_attention on the bf16 path takes a workspace
 *     of heads * ceil(n/32) * (1040 + 16 * E) bytes, E = s + 16 rounded up to
 *     even, stream-ordered on `stream` (hipMallocFromPoolAsync) and releases
 *     it on the same stream (hipFreeAsync) within the call;
 *     plsh_alibi_attention_ws takes the same workspace from the caller
 *     instead.  The ablation and backward entry points allocate their own
 *     workspaces the same way; the others allocate no device memory.  These
 *     workspaces come from a memory pool of the library's own on each device
 *     (created on first use, kept until the process ends), which holds up to
 *     1 GiB of released memory for later calls instead of returning it to
 *     the driver at each synchronisation.
 *   - The library keeps no state besides a thread-local error string, the
 *     thread-local kernel timer below, those pools and the static scratch of
 *     plsh_alibi_attention_noalloc.
 */
#ifndef PLSH_H
#define PLSH_H

#include <stdint.h>

/* The library is built with hidden visibility: the functions declared here
 * are its only exported symbols. */
#if defined(__GNUC__) || defined(__clang__)
#define PLSH_API __attribute__((visibility("default")))
#else
#define PLSH_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PLSH_OK = 0,
  PLSH_ERR_ARG = 1,          /* null pointer, bad size, bad sigma, aliasing       */
  PLSH_ERR_TABLE = 2,        /* malformed table or table/call mismatch            */
  PLSH_ERR_UNSUPPORTED = 3,  /* head dim / dtype / size not supported             */
  PLSH_ERR_CAPACITY = 4,     /* caller buffer too small (sampler two-call protocol)*/
  PLSH_ERR_HIP = 5           /* no HIP device, or a HIP launch/runtime error      */
} plsh_status;

typedef enum { PLSH_BF16 = 0, PLSH_F32 = 1 } plsh_dtype;

/* A HIP stream handle (hipStream_t); NULL selects the null stream. */
typedef void *plsh_stream_t;

/*
 * Boundary table of s random-binning hashes per head (a view: the caller owns
 * every array).  For head h and sample k, row r = h*s + k:
 *   params[2r] = delta (pitch, > 0), params[2r+1] = u (offset, 0 <= u < delta);
 *   bin_r(x) = floor((x + u) / delta) in IEEE binary64 (add, divide, floor);
 *   starts[offsets[r] .. offsets[r+1]) lists 0, every x in 1..n-1 with
 *   bin_r(x) != bin_r(x-1), and finally n (strictly increasing).
 * (Methodology §1: a hash partitions positions into contiguous bins.)
 * Depending on the call the arrays are host or device pointers (see below).
 */
typedef struct {
  int32_t n;
  int32_t heads;
  int32_t s;
  const double *params;    /* [heads*s][2]                                      */
  const int32_t *offsets;  /* [heads*s + 1], offsets[0] == 0                    */
  const int32_t *starts;   /* [offsets[heads*s]]                                */
} plsh_tables;

/*
 * plsh_sample_tables -- draw the hashes and build their boundary table (host).
 * Methodology §1 (random binning on positions) and §2 (Gamma law): for every
 * (head h, sample k) draws delta ~ Gamma(shape 2, scale sigma[h]) as
 * -sigma (ln U1 + ln U2) and u = delta * U3, U1, U2 in (0,1), U3 in [0,1),
 * from a SplitMix64 stream used as a counter-based generator keyed by
 * (seed, h, k): draw i = ((h << 32) | k) * 4 + j, j = 0, 1, 2.  Deterministic
 * in (seed, n, sigma[], s); sample k of head h does not depend on s.
 *   seed            generator key
 *   n               sequence length, >= 1
 *   heads, sigma    sigma[heads] (host), each in [1e-280, 1e300] (so that
 *                   every pitch is a finite normal double with finite bins)
 *   s               samples per head, >= 1
 *   params          out, host [heads*s][2]
 *   offsets         out, host [heads*s + 1]
 *   starts          out, host [starts_capacity], may be NULL
 *   starts_needed   out, host: total entries the table needs
 * Two-call protocol: with starts == NULL (or too small a capacity) params,
 * offsets and *starts_needed are written and the call returns PLSH_OK
 * (starts == NULL) or PLSH_ERR_CAPACITY (capacity too small); a second call
 * with a large enough buffer fills starts.  Needs no GPU.
 */
PLSH_API plsh_status plsh_sample_tables(uint64_t seed, int32_t n, int32_t heads, const double *sigma,
                               int32_t s, double *params, int32_t *offsets, int32_t *starts,
                               int64_t starts_capacity, int64_t *starts_needed);

/*
 * plsh_build_tables -- the boundary table of caller-given hashes: for every
 * row r = h*s + k of params ([heads*s][2] = {delta, u}, host), the block
 * starts of bin(x) = floor((x + u) / delta) (Methodology §1; the same scan as
 * plsh_sample_tables, which draws the parameters itself).  Deterministic
 * tables -- e.g. "fixed blocks" of constant width w with offset 0, every
 * sample alike (Experimental Validation: the baseline the method beats) --
 * are built this way.  Two-call protocol as plsh_sample_tables: with
 * starts == NULL it fills offsets ([heads*s + 1]) and *starts_needed; the
 * second call also fills starts.
 * Errors: PLSH_ERR_ARG (null pointer, n/heads/s < 1, a row without
 * delta > 0 finite and normal, 0 <= u < delta and (n + u) / delta finite),
 * PLSH_ERR_CAPACITY (starts_capacity
 * too small, or more than 2^31 - 1 entries).
 */
PLSH_API plsh_status plsh_build_tables(int32_t n, int32_t heads, int32_t s, const double *params,
                              int32_t *offsets, int32_t *starts, int64_t starts_capacity,
                              int64_t *starts_needed);

/*
 * plsh_validate_tables -- check a table (all arrays HOST pointers): sizes > 0,
 * every delta finite and > 0, 0 <= u < delta, offsets[0] == 0 and
 * non-decreasing, each row strictly increasing from 0 to n, and every row's
 * starts equal to the bin changes of its (delta, u) (Methodology §1: bins are
 * contiguous and non-overlapping).  Returns PLSH_ERR_TABLE on the first
 * violation.  Needs no GPU.
 */
PLSH_API plsh_status plsh_validate_tables(const plsh_tables *host_tables);

/*
 * plsh_count_work -- work counts of one batch element, summed over heads
 * (HOST table).  Methodology §3 (Theorem 2.2 cost):
 *   pairs_alg      = sum over (h, k, block of length L) of L^2 (causal:
 *                    L(L+1)/2): the literal s-short-attention pair count;
 *   pairs_distinct = sum over (h, i) of |U_h(i) & J(i)|, U_h(i) the union of
 *                    the s blocks containing i (one interval), J(i) = [0, n)
 *                    or [0, i] when causal: the nonzeros of M~ o C.
 * Needs no GPU.
 */
PLSH_API plsh_status plsh_count_work(const plsh_tables *host_tables, int32_t causal,
                            int64_t *pairs_alg, int64_t *pairs_distinct);

/*
 * plsh_alibi_attention -- the estimator T~ on the GPU (asynchronous).
 * Methodology §3 (Theorem 2.2): s randomized short-context attentions without
 * positional bias, fused over the samples: each query row i attends to the
 * union of its s blocks with integer weights c_ij = #{k : j in B_k(i)}
 * (times the causal mask), T~_i = sum_j c_ij e^{q_i.k_j} v_j /
 * sum_j c_ij e^{q_i.k_j}.
 *   q, out      DEVICE [batch][heads][n][d], contiguous
 *   k, v        DEVICE [batch][kv_heads][n][d], contiguous; query head h reads
 *               kv head h / (heads / kv_heads)
 *   dtype       element type of q, k, v and out (bf16 or fp32); accumulation
 *               is fp32; bf16 results are rounded to nearest even
 *   d           head dim: 64 or 128
 *   sigma       HOST [heads], finite and > 0: checked, and orders the heads
 *               heavy-first for scheduling; the blocks come from `boundaries`
 *   s           samples per head (== boundaries->s)
 *   boundaries  HOST struct; params is a DEVICE pointer read by the kernel
 *               (block intervals are recomputed from (delta, u) with the same
 *               binary64 predicate); offsets/starts are not read and may be
 *               NULL.  n/heads/s must match the call.
 *   causal      0 or 1
 *   stream      HIP stream for the launches
 * Kernels: bf16 (s <= 255) runs a block-edge pre-pass (per head and
 * 32-row group: sorted block ends and the diagonal tile's multiplicities,
 * into the workspace) and then the MFMA attention kernel; fp32
 * runs the one-row-per-wave VALU kernel (no workspace).
 * Buffers must be 16-byte aligned; out must not overlap q, k or v.
 * Errors: PLSH_ERR_ARG (null pointer, n < 1, batch < 1, heads or kv_heads < 1,
 * heads % kv_heads != 0, s < 1, sigma not finite or <= 0, aliasing),
 * PLSH_ERR_TABLE (boundaries mismatch), PLSH_ERR_UNSUPPORTED (d not 64/128,
 * batch*heads*n*d >= 2^31, bf16 with (n + 31)*d*2 >= 2^32, s > 255),
 * PLSH_ERR_HIP (launch error, workspace allocation failure).  Execution
 * faults surface at the caller's next synchronisation.
 */
PLSH_API plsh_status plsh_alibi_attention(const void *q, const void *k, const void *v, void *out,
                                 int32_t batch, int32_t n, int32_t heads, int32_t kv_heads,
                                 int32_t d, plsh_dtype dtype, const double *sigma, int32_t s,
                                 const plsh_tables *boundaries, int32_t causal,
                                 plsh_stream_t stream);

/*
 * plsh_attention_workspace_size -- bytes of device workspace that
 * plsh_alibi_attention_ws needs for a call with these sizes: the block-edge
 * records of the pre-pass, heads * ceil(n/32) * (1040 + 16 * E) bytes with
 * E = s + 16 rounded up to even (bf16), else 0 (the VALU
 * kernel needs none).  Host only; needs no device.
 *   bytes  HOST int64 output
 * Errors: PLSH_ERR_ARG (null pointer, n, heads or s < 1),
 * PLSH_ERR_UNSUPPORTED (unknown dtype).
 */
PLSH_API plsh_status plsh_attention_workspace_size(int32_t n, int32_t heads, int32_t s, plsh_dtype dtype,
                                          int64_t *bytes);

/*
 * plsh_alibi_attention_ws -- plsh_alibi_attention (same estimator, same
 * kernels, bitwise the same output) with the pre-pass records written to a
 * caller-owned DEVICE workspace instead of one from the stream-ordered
 * allocator, so that a caller with its own caching allocator adds no
 * allocator operations to the stream.  Methodology §3 (Theorem 2.2), as for
 * plsh_alibi_attention; every other argument is as there.
 *   workspace        DEVICE, 16-byte aligned, at least
 *                    plsh_attention_workspace_size bytes (may be NULL when
 *                    that is 0); overwritten by the call's pre-pass and read
 *                    by its attention kernel, so it must stay alive and
 *                    untouched until the stream work completes; calls that
 *                    share a workspace must be ordered (same stream).
 *   workspace_bytes  its size in bytes
 * Errors: those of plsh_alibi_attention, plus PLSH_ERR_CAPACITY (workspace
 * smaller than needed) and PLSH_ERR_ARG (null or misaligned workspace, or one
 * overlapping q, k, v or out).
 */
PLSH_API plsh_status plsh_alibi_attention_ws(const void *q, const void *k, const void *v, void *out,
                                    int32_t batch, int32_t n, int32_t heads, int32_t kv_heads,
                                    int32_t d, plsh_dtype dtype, const double *sigma, int32_t s,
                                    const plsh_tables *boundaries, int32_t causal, void *workspace,
                                    int64_t workspace_bytes, plsh_stream_t stream);

/*
 * plsh_alibi_records -- the pre-pass alone: the block-edge records of every
 * (head, 32-row group) of a table, into a caller-owned DEVICE workspace, for
 * plsh_alibi_attention_from_records.  The records are the per-row block
 * intervals of Methodology §1 (the blocks of each row in every sample, with
 * the multiplicities of the diagonal tile); they depend only on the table
 * (n, heads, s, the (delta, u) rows) and on causal, not on q, k or v, so a
 * caller whose hashes stay fixed across calls (inference with fixed tables)
 * builds them once.
 *   boundaries       HOST struct, params DEVICE (as for plsh_alibi_attention)
 *   causal           0 or 1, as the attention calls that will read them
 *   workspace        DEVICE, 16-byte aligned, at least
 *                    plsh_attention_workspace_size(n, heads, s, PLSH_BF16)
 *                    bytes; overwritten
 *   workspace_bytes  its size in bytes
 * Errors: PLSH_ERR_ARG (null pointer, misaligned workspace), PLSH_ERR_TABLE
 * (n, heads or s < 1), PLSH_ERR_UNSUPPORTED (s above 255, heads above 128),
 * PLSH_ERR_CAPACITY (workspace too small), PLSH_ERR_HIP.
 */
PLSH_API plsh_status plsh_alibi_records(const plsh_tables *boundaries, int32_t causal, void *workspace,
                               int64_t workspace_bytes, plsh_stream_t stream);

/*
 * plsh_alibi_attention_from_records -- plsh_alibi_attention_ws without its
 * pre-pass: the attention kernel alone, over records that plsh_alibi_records
 * wrote to `workspace` for the same boundaries and causal flag (then the
 * output is bitwise that of plsh_alibi_attention_ws).  Methodology §3
 * (Theorem 2.2), as for plsh_alibi_attention; every argument is as for
 * plsh_alibi_attention_ws.  bf16 with s <= 255 only (the VALU path of fp32
 * has no records).  Records of another table or shape give a wrong estimate
 * but no global access outside q, k, v, out and the workspace, and the call
 * still ends: the kernel clamps every key range it reads from them and
 * bounds every walk over their edge lists.
 * Errors: those of plsh_alibi_attention_ws, plus PLSH_ERR_UNSUPPORTED for
 * fp32.
 */
PLSH_API plsh_status plsh_alibi_attention_from_records(const void *q, const void *k, const void *v, void *out,
                                              int32_t batch, int32_t n, int32_t heads, int32_t kv_heads,
                                              int32_t d, plsh_dtype dtype, const double *sigma, int32_t s,
                                              const plsh_tables *boundaries, int32_t causal,
                                              const void *workspace, int64_t workspace_bytes,
                                              plsh_stream_t stream);

/*
 * plsh_alibi_attention_noalloc -- plsh_alibi_attention (same estimator, same
 * kernels, bitwise the same output) for callers that cannot allocate device
 * memory during the call: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The pre-pass records go to a static
 * scratch array of the library (64 MiB, allocated with the library's code
 * object on each device it runs on and held until the process ends); the
 * call allocates nothing and frees nothing.  Every argument is as for
 * plsh_alibi_attention.
 *   Limit: heads * ceil(n/32) * (1040 + 16 * E) <= 64 MiB (E = s + 16
 *   rounded up to even) on the bf16 path (e.g. 32 heads, n = 16384,
 *   s <= 56); the fp32 path uses no scratch.
 *   Concurrency: every call on one device shares that device's scratch and
 *   overwrites it (each call's pre-pass writes every record its attention
 *   kernel reads, so nothing carries over): calls whose work overlaps on one
 *   device (different streams, or threads) race and must be ordered by the
 *   caller.
 * Errors: those of plsh_alibi_attention, plus PLSH_ERR_CAPACITY (records
 * beyond the scratch size) and PLSH_ERR_UNSUPPORTED (device ordinal >= 64).
 */
PLSH_API plsh_status plsh_alibi_attention_noalloc(const void *q, const void *k, const void *v, void *out,
                                                  int32_t batch, int32_t n, int32_t heads, int32_t kv_heads,
                                                  int32_t d, plsh_dtype dtype, const double *sigma, int32_t s,
                                                  const plsh_tables *boundaries, int32_t causal,
                                                  plsh_stream_t stream);

/*
 * plsh_sample_params_device -- the hash parameters of plsh_sample_tables,
 * drawn on the GPU (Methodology §1 random binning, §2 Gamma(2, sigma)
 * pitch): params[h*s + k] = (delta, u) of sample k of head h, bit for bit
 * those plsh_sample_tables writes for the same seed (same counter-based
 * generator positions and the same IEEE double operations, including the
 * logarithm of the Erlang-2 draw).  For resampling the tables at every
 * training step on the device: the attention entry points read only params
 * (offsets and starts of a plsh_tables may be null there).
 *   seed    generator seed (one per step for per-step resampling)
 *   heads   1 .. 128; sigma HOST double [heads], each in [1e-280, 1e300]
 *           (the range plsh_sample_tables accepts)
 *   s       1 .. 255 samples per head
 *   params  DEVICE double [heads*s][2] output, 16-byte aligned
 *   stream  HIP stream for the launch (one kernel, one thread per row)
 * Errors: PLSH_ERR_ARG (null pointer, heads or s < 1, bad sigma, alignment),
 * PLSH_ERR_UNSUPPORTED (heads > 128, s > 255), PLSH_ERR_HIP (no device,
 * launch error).
 */
PLSH_API plsh_status plsh_sample_params_device(uint64_t seed, int32_t heads, const double *sigma, int32_t s,
                                      double *params, plsh_stream_t stream);

/*
 * plsh_debug_block_intervals -- writes, for every (head h, sample k, position
 * i), the block [lo, hi) containing i as recomputed on the GPU by the same
 * per-tile interval code the attention kernel runs (Methodology §1 blocks):
 *   lohi  DEVICE int32 [heads*s][n][2], (lo, hi) pairs
 * boundaries as for plsh_alibi_attention (params on the device).  Test aid:
 * the result must equal the host table bit for bit.
 */
PLSH_API plsh_status plsh_debug_block_intervals(const plsh_tables *boundaries, int32_t *lohi,
                                       plsh_stream_t stream);

/*
 * plsh_debug_attention_reference -- the estimator of plsh_alibi_attention
 * (Methodology §3, Theorem 2.2: the s block-local attentions fused as one
 * ratio of sums with weights c_ij = #{k : j in B_k(i)}) through a second,
 * independent GPU formulation: one wave per query row, the row's s block
 * intervals recomputed from (delta, u) with the binary64 predicate of
 * plsh_debug_block_intervals, c_ij counted key by key, logits and weights in
 * fp32 (exp, no matrix cores), P rounded to bf16 for the value sum on the
 * bf16 path as in the MFMA kernel.  Test aid: the same estimate computed
 * another way, and the path every fp32 call of plsh_alibi_attention takes.
 * Arguments, layouts and errors as plsh_alibi_attention (bf16 or fp32,
 * d 64 or 128, s <= 255); it launches one kernel and allocates no device
 * memory.
 */
PLSH_API plsh_status plsh_debug_attention_reference(const void *q, const void *k, const void *v, void *out,
                                           int32_t batch, int32_t n, int32_t heads, int32_t kv_heads,
                                           int32_t d, plsh_dtype dtype, const double *sigma, int32_t s,
                                           const plsh_tables *boundaries, int32_t causal,
                                           plsh_stream_t stream);

/*
 * plsh_alibi_attention_walk -- the same estimate as plsh_alibi_attention,
 * computed the literal way of Methodology §3 (Theorem 2.2): for every
 * sample k in turn, attention of each row i to its block B_k(i) alone (a
 * 0/1 mask), all samples accumulated into one online softmax per row, so
 * that out_i = sum_k sum_{j in B_k(i)} e^{q_i.k_j} v_j / sum_k sum_{j in
 * B_k(i)} e^{q_i.k_j}: the ratio of sums of the fused kernel, with each
 * in-block pair evaluated once per sample that holds it.  An ablation of the
 * sample fusion (its MFMA work is the s-walk count of plsh_count_work).
 * Arguments as plsh_alibi_attention; bf16 only, s <= 255.
 * Kernels: the block-edge pre-pass over heads*s single-sample record sets,
 * then the MFMA attention kernel looping over the samples.
 * Device memory: heads*s*ceil(n/32)*1328 bytes of records from the
 * library's pool (stream-ordered on `stream`), released within the call.
 * Errors: as plsh_alibi_attention, and PLSH_ERR_UNSUPPORTED for fp32 or when
 * heads*s*ceil(n/32) exceeds 2^31.
 */
PLSH_API plsh_status plsh_alibi_attention_walk(const void *q, const void *k, const void *v, void *out,
                                      int32_t batch, int32_t n, int32_t heads, int32_t kv_heads,
                                      int32_t d, plsh_dtype dtype, const double *sigma, int32_t s,
                                      const plsh_tables *boundaries, int32_t causal,
                                      plsh_stream_t stream);

/*
 * plsh_alibi_attention_backward -- gradients of the estimate of
 * plsh_alibi_attention for fixed tables (the pages train with the method,
 * Experimental Validation).  With P_ij = c_ij e^{q_i.k_j} / sum_l c_il
 * e^{q_i.k_l} (c from the tables, a constant) and the upstream gradient dO:
 *   dV_j = sum_i P_ij dO_i,  dS_ij = P_ij (dO_i.v_j - dO_i.O_i),
 *   dQ_i = sum_j dS_ij k_j,  dK_j = sum_i dS_ij q_i,
 * dK and dV summed over the query heads of each GQA group.
 *   dout        DEVICE [batch, heads, n, d], the dtype of q
 *   dq          DEVICE [batch, heads, n, d] output
 *   dk, dv      DEVICE [batch, kv_heads, n, d] outputs
 *   the other arguments as for plsh_alibi_attention; bf16, s <= 124.
 * Launches: the block-edge pre-pass (for causal calls one pass that writes
 * both the causal records and the non-causal ones the dK/dV kernel takes);
 * the estimator's forward kernel over those records, writing O (bf16, into
 * a buffer of the call's own) and each row's normaliser, as
 * plsh_alibi_attention_lse does; then as plsh_alibi_attention_backward_saved
 * from that output: the dQ kernel (rows as in the estimator, same records),
 * which also forms D_i = dO_i.O_i, and the dK/dV kernel (key positions in
 * place of rows, using c_ij = c_ji; one workgroup per 128 key positions of a
 * KV head, looping over that head's query heads).  The gradients are
 * therefore bitwise those of plsh_alibi_attention_lse followed by
 * plsh_alibi_attention_backward_saved.  dq, dk, dv are written whole (no
 * accumulation into them).
 * Device memory: batch*heads*n*d*2 bytes (rounded up to 256) of forward
 * output and 8 * batch*heads*ceil32(n) bytes of statistics from the
 * library's pool (stream-ordered on `stream`), released within the call,
 * plus the pre-pass workspaces.  dout, dk, dv 16-byte aligned; dq, dk, dv
 * must not overlap q, k, v, dout or each other.
 * Errors: as plsh_alibi_attention (null dout, dq, dk or dv, misalignment and
 * aliasing: PLSH_ERR_ARG), and PLSH_ERR_UNSUPPORTED for fp32 or s > 124.
 */
PLSH_API plsh_status plsh_alibi_attention_backward(const void *q, const void *k, const void *v,
                                          const void *dout, void *dq, void *dk, void *dv,
                                          int32_t batch, int32_t n, int32_t heads, int32_t kv_heads,
                                          int32_t d, plsh_dtype dtype, const double *sigma, int32_t s,
                                          const plsh_tables *boundaries, int32_t causal,
                                          plsh_stream_t stream);

/*
 * plsh_alibi_attention_lse -- plsh_alibi_attention (the same kernels, bitwise
 * the same out) that also writes each row's normaliser, the statistic a
 * later backward needs (Methodology §3, Theorem 2.2: the diagonal of
 * s D~, D~ = diag((A o M~ o C) 1)):
 *   lse2[b][h][i] = log2 sum_j c_ij e^{q_i.k_j}   (base 2; fp32)
 *   lse2        DEVICE float [batch][heads][ceil32(n)] output, 16-byte
 *               aligned; rows n .. ceil32(n)-1 of each (batch, head) get 0
 *   workspace, workspace_bytes
 *               the pre-pass workspace as for plsh_alibi_attention_ws, or
 *               NULL: then the call takes it from the stream-ordered
 *               allocator as plsh_alibi_attention does
 *   the other arguments as for plsh_alibi_attention; bf16, s <= 255.
 * Errors: as plsh_alibi_attention, plus PLSH_ERR_ARG (null, misaligned or
 * overlapping lse2; misaligned or overlapping workspace), PLSH_ERR_CAPACITY
 * (workspace too small) and PLSH_ERR_UNSUPPORTED (fp32).
 */
PLSH_API plsh_status plsh_alibi_attention_lse(const void *q, const void *k, const void *v, void *out,
                                     int32_t batch, int32_t n, int32_t heads, int32_t kv_heads,
                                     int32_t d, plsh_dtype dtype, const double *sigma, int32_t s,
                                     const plsh_tables *boundaries, int32_t causal, float *lse2,
                                     void *workspace, int64_t workspace_bytes, plsh_stream_t stream);

/*
 * plsh_alibi_attention_backward_saved -- plsh_alibi_attention_backward from a
 * saved forward: `out` and `lse2` as written by plsh_alibi_attention_lse for
 * the same q, k, v, tables and causal flag (Experimental Validation: training
 * with the method).  No forward runs: the dQ kernel forms D_i = dO_i . out_i
 * (fp32 sums of the bf16 products) from the saved output and writes it for
 * the dK/dV kernel; the other launches are plsh_alibi_attention_backward's.
 * D is taken from the bf16 output, not from the fp32 estimate: the
 * gradients differ from those with the exact D by the output's rounding
 * (relative 2^-8 per element at most).
 *   out    DEVICE [batch, heads, n, d] bf16, 16-byte aligned
 *   lse2   DEVICE float [batch][heads][ceil32(n)], 16-byte aligned
 *   the other arguments as for plsh_alibi_attention_backward.
 * Device memory: 4 * batch*heads*ceil32(n) bytes for D from the library's
 * pool (stream-ordered on `stream`), released within the call, plus the
 * pre-pass workspaces.  dq, dk, dv must not overlap any input (out and lse2
 * included).
 * Errors: as plsh_alibi_attention_backward, plus PLSH_ERR_ARG for a null or
 * misaligned out or lse2.
 */
PLSH_API plsh_status plsh_alibi_attention_backward_saved(const void *q, const void *k, const void *v,
                                                const void *out, const float *lse2,
                                                const void *dout, void *dq, void *dk, void *dv,
                                                int32_t batch, int32_t n, int32_t heads,
                                                int32_t kv_heads, int32_t d, plsh_dtype dtype,
                                                const double *sigma, int32_t s,
                                                const plsh_tables *boundaries, int32_t causal,
                                                plsh_stream_t stream);

/*
 * plsh_alibi_attention_unfused -- the same estimate computed the way the
 * pages state the reduction (Methodology §3, Theorem 2.2: s short-context
 * attentions without positional bias): for each sample k a pass over every
 * row's block B_k(i) alone, writing fp32 partials (O_k normalised over the
 * block, lse_k = ln sum_{j in B_k(i)} exp(q_i.k_j)), then a log-sum-exp
 * combine out_i = sum_k e^{lse_k} O_k / sum_k e^{lse_k}.  An ablation of the
 * sample fusion of plsh_alibi_attention (same arguments, same result up to
 * rounding); bf16 only.  Device memory: s * batch * heads * n * (d + 1) * 4
 * bytes of partials from the library's pool (stream-ordered on `stream`),
 * released within the call, plus each pass's pre-pass workspace.
 * Errors: as plsh_alibi_attention, and PLSH_ERR_UNSUPPORTED for fp32.
 */
PLSH_API plsh_status plsh_alibi_attention_unfused(const void *q, const void *k, const void *v, void *out,
                                         int32_t batch, int32_t n, int32_t heads, int32_t kv_heads,
                                         int32_t d, plsh_dtype dtype, const double *sigma, int32_t s,
                                         const plsh_tables *boundaries, int32_t causal,
                                         plsh_stream_t stream);

/*
 * plsh_exact_alibi_attention -- exact ALiBi attention, the dense comparator
 * of the estimator (Problem Statement: the O(n^2) cost the method avoids;
 * Methodology §1: the bias exp(-|i-j|/sigma) as a Laplacian kernel):
 *   out_i = sum_j exp(q_i.k_j - |i-j|/sigma_h) v_j / sum_j exp(q_i.k_j - |i-j|/sigma_h)
 * over j in [0, n), or j <= i when causal; logits with scale 1 as in
 * plsh_alibi_attention.  Every key is visited (no table, no sampling).
 *   q, k, v, out, batch, n, heads, kv_heads, d, sigma, causal, stream as for
 *   plsh_alibi_attention; dtype must be PLSH_BF16 (MFMA kernel; fp32
 *   accumulation, P rounded to bf16 for the PV product, out rounded to
 *   nearest-even bf16).
 * No device memory is allocated.  Errors: PLSH_ERR_ARG (null pointer, sizes
 * < 1, heads % kv_heads != 0, sigma not finite or <= 0, aliasing,
 * misalignment), PLSH_ERR_UNSUPPORTED (dtype not bf16, d not 64/128,
 * batch*heads*n*d >= 2^31, heads > 128), PLSH_ERR_HIP (launch error).
 */
PLSH_API plsh_status plsh_exact_alibi_attention(const void *q, const void *k, const void *v, void *out,
                                       int32_t batch, int32_t n, int32_t heads, int32_t kv_heads,
                                       int32_t d, plsh_dtype dtype, const double *sigma,
                                       int32_t causal, plsh_stream_t stream);

/*
 * plsh_kernel_timer -- measurement aid (no part of the method).  With
 * enable != 0, every later call of this thread launches each attention kernel
 * (the estimator's, the walk's, the backward's dQ and dK/dV, the exact
 * comparator's and the VALU reference's; not the block-edge pre-pass) with a
 * pair of HIP events that the dispatch itself stamps at the kernel's start
 * and end (hipExtLaunchKernelGGL: no extra packets on the stream); enable == 0
 * stops recording.  Either call discards pairs not yet read.  The events are
 * created on first use and kept for reuse by the thread.
 */
PLSH_API plsh_status plsh_kernel_timer(int32_t enable);

/*
 * plsh_kernel_timer_read -- waits for the recorded pairs of this thread,
 * writes their number to *launches and the summed elapsed time (ms) to
 * *total_ms, and discards them.  PLSH_ERR_ARG on null pointers, PLSH_ERR_HIP
 * if an event cannot be read.
 */
PLSH_API plsh_status plsh_kernel_timer_read(int32_t *launches, double *total_ms);

/* Thread-local, NUL-terminated description of the last non-OK status of this
 * thread ("" if none).  Valid until the thread's next plsh_* call. */
PLSH_API const char *plsh_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PLSH_H */
