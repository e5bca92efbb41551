// plsh_attention.hip -- the C ABI of libplsh's GPU half (gfx950): argument
// checks, workspaces (the pre-pass records from the stream-ordered
// allocator, a caller's buffer, or the static scratch of the allocation-free
// entry), the kernel timer, and the dispatch to the kernel translation units:
//   plsh_prepass.hip  block-edge records, interval dump, VALU kernel;
//   plsh_fwd.hip      the estimator's forward kernel (32-row waves);
//   plsh_mfma16.hip   unfused form, per-sample walk, backward;
//   plsh_exact.hip    dense exact-ALiBi comparator.
//
// "Positional LSH: Binary Block Matrix Approximation for Attention with Linear
// Biases" (technical-summary pages):
//   Methodology §1 -- a random-binning hash splits positions into contiguous
//     blocks; M(h)_ij = 1 when i and j share a block; L* = E_h[M(h)].
//   Methodology §2 (Theorem 2.1) -- M~ = (1/s) sum_k M(h_k); blocks stay short.
//   Methodology §3 (Theorem 2.2) -- ALiBi attention becomes s randomized
//     short-context attentions without positional bias.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <numeric>
#include <utility>
#include <vector>

#include "plsh_device.h"
#include "plsh_fwd.h"
#include "plsh_hip_status.h"
#include "plsh_internal.h"
#include "plsh_kernels.h"

namespace plsh {
namespace {


bool finite_pos(double v) { return isfinite(v) && v > 0.0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

plsh_status check_common(const void *q, const void *k, const void *v, void *out, int32_t batch,
                         int32_t n, int32_t heads, int32_t kv_heads, int32_t d, plsh_dtype dtype,
                         const double *sigma, int32_t s, const plsh_tables *bt, const char *who) {
  if (!q || !k || !v || !out || !sigma || !bt)
    return fail(PLSH_ERR_ARG, "%s: null pointer argument", who);
  if (n < 1 || batch < 1 || heads < 1 || kv_heads < 1 || s < 1)
    return fail(PLSH_ERR_ARG, "%s: need n, batch, heads, kv_heads, s >= 1", who);
  if (heads % kv_heads != 0)
    return fail(PLSH_ERR_ARG, "%s: heads (%d) must be a multiple of kv_heads (%d)", who, heads, kv_heads);
  for (int32_t h = 0; h < heads; ++h)
    if (!finite_pos(sigma[h])) return fail(PLSH_ERR_ARG, "%s: sigma[%d] must be finite and > 0", who, h);
  if (dtype != PLSH_BF16 && dtype != PLSH_F32) return fail(PLSH_ERR_UNSUPPORTED, "%s: unknown dtype", who);
  if (d != 64 && d != 128) return fail(PLSH_ERR_UNSUPPORTED, "%s: head dim %d not supported (64, 128)", who, d);
  if (s > kMaxSamples) return fail(PLSH_ERR_UNSUPPORTED, "%s: s = %d exceeds %d", who, s, kMaxSamples);
  if (heads > dev::kMaxHeadsArg)
    return fail(PLSH_ERR_UNSUPPORTED, "%s: heads = %d exceeds %d", who, heads, dev::kMaxHeadsArg);
  if ((int64_t)batch * heads * n * d >= ((int64_t)1 << 31) ||
      (int64_t)batch * kv_heads * n * d >= ((int64_t)1 << 31))
    return fail(PLSH_ERR_UNSUPPORTED, "%s: tensor has >= 2^31 elements", who);
  // (the bf16 kernels address a head's K or V rows, up to the last 32-row
  // tile's end, through 32-bit buffer offsets)
  if (dtype == PLSH_BF16 && ((int64_t)n + 31) * d * 2 >= ((int64_t)1 << 32))
    return fail(PLSH_ERR_UNSUPPORTED, "%s: n = %d too long for d = %d in bf16", who, n, d);
  if (!bt->params) return fail(PLSH_ERR_ARG, "%s: boundaries->params is null", who);
  if (bt->n != n || bt->heads != heads || bt->s != s)
    return fail(PLSH_ERR_TABLE, "%s: boundaries (n=%d, heads=%d, s=%d) do not match the call (n=%d, heads=%d, s=%d)",
                who, bt->n, bt->heads, bt->s, n, heads, s);
  const size_t esz = dtype == PLSH_F32 ? 4 : 2;
  const size_t qbytes = (size_t)batch * heads * n * d * esz;
  const size_t kbytes = (size_t)batch * kv_heads * n * d * esz;
  if (overlaps(out, qbytes, q, qbytes) || overlaps(out, qbytes, k, kbytes) || overlaps(out, qbytes, v, kbytes))
    return fail(PLSH_ERR_ARG, "%s: out overlaps q, k or v", who);
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15u)
    return fail(PLSH_ERR_ARG, "%s: buffers must be 16-byte aligned", who);
  return PLSH_OK;
}

void fill_args(dev::AttnArgs &a, const void *q, const void *k, const void *v, void *out, int32_t batch,
               int32_t n, int32_t heads, int32_t kv_heads, const double *sigma, int32_t s,
               const plsh_tables *bt) {
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.params = bt->params;
  a.batch = batch;
  a.n = n;
  a.heads = heads;
  a.kv_heads = kv_heads;
  a.s = s;
  a.groups = (n + 127) / 128;
  a.pstride = s;
  a.o32 = nullptr;
  a.lse = nullptr;
  a.dout = nullptr;
  a.lse2 = nullptr;
  a.dvec = nullptr;
  a.stat_dvec = nullptr;
  a.save_lse2 = nullptr;
  a.saved_out = nullptr;
  // heavy heads first: per-row work grows with sigma
  int idx[dev::kMaxHeadsArg];
  std::iota(idx, idx + heads, 0);
  std::stable_sort(idx, idx + heads, [&](int x, int y) { return sigma[x] > sigma[y]; });
  for (int i = 0; i < dev::kMaxHeadsArg; ++i) a.order[i] = i < heads ? idx[i] : 0;
}

// Per-thread timer of the attention kernel (measurement aid): while enabled,
// every attention kernel is launched with a pair of events that the dispatch
// itself stamps at its start and end (no extra packets on the stream).  The
// events are created on first use and reused.
struct KernelTimer {
  bool on = false;
  size_t used = 0;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev;
};
thread_local KernelTimer g_timer;

// Scratch of the allocation-free entry point: the block-edge records of one
// call in a file-scope device array (each device that loads the library
// holds its own copy until the process ends).  Host code never uses the
// array's name as an address: the address on the current device comes from
// hipGetSymbolAddress, taken once per device.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices] = {};

// The scratch array's address on the current device.
plsh_status scratch_ptr(const char *who, void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PLSH_ERR_HIP, "%s: no HIP device: %s", who, hipGetErrorString(e));
  }
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(PLSH_ERR_UNSUPPORTED, "%s: device %d beyond the %d the scratch table covers", who, dev,
                kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(PLSH_ERR_HIP, "%s: scratch address on device %d: %s", who, dev, hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PLSH_OK;
}

// Workspaces of the allocating entry points come, stream-ordered, from a
// memory pool of the library's own on each device.  The pool keeps up to
// kPoolKeepBytes of released memory for later calls; the device's default
// pool returns it to the driver at every synchronisation, so that each call
// mapped its workspace afresh (the backward from a saved forward, 16k
// Mistral-shaped layer, synchronised per call: 0.74 ms, 0.56 ms from a pool
// that keeps its memory).
// (a device whose pool cannot be made keeps the default pool)
constexpr uint64_t kPoolKeepBytes = (uint64_t)1 << 30;
std::mutex g_pool_mu;
hipMemPool_t g_pool[kMaxScratchDevices] = {};
bool g_pool_tried[kMaxScratchDevices] = {};

hipError_t pool_alloc(void **p, size_t bytes, hipStream_t st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  hipMemPool_t pool = nullptr;
  if (dev >= 0 && dev < kMaxScratchDevices) {
    std::lock_guard<std::mutex> lock(g_pool_mu);
    if (!g_pool_tried[dev]) {
      g_pool_tried[dev] = true;
      hipMemPoolProps props = {};
      props.allocType = hipMemAllocationTypePinned;
      props.handleTypes = hipMemHandleTypeNone;
      props.location.type = hipMemLocationTypeDevice;
      props.location.id = dev;
      hipMemPool_t created = nullptr;
      if (hipMemPoolCreate(&created, &props) == hipSuccess) {
        uint64_t keep = kPoolKeepBytes;
        if (hipMemPoolSetAttribute(created, hipMemPoolAttrReleaseThreshold, &keep) == hipSuccess)
          g_pool[dev] = created;
        else
          (void)hipMemPoolDestroy(created);
      }
      (void)hipGetLastError();
    }
    pool = g_pool[dev];
  }
  return pool ? hipMallocFromPoolAsync(p, bytes, pool, st) : hipMallocAsync(p, bytes, st);
}

// the event pair for the next timed launch, or nullptr when timing is off

}  // namespace

std::pair<hipEvent_t, hipEvent_t> *timer_slot() {
  if (!g_timer.on) return nullptr;
  if (g_timer.used == g_timer.ev.size()) {
    hipEvent_t b = nullptr, e = nullptr;
    if (hipEventCreate(&b) != hipSuccess || hipEventCreate(&e) != hipSuccess) {
      (void)hipGetLastError();
      if (b) (void)hipEventDestroy(b);
      return nullptr;
    }
    g_timer.ev.emplace_back(b, e);
  }
  return &g_timer.ev[g_timer.used++];
}

namespace {

// bytes of the block-edge records of every (head, 32-row group)
size_t records_bytes(int n, int heads, int s) { return (size_t)heads * ((n + 31) / 32) * dev::rec_bytes(s); }

// The records into a workspace from the library's pool (released by
// free_records).
plsh_status build_records(const dev::AttnArgs &a, bool causal, hipStream_t st, const char *who, void **ws) {
  const size_t ws_bytes = records_bytes(a.n, a.heads, a.s);
  *ws = nullptr;
  hipError_t e = pool_alloc(ws, ws_bytes, st);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    *ws = nullptr;
    return fail(PLSH_ERR_HIP, "%s: workspace allocation of %zu bytes failed: %s", who, ws_bytes,
                hipGetErrorString(e));
  }
  return launch_edges(a, causal, st, who, *ws);
}

// Causal and non-causal records in one pre-pass (the causal backward's two
// record sets), each in its own workspace from the library's pool.
plsh_status build_record_pair(const dev::AttnArgs &a, hipStream_t st, const char *who, void **ws_causal,
                              void **ws_nc) {
  const size_t ws_bytes = records_bytes(a.n, a.heads, a.s);
  *ws_causal = *ws_nc = nullptr;
  for (void **p : {ws_causal, ws_nc}) {
    const hipError_t e = pool_alloc(p, ws_bytes, st);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      *p = nullptr;
      return fail(PLSH_ERR_HIP, "%s: workspace allocation of %zu bytes failed: %s", who, ws_bytes,
                  hipGetErrorString(e));
    }
  }
  return launch_edges(a, false, st, who, *ws_nc, *ws_causal);
}

plsh_status free_records(void *ws, hipStream_t st, const char *who, plsh_status rc) {
  if (!ws) return rc;
  const hipError_t e = hipFreeAsync(ws, st);
  if (e != hipSuccess && rc == PLSH_OK) {
    (void)hipGetLastError();
    return fail(PLSH_ERR_HIP, "%s: workspace release failed: %s", who, hipGetErrorString(e));
  }
  return rc;
}


// The estimator: its records, then attn_mfma_kernel.  The records go to the
// caller's workspace when one is given, else to one from the stream-ordered
// allocator.
plsh_status launch_mfma(const dev::AttnArgs &a, const double *sigma, int d, int causal, hipStream_t st,
                        const char *who, void *caller_ws = nullptr, bool records_ready = false) {
  auto forward = [&](const void *ws) {
    FwdCall c;
    c.q = a.q;
    c.k = a.k;
    c.v = a.v;
    c.out = a.out;
    c.save_lse2 = a.save_lse2;
    c.ws = ws;
    c.sigma = sigma;
    c.batch = a.batch;
    c.n = a.n;
    c.heads = a.heads;
    c.kv_heads = a.kv_heads;
    c.d = d;
    c.s = a.s;
    c.causal = causal != 0;
    return launch_fwd(c, st, timer_slot(), who);
  };
  // (the fp32 partials of the unfused form come from attn_mfma_kernel, the
  // only kernel with that epilogue and a head stride into the table)
  auto attend = [&](const void *ws) {
    return a.o32 ? launch_attn(a, d, causal, st, who, 0, ws) : forward(ws);
  };
  if (caller_ws) {
    plsh_status rc = records_ready ? PLSH_OK : launch_edges(a, causal != 0, st, who, caller_ws);
    return rc == PLSH_OK ? attend(caller_ws) : rc;
  }
  void *ws = nullptr;
  plsh_status rc = build_records(a, causal != 0, st, who, &ws);
  if (rc == PLSH_OK) rc = attend(ws);
  return free_records(ws, st, who, rc);
}


// Exact ALiBi: the same checks as the estimator minus the table, bf16 only.
plsh_status check_exact(const void *q, const void *k, const void *v, void *out, int32_t batch, int32_t n,
                        int32_t heads, int32_t kv_heads, int32_t d, plsh_dtype dtype, const double *sigma,
                        const char *who) {
  if (!q || !k || !v || !out || !sigma) return fail(PLSH_ERR_ARG, "%s: null pointer argument", who);
  if (n < 1 || batch < 1 || heads < 1 || kv_heads < 1)
    return fail(PLSH_ERR_ARG, "%s: need n, batch, heads, kv_heads >= 1", who);
  if (heads % kv_heads != 0)
    return fail(PLSH_ERR_ARG, "%s: heads (%d) must be a multiple of kv_heads (%d)", who, heads, kv_heads);
  for (int32_t h = 0; h < heads; ++h)
    if (!finite_pos(sigma[h])) return fail(PLSH_ERR_ARG, "%s: sigma[%d] must be finite and > 0", who, h);
  if (dtype != PLSH_BF16) return fail(PLSH_ERR_UNSUPPORTED, "%s: only bf16 is supported", who);
  if (d != 64 && d != 128) return fail(PLSH_ERR_UNSUPPORTED, "%s: head dim %d not supported (64, 128)", who, d);
  if (heads > dev::kMaxHeadsArg)
    return fail(PLSH_ERR_UNSUPPORTED, "%s: heads = %d exceeds %d", who, heads, dev::kMaxHeadsArg);
  if ((int64_t)batch * heads * n * d >= ((int64_t)1 << 31) ||
      (int64_t)batch * kv_heads * n * d >= ((int64_t)1 << 31))
    return fail(PLSH_ERR_UNSUPPORTED, "%s: tensor has >= 2^31 elements", who);
  // (the bf16 kernels address a head's K or V rows, up to the last 32-row
  // tile's end, through 32-bit buffer offsets)
  if (dtype == PLSH_BF16 && ((int64_t)n + 31) * d * 2 >= ((int64_t)1 << 32))
    return fail(PLSH_ERR_UNSUPPORTED, "%s: n = %d too long for d = %d in bf16", who, n, d);
  if ((int64_t)((n + 127) / 128) * batch * heads >= ((int64_t)1 << 31))
    return fail(PLSH_ERR_UNSUPPORTED, "%s: too many row tiles", who);
  const size_t qbytes = (size_t)batch * heads * n * d * 2;
  const size_t kbytes = (size_t)batch * kv_heads * n * d * 2;
  if (overlaps(out, qbytes, q, qbytes) || overlaps(out, qbytes, k, kbytes) || overlaps(out, qbytes, v, kbytes))
    return fail(PLSH_ERR_ARG, "%s: out overlaps q, k or v", who);
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15u)
    return fail(PLSH_ERR_ARG, "%s: buffers must be 16-byte aligned", who);
  return PLSH_OK;
}

}  // namespace
}  // namespace plsh


using namespace plsh;

extern "C" plsh_status plsh_alibi_attention(const void *q, const void *k, const void *v, void *out,
                                            int32_t batch, int32_t n, int32_t heads, int32_t kv_heads,
                                            int32_t d, plsh_dtype dtype, const double *sigma, int32_t s,
                                            const plsh_tables *boundaries, int32_t causal,
                                            plsh_stream_t stream) {
  static const char *who = "plsh_alibi_attention";
  clear_error();
  plsh_status st = check_common(q, k, v, out, batch, n, heads, kv_heads, d, dtype, sigma, s, boundaries, who);
  if (st != PLSH_OK) return st;
  if ((st = have_device(who)) != PLSH_OK) return st;
  dev::AttnArgs a;
  fill_args(a, q, k, v, out, batch, n, heads, kv_heads, sigma, s, boundaries);
  if (dtype == PLSH_BF16 && s <= dev::kMaxFwdSamples) return launch_mfma(a, sigma, d, causal != 0, (hipStream_t)stream, who);
  return launch_valu(a, d, dtype, causal != 0, (hipStream_t)stream, who);
}

// Bytes of workspace plsh_alibi_attention_ws takes for a call (0 on the
// paths that need none).
extern "C" plsh_status plsh_attention_workspace_size(int32_t n, int32_t heads, int32_t s, plsh_dtype dtype,
                                                     int64_t *bytes) {
  clear_error();
  if (!bytes) return fail(PLSH_ERR_ARG, "plsh_attention_workspace_size: null pointer argument");
  if (n < 1 || heads < 1 || s < 1) return fail(PLSH_ERR_ARG, "plsh_attention_workspace_size: need n, heads, s >= 1");
  if (dtype != PLSH_BF16 && dtype != PLSH_F32) return fail(PLSH_ERR_UNSUPPORTED, "plsh_attention_workspace_size: unknown dtype");
  *bytes = (dtype == PLSH_BF16 && s <= dev::kMaxFwdSamples) ? (int64_t)records_bytes(n, heads, s) : 0;
  return PLSH_OK;
}

// plsh_alibi_attention with the pre-pass records in a caller-owned workspace.
extern "C" plsh_status plsh_alibi_attention_ws(const void *q, const void *k, const void *v, void *out,
                                               int32_t batch, int32_t n, int32_t heads, int32_t kv_heads,
                                               int32_t d, plsh_dtype dtype, const double *sigma, int32_t s,
                                               const plsh_tables *boundaries, int32_t causal, void *workspace,
                                               int64_t workspace_bytes, plsh_stream_t stream) {
  static const char *who = "plsh_alibi_attention_ws";
  clear_error();
  plsh_status st = check_common(q, k, v, out, batch, n, heads, kv_heads, d, dtype, sigma, s, boundaries, who);
  if (st != PLSH_OK) return st;
  const bool mfma = dtype == PLSH_BF16 && s <= dev::kMaxFwdSamples;
  const size_t need = mfma ? records_bytes(n, heads, s) : 0;
  if (workspace_bytes < 0 || (size_t)workspace_bytes < need)
    return fail(PLSH_ERR_CAPACITY, "%s: workspace of %lld bytes, the call needs %zu", who,
                (long long)workspace_bytes, need);
  if (need && !workspace) return fail(PLSH_ERR_ARG, "%s: null workspace", who);
  if ((uintptr_t)workspace & 15u) return fail(PLSH_ERR_ARG, "%s: workspace must be 16-byte aligned", who);
  if (need) {
    const size_t esz = dtype == PLSH_F32 ? 4 : 2;
    const size_t qbytes = (size_t)batch * heads * n * d * esz, kbytes = (size_t)batch * kv_heads * n * d * esz;
    if (overlaps(workspace, need, q, qbytes) || overlaps(workspace, need, k, kbytes) ||
        overlaps(workspace, need, v, kbytes) || overlaps(workspace, need, out, qbytes))
      return fail(PLSH_ERR_ARG, "%s: workspace overlaps q, k, v or out", who);
  }
  if ((st = have_device(who)) != PLSH_OK) return st;
  dev::AttnArgs a;
  fill_args(a, q, k, v, out, batch, n, heads, kv_heads, sigma, s, boundaries);
  if (mfma) return launch_mfma(a, sigma, d, causal != 0, (hipStream_t)stream, who, workspace);
  return launch_valu(a, d, dtype, causal != 0, (hipStream_t)stream, who);
}

// The pre-pass alone, into a caller's workspace (see include/plsh.h).
extern "C" plsh_status plsh_alibi_records(const plsh_tables *boundaries, int32_t causal, void *workspace,
                                          int64_t workspace_bytes, plsh_stream_t stream) {
  static const char *who = "plsh_alibi_records";
  clear_error();
  if (!boundaries || !boundaries->params || !workspace) return fail(PLSH_ERR_ARG, "%s: null pointer argument", who);
  const int32_t n = boundaries->n, heads = boundaries->heads, s = boundaries->s;
  if (n < 1 || heads < 1 || s < 1) return fail(PLSH_ERR_TABLE, "%s: need n, heads, s >= 1", who);
  if (s > dev::kMaxFwdSamples) return fail(PLSH_ERR_UNSUPPORTED, "%s: s = %d exceeds %d", who, s, dev::kMaxFwdSamples);
  if (heads > dev::kMaxHeadsArg)
    return fail(PLSH_ERR_UNSUPPORTED, "%s: heads = %d exceeds %d", who, heads, dev::kMaxHeadsArg);
  if ((uintptr_t)workspace & 15u) return fail(PLSH_ERR_ARG, "%s: workspace must be 16-byte aligned", who);
  const size_t need = records_bytes(n, heads, s);
  if (workspace_bytes < 0 || (size_t)workspace_bytes < need)
    return fail(PLSH_ERR_CAPACITY, "%s: workspace of %lld bytes, the records need %zu", who,
                (long long)workspace_bytes, need);
  plsh_status st = have_device(who);
  if (st != PLSH_OK) return st;
  dev::AttnArgs a{};
  a.params = boundaries->params;
  a.n = n;
  a.heads = heads;
  a.s = s;
  a.pstride = s;
  return launch_edges(a, causal != 0, (hipStream_t)stream, who, workspace);
}

// The attention kernel alone over records already in the workspace (see
// include/plsh.h).
extern "C" plsh_status plsh_alibi_attention_from_records(const void *q, const void *k, const void *v, void *out,
                                                         int32_t batch, int32_t n, int32_t heads, int32_t kv_heads,
                                                         int32_t d, plsh_dtype dtype, const double *sigma, int32_t s,
                                                         const plsh_tables *boundaries, int32_t causal,
                                                         const void *workspace, int64_t workspace_bytes,
                                                         plsh_stream_t stream) {
  static const char *who = "plsh_alibi_attention_from_records";
  clear_error();
  plsh_status st = check_common(q, k, v, out, batch, n, heads, kv_heads, d, dtype, sigma, s, boundaries, who);
  if (st != PLSH_OK) return st;
  if (dtype != PLSH_BF16 || s > dev::kMaxFwdSamples)
    return fail(PLSH_ERR_UNSUPPORTED, "%s: bf16 with s <= %d only", who, dev::kMaxFwdSamples);
  const size_t need = records_bytes(n, heads, s);
  if (!workspace) return fail(PLSH_ERR_ARG, "%s: null workspace", who);
  if ((uintptr_t)workspace & 15u) return fail(PLSH_ERR_ARG, "%s: workspace must be 16-byte aligned", who);
  if (workspace_bytes < 0 || (size_t)workspace_bytes < need)
    return fail(PLSH_ERR_CAPACITY, "%s: workspace of %lld bytes, the records need %zu", who,
                (long long)workspace_bytes, need);
  // (the kernel only reads the records, so only out must not overlap them)
  if (overlaps(workspace, need, out, (size_t)batch * heads * n * d * 2))
    return fail(PLSH_ERR_ARG, "%s: workspace overlaps out", who);
  if ((st = have_device(who)) != PLSH_OK) return st;
  dev::AttnArgs a;
  fill_args(a, q, k, v, out, batch, n, heads, kv_heads, sigma, s, boundaries);
  return launch_mfma(a, sigma, d, causal != 0, (hipStream_t)stream, who, const_cast<void *>(workspace), true);
}

// plsh_alibi_attention with its records in the library's static scratch: no
// device memory is allocated by the call (see include/plsh.h).
extern "C" plsh_status plsh_alibi_attention_noalloc(const void *q, const void *k, const void *v, void *out,
                                                    int32_t batch, int32_t n, int32_t heads, int32_t kv_heads,
                                                    int32_t d, plsh_dtype dtype, const double *sigma, int32_t s,
                                                    const plsh_tables *boundaries, int32_t causal,
                                                    plsh_stream_t stream) {
  static const char *who = "plsh_alibi_attention_noalloc";
  clear_error();
  plsh_status st = check_common(q, k, v, out, batch, n, heads, kv_heads, d, dtype, sigma, s, boundaries, who);
  if (st != PLSH_OK) return st;
  const bool mfma = dtype == PLSH_BF16 && s <= dev::kMaxFwdSamples;
  const size_t need = mfma ? records_bytes(n, heads, s) : 0;
  if (need > kScratchBytes)
    return fail(PLSH_ERR_CAPACITY, "%s: the call's records need %zu bytes, the static scratch holds %zu", who, need,
                kScratchBytes);
  if ((st = have_device(who)) != PLSH_OK) return st;
  dev::AttnArgs a;
  fill_args(a, q, k, v, out, batch, n, heads, kv_heads, sigma, s, boundaries);
  if (!mfma) return launch_valu(a, d, dtype, causal != 0, (hipStream_t)stream, who);
  void *ws = nullptr;
  if ((st = scratch_ptr(who, &ws)) != PLSH_OK) return st;
  return launch_mfma(a, sigma, d, causal != 0, (hipStream_t)stream, who, ws);
}

// Test aid: the same estimator through the one-row-per-wave VALU kernel.
extern "C" plsh_status plsh_debug_attention_reference(const void *q, const void *k, const void *v,
                                                      void *out, int32_t batch, int32_t n, int32_t heads,
                                                      int32_t kv_heads, int32_t d, plsh_dtype dtype,
                                                      const double *sigma, int32_t s,
                                                      const plsh_tables *boundaries, int32_t causal,
                                                      plsh_stream_t stream) {
  static const char *who = "plsh_debug_attention_reference";
  clear_error();
  plsh_status st = check_common(q, k, v, out, batch, n, heads, kv_heads, d, dtype, sigma, s, boundaries, who);
  if (st != PLSH_OK) return st;
  if ((st = have_device(who)) != PLSH_OK) return st;
  dev::AttnArgs a;
  fill_args(a, q, k, v, out, batch, n, heads, kv_heads, sigma, s, boundaries);
  return launch_valu(a, d, dtype, causal != 0, (hipStream_t)stream, who);
}

extern "C" plsh_status plsh_debug_block_intervals(const plsh_tables *bt, int32_t *lohi, plsh_stream_t stream) {
  static const char *who = "plsh_debug_block_intervals";
  clear_error();
  if (!bt || !bt->params || !lohi) return fail(PLSH_ERR_ARG, "%s: null pointer argument", who);
  if (bt->n < 1 || bt->heads < 1 || bt->s < 1) return fail(PLSH_ERR_TABLE, "%s: need n, heads, s >= 1", who);
  if (bt->s > kMaxSamples) return fail(PLSH_ERR_UNSUPPORTED, "%s: s exceeds %d", who, kMaxSamples);
  plsh_status st = have_device(who);
  if (st != PLSH_OK) return st;
  return launch_debug_intervals(bt, lohi, (hipStream_t)stream, who);
}

extern "C" plsh_status plsh_exact_alibi_attention(const void *q, const void *k, const void *v, void *out,
                                                  int32_t batch, int32_t n, int32_t heads, int32_t kv_heads,
                                                  int32_t d, plsh_dtype dtype, const double *sigma,
                                                  int32_t causal, plsh_stream_t stream) {
  static const char *who = "plsh_exact_alibi_attention";
  clear_error();
  plsh_status st = check_exact(q, k, v, out, batch, n, heads, kv_heads, d, dtype, sigma, who);
  if (st != PLSH_OK) return st;
  if ((st = have_device(who)) != PLSH_OK) return st;
  dev::ExactArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.batch = batch;
  a.n = n;
  a.heads = heads;
  a.kv_heads = kv_heads;
  a.groups = (n + 127) / 128;
  for (int i = 0; i < dev::kMaxHeadsArg; ++i) a.slope2[i] = i < heads ? (float)(1.4426950408889634 / sigma[i]) : 0.f;
  return launch_exact(a, d, causal != 0, (hipStream_t)stream, who);
}

// The unfused form of the estimator (an ablation of the sample fusion): s
// single-sample passes of the same kernels writing fp32 partials, then the
// log-sum-exp combine.
extern "C" plsh_status plsh_alibi_attention_unfused(const void *q, const void *k, const void *v, void *out,
                                                    int32_t batch, int32_t n, int32_t heads, int32_t kv_heads,
                                                    int32_t d, plsh_dtype dtype, const double *sigma, int32_t s,
                                                    const plsh_tables *boundaries, int32_t causal,
                                                    plsh_stream_t stream) {
  static const char *who = "plsh_alibi_attention_unfused";
  clear_error();
  plsh_status st = check_common(q, k, v, out, batch, n, heads, kv_heads, d, dtype, sigma, s, boundaries, who);
  if (st != PLSH_OK) return st;
  if (dtype != PLSH_BF16) return fail(PLSH_ERR_UNSUPPORTED, "%s: only bf16 is supported", who);
  if ((st = have_device(who)) != PLSH_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  const int64_t rows = (int64_t)batch * heads * n;
  const size_t bytes = (size_t)s * rows * ((size_t)d + 1) * sizeof(float);
  void *ws = nullptr;
  hipError_t e = pool_alloc(&ws, bytes, hs);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PLSH_ERR_HIP, "%s: partials allocation of %zu bytes failed: %s", who, bytes, hipGetErrorString(e));
  }
  float *o32 = (float *)ws;
  float *lse = o32 + (size_t)s * rows * d;
  plsh_status rc = PLSH_OK;
  for (int32_t kk = 0; kk < s && rc == PLSH_OK; ++kk) {
    dev::AttnArgs a;
    fill_args(a, q, k, v, out, batch, n, heads, kv_heads, sigma, s, boundaries);
    a.params = boundaries->params + 2 * kk;  // sample kk of every head: rows h * s + kk
    a.pstride = s;
    a.s = 1;
    a.o32 = o32 + (size_t)kk * rows * d;
    a.lse = lse + (size_t)kk * rows;
    rc = launch_mfma(a, sigma, d, causal != 0, hs, who);
  }
  if (rc == PLSH_OK) rc = launch_combine(o32, lse, s, rows, d, out, hs, who);
  e = hipFreeAsync(ws, hs);
  if (e != hipSuccess && rc == PLSH_OK) {
    (void)hipGetLastError();
    return fail(PLSH_ERR_HIP, "%s: partials release failed: %s", who, hipGetErrorString(e));
  }
  return rc;
}

// The estimate with the samples walked one by one (see include/plsh.h).
extern "C" plsh_status plsh_alibi_attention_walk(const void *q, const void *k, const void *v, void *out,
                                                 int32_t batch, int32_t n, int32_t heads, int32_t kv_heads,
                                                 int32_t d, plsh_dtype dtype, const double *sigma, int32_t s,
                                                 const plsh_tables *boundaries, int32_t causal,
                                                 plsh_stream_t stream) {
  static const char *who = "plsh_alibi_attention_walk";
  clear_error();
  plsh_status st = check_common(q, k, v, out, batch, n, heads, kv_heads, d, dtype, sigma, s, boundaries, who);
  if (st != PLSH_OK) return st;
  if (dtype != PLSH_BF16) return fail(PLSH_ERR_UNSUPPORTED, "%s: only bf16 is supported", who);
  if ((int64_t)heads * s > INT32_MAX / ((n + 31) / 32))
    return fail(PLSH_ERR_UNSUPPORTED, "%s: heads * s * ceil(n / 32) records exceed 2^31", who);
  if ((st = have_device(who)) != PLSH_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  dev::AttnArgs a;
  fill_args(a, q, k, v, out, batch, n, heads, kv_heads, sigma, s, boundaries);
  // single-sample records: (head h, sample k) as pseudo-head h s + k, whose
  // parameters are row h s + k of the table
  dev::AttnArgs ar = a;
  ar.heads = heads * s;
  ar.s = 1;
  ar.pstride = 1;
  void *rec = nullptr;
  plsh_status rc = build_records(ar, causal != 0, hs, who, &rec);
  if (rc == PLSH_OK) rc = launch_attn(a, d, causal != 0, hs, who, 3, rec);
  return free_records(rec, hs, who, rc);
}

// The backward of the estimate for fixed tables (see include/plsh.h).  With
// saved_out and saved_lse2 (the output and row normalisers of
// plsh_alibi_attention_lse) no forward runs; without them the call first
// runs that forward into a buffer of its own.
static plsh_status backward_common(const char *who, const void *q, const void *k, const void *v,
                                   const void *dout, void *dq, void *dk, void *dv, int32_t batch, int32_t n,
                                   int32_t heads, int32_t kv_heads, int32_t d, plsh_dtype dtype,
                                   const double *sigma, int32_t s, const plsh_tables *boundaries,
                                   int32_t causal, plsh_stream_t stream, bool saved, const void *saved_out,
                                   const float *saved_lse2) {
  clear_error();
  plsh_status st = check_common(q, k, v, dq, batch, n, heads, kv_heads, d, dtype, sigma, s, boundaries, who);
  if (st != PLSH_OK) return st;
  if (!dout || !dk || !dv || (saved && (!saved_out || !saved_lse2)))
    return fail(PLSH_ERR_ARG, "%s: null pointer argument", who);
  if (((uintptr_t)dout | (uintptr_t)dk | (uintptr_t)dv | (uintptr_t)saved_out | (uintptr_t)saved_lse2) & 15u)
    return fail(PLSH_ERR_ARG, "%s: buffers must be 16-byte aligned", who);
  const int ns = (n + 31) & ~31;
  {
    const size_t qb = (size_t)batch * heads * n * d * 2, kb = (size_t)batch * kv_heads * n * d * 2;
    const size_t lb = (size_t)batch * heads * ns * sizeof(float);
    const void *ins[6] = {q, k, v, dout, saved_out, saved_lse2};
    const size_t insz[6] = {qb, kb, kb, qb, saved ? qb : 0, saved ? lb : 0};
    void *outs[3] = {dq, dk, dv};
    const size_t outsz[3] = {qb, kb, kb};
    for (int o = 0; o < 3; ++o) {
      for (int i = 0; i < 6; ++i)
        if (insz[i] && overlaps(outs[o], outsz[o], ins[i], insz[i]))
          return fail(PLSH_ERR_ARG, "%s: dq, dk or dv overlaps an input", who);
      for (int o2 = o + 1; o2 < 3; ++o2)
        if (overlaps(outs[o], outsz[o], outs[o2], outsz[o2]))
          return fail(PLSH_ERR_ARG, "%s: dq, dk and dv overlap", who);
    }
  }
  if (dtype != PLSH_BF16 || s > dev::kMaxMfmaSamples)
    return fail(PLSH_ERR_UNSUPPORTED, "%s: bf16 with s <= %d only", who, dev::kMaxMfmaSamples);
  if ((st = have_device(who)) != PLSH_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  const int64_t prows = (int64_t)batch * heads * ns;
  // the recomputing backward first runs the forward that writes each row's
  // normaliser, into an output of its own, and then proceeds as from that
  // saved forward: [O (bf16, as q)][lse2][D]; from a saved forward only [D]
  const size_t obytes = saved ? 0 : ((size_t)batch * heads * n * d * 2 + 255) & ~(size_t)255;
  const size_t bytes = obytes + (saved ? 1 : 2) * (size_t)prows * sizeof(float);
  void *stats = nullptr;
  hipError_t e = pool_alloc(&stats, bytes, hs);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PLSH_ERR_HIP, "%s: statistics allocation of %zu bytes failed: %s", who, bytes, hipGetErrorString(e));
  }
  float *tail = (float *)((char *)stats + obytes);
  const void *out_used = saved ? saved_out : stats;
  const float *lse2 = saved ? saved_lse2 : tail;
  float *dvec = saved ? tail : tail + prows;
  dev::AttnArgs a;
  fill_args(a, q, k, v, dq, batch, n, heads, kv_heads, sigma, s, boundaries);
  a.dout = dout;
  plsh_status rc = PLSH_OK;
  // the records of the estimator serve its forward and dQ; dK/dV takes
  // non-causal ones (the same records when the call is not causal; a causal
  // call gets both sets from one pre-pass)
  void *rec = nullptr, *rec_nc = nullptr;
  if (rc == PLSH_OK) {
    if (causal) rc = build_record_pair(a, hs, who, &rec, &rec_nc);
    else rc = build_records(a, false, hs, who, &rec);
  }
  if (rc == PLSH_OK && !saved) {
    // the forward with each row's normaliser (the forward kernel over the
    // records just built)
    dev::AttnArgs f = a;
    f.out = stats;
    f.save_lse2 = tail;
    rc = launch_mfma(f, sigma, d, causal != 0, hs, who, rec, true);
  }
  if (rc == PLSH_OK) {
    // dQ; it also forms D = dO . O from the forward's output into dvec
    a.stat_dvec = dvec;
    a.saved_out = out_used;
    a.lse2 = lse2;
    rc = launch_attn(a, d, causal != 0, hs, who, 1, rec);
    a.stat_dvec = nullptr;
    a.saved_out = nullptr;
    a.dvec = dvec;
  }
  if (rc == PLSH_OK) {
    // dK/dV workgroups run per KV head: the group with the largest summed
    // sigma first
    const int grp = heads / kv_heads;
    std::vector<double> w(kv_heads, 0.0);
    for (int h = 0; h < heads; ++h) w[h / grp] += sigma[h];
    int idx[dev::kMaxHeadsArg];
    std::iota(idx, idx + kv_heads, 0);
    std::stable_sort(idx, idx + kv_heads, [&](int x, int y) { return w[x] > w[y]; });
    for (int i = 0; i < dev::kMaxHeadsArg; ++i) a.order[i] = i < kv_heads ? idx[i] : 0;
    rc = launch_attn(a, d, causal != 0, hs, who, 2, causal ? rec_nc : rec, dk, dv);
  }
  rc = free_records(rec_nc, hs, who, rc);
  rc = free_records(rec, hs, who, rc);
  e = hipFreeAsync(stats, hs);
  if (e != hipSuccess && rc == PLSH_OK) {
    (void)hipGetLastError();
    return fail(PLSH_ERR_HIP, "%s: statistics release failed: %s", who, hipGetErrorString(e));
  }
  return rc;
}

extern "C" plsh_status plsh_alibi_attention_backward(const void *q, const void *k, const void *v,
                                                     const void *dout, void *dq, void *dk, void *dv,
                                                     int32_t batch, int32_t n, int32_t heads, int32_t kv_heads,
                                                     int32_t d, plsh_dtype dtype, const double *sigma, int32_t s,
                                                     const plsh_tables *boundaries, int32_t causal,
                                                     plsh_stream_t stream) {
  return backward_common("plsh_alibi_attention_backward", q, k, v, dout, dq, dk, dv, batch, n, heads, kv_heads,
                         d, dtype, sigma, s, boundaries, causal, stream, false, nullptr, nullptr);
}

extern "C" plsh_status plsh_alibi_attention_backward_saved(const void *q, const void *k, const void *v,
                                                           const void *out, const float *lse2,
                                                           const void *dout, void *dq, void *dk, void *dv,
                                                           int32_t batch, int32_t n, int32_t heads,
                                                           int32_t kv_heads, int32_t d, plsh_dtype dtype,
                                                           const double *sigma, int32_t s,
                                                           const plsh_tables *boundaries, int32_t causal,
                                                           plsh_stream_t stream) {
  return backward_common("plsh_alibi_attention_backward_saved", q, k, v, dout, dq, dk, dv, batch, n, heads,
                         kv_heads, d, dtype, sigma, s, boundaries, causal, stream, true, out, lse2);
}

// The estimator, writing each row's log2 normaliser beside the output.
extern "C" plsh_status plsh_alibi_attention_lse(const void *q, const void *k, const void *v, void *out,
                                                int32_t batch, int32_t n, int32_t heads, int32_t kv_heads,
                                                int32_t d, plsh_dtype dtype, const double *sigma, int32_t s,
                                                const plsh_tables *boundaries, int32_t causal, float *lse2,
                                                void *workspace, int64_t workspace_bytes,
                                                plsh_stream_t stream) {
  static const char *who = "plsh_alibi_attention_lse";
  clear_error();
  plsh_status st = check_common(q, k, v, out, batch, n, heads, kv_heads, d, dtype, sigma, s, boundaries, who);
  if (st != PLSH_OK) return st;
  if (!lse2) return fail(PLSH_ERR_ARG, "%s: null pointer argument", who);
  if ((uintptr_t)lse2 & 15u) return fail(PLSH_ERR_ARG, "%s: lse2 must be 16-byte aligned", who);
  const size_t ns = (size_t)((n + 31) & ~31);
  const size_t lb = (size_t)batch * heads * ns * sizeof(float), esz = dtype == PLSH_F32 ? 4 : 2;
  const size_t qb = (size_t)batch * heads * n * d * esz, kb = (size_t)batch * kv_heads * n * d * esz;
  if (overlaps(lse2, lb, q, qb) || overlaps(lse2, lb, k, kb) || overlaps(lse2, lb, v, kb) ||
      overlaps(lse2, lb, out, qb))
    return fail(PLSH_ERR_ARG, "%s: lse2 overlaps q, k, v or out", who);
  if (dtype != PLSH_BF16 || s > dev::kMaxFwdSamples)
    return fail(PLSH_ERR_UNSUPPORTED, "%s: bf16 with s <= %d only", who, dev::kMaxFwdSamples);
  if (workspace) {
    const size_t need = records_bytes(n, heads, s);
    if (workspace_bytes < 0 || (size_t)workspace_bytes < need)
      return fail(PLSH_ERR_CAPACITY, "%s: workspace of %lld bytes, the call needs %zu", who,
                  (long long)workspace_bytes, need);
    if ((uintptr_t)workspace & 15u) return fail(PLSH_ERR_ARG, "%s: workspace must be 16-byte aligned", who);
    if (overlaps(workspace, need, q, qb) || overlaps(workspace, need, k, kb) || overlaps(workspace, need, v, kb) ||
        overlaps(workspace, need, out, qb) || overlaps(workspace, need, lse2, lb))
      return fail(PLSH_ERR_ARG, "%s: workspace overlaps q, k, v, out or lse2", who);
  }
  if ((st = have_device(who)) != PLSH_OK) return st;
  dev::AttnArgs a;
  fill_args(a, q, k, v, out, batch, n, heads, kv_heads, sigma, s, boundaries);
  a.save_lse2 = lse2;
  return launch_mfma(a, sigma, d, causal != 0, (hipStream_t)stream, who, workspace);
}

extern "C" plsh_status plsh_kernel_timer(int32_t enable) {
  clear_error();
  g_timer.on = enable != 0;
  g_timer.used = 0;
  return PLSH_OK;
}

extern "C" plsh_status plsh_kernel_timer_read(int32_t *launches, double *total_ms) {
  static const char *who = "plsh_kernel_timer_read";
  clear_error();
  if (!launches || !total_ms) return fail(PLSH_ERR_ARG, "%s: null pointer argument", who);
  double sum = 0.0;
  for (size_t i = 0; i < g_timer.used; ++i) {
    float ms = 0.f;
    const auto &pr = g_timer.ev[i];
    hipError_t e = hipEventSynchronize(pr.second);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, pr.first, pr.second);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      g_timer.used = 0;
      return fail(PLSH_ERR_HIP, "%s: %s", who, hipGetErrorString(e));
    }
    sum += ms;
  }
  *launches = (int32_t)g_timer.used;
  *total_ms = sum;
  g_timer.used = 0;
  return PLSH_OK;
}
