// plsh_attention.hip -- GPU half of libplsh: Positional-LSH ALiBi attention
// for gfx950 (MI355X).
//
// "Positional LSH: Binary Block Matrix Approximation for Attention with Linear
// Biases" (technical-summary pages):
//   Methodology §1 -- a random-binning hash splits positions into contiguous
//     blocks; M(h)_ij = 1 when i and j share a block; L* = E_h[M(h)].
//   Methodology §2 (Theorem 2.1) -- M~ = (1/s) sum_k M(h_k); blocks stay short.
//   Methodology §3 (Theorem 2.2) -- ALiBi attention becomes s randomized
//     short-context attentions without positional bias.
//
// Every kernel evaluates the ratio-of-sums estimator
//   T~_i = sum_j c_ij e^{q_i.k_j} v_j / sum_j c_ij e^{q_i.k_j},
//   c_ij = #{k : j in B_k(i)}  (times the causal mask),
// which is the s block-local attentions summed sample by sample with the
// per-pair sums regrouped: each (i, j) pair in the union of i's blocks is
// evaluated once and weighted by how many samples contain it.  The union of
// the s blocks that hold i is one interval (they all contain i), so each row
// walks a single contiguous key range.
//
// Block intervals are recomputed on the device from (delta, u) with the same
// binary64 predicate as the host table (plsh_binning.h), per wave of 32 query
// rows:
//   lead_k  = first position of the block of sample k holding row r0,
//   trail_k = one past the block of sample k holding the wave's last row,
//   mask_k  = bit t (1..31) set when r0 + t starts a block of sample k.
// Row i = r0 + t then has lo_k(i) = r0 + (highest set bit <= t) or lead_k, and
// hi_k(i) = r0 + (lowest set bit > t) or trail_k.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <numeric>

#include "plsh_binning.h"
#include "plsh_internal.h"

namespace plsh {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxHeadsArg = 128;
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
  const void *q;
  const void *k;
  const void *v;
  void *out;
  const double *params;
  int32_t batch, n, heads, kv_heads, s;
  int32_t groups;  // query-row tiles per (batch, head)
  int32_t order[kMaxHeadsArg];  // head processed in slot i, heaviest sigma first
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// Orders the wave's LDS traffic: lanes see each other's LDS writes after this.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = min(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o));
  return x;
}

// Value of x in the other half of the wave (lane l <-> l ^ 32), via the two
// results of v_permlane32_swap: lanes < 32 get the upper half in [1], lanes
// >= 32 get the lower half in [0].
__device__ __forceinline__ uint32_t other_half(uint32_t x, int lane) {
  auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return lane < 32 ? p[1] : p[0];
}
__device__ __forceinline__ float other_half_f(float x, int lane) {
  return __uint_as_float(other_half(__float_as_uint(x), lane));
}

// bits 1..t of a 32-bit mask (t in [0, 31])
__device__ __forceinline__ uint32_t bits_1_to(int t) {
  return t == 0 ? 0u : ((0xFFFFFFFFu >> (31 - t)) & ~1u);
}

// Per-wave block setup for rows [r0, r0 + 32) of one head (see file header).
// Lanes take samples k = lane, lane + 64, ...
__device__ void wave_setup(const double *prm, int s, int n, int r0, int lane, int32_t *lead,
                           int32_t *trail, uint32_t *mask) {
  const int last = min(r0 + 31, n - 1);
  for (int k = lane; k < s; k += 64) {
    const double dl = prm[2 * k], u = prm[2 * k + 1];
    const double b = bin_of(r0, dl, u);
    const int32_t lo = block_lo(r0, dl, u, b);
    int32_t y = block_hi(r0, n, dl, u, b);
    uint32_t m = 0;
    while (y <= last) {  // y starts a block inside (r0, last]
      m |= 1u << (y - r0);
      y = block_hi(y, n, dl, u, bin_of(y, dl, u));
    }
    lead[k] = lo;
    trail[k] = y;
    mask[k] = m;
  }
}

__device__ __forceinline__ int32_t row_lo(int32_t lead, uint32_t mask, int r0, int t) {
  const uint32_t mk = mask & bits_1_to(t);
  return mk ? r0 + (31 - __builtin_clz(mk)) : lead;
}
__device__ __forceinline__ int32_t row_hi(int32_t trail, uint32_t mask, int r0, int t) {
  const uint32_t mk = mask & ~((2u << t) - 1u);
  return mk ? r0 + __builtin_ctz(mk) : trail;
}

// ---------------------------------------------------------------------------
// Debug: every (h, k, i) interval through the per-wave setup above.
// One wave per (head, 32-row group).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void debug_intervals_kernel(const double *params, int n, int heads,
                                                             int s, int groups, int32_t *lohi) {
  extern __shared__ uint8_t smem[];
  int32_t *lead = (int32_t *)smem;
  int32_t *trail = lead + s;
  uint32_t *mask = (uint32_t *)(trail + s);
  const int lane = threadIdx.x;
  const int h = blockIdx.x / groups;
  const int r0 = (blockIdx.x % groups) * 32;
  if (h >= heads) return;
  wave_setup(params + 2 * (int64_t)h * s, s, n, r0, lane, lead, trail, mask);
  wave_sync();
  const int t = lane & 31;
  const int i = r0 + t;
  if (i >= n) return;
  for (int k = (lane >> 5); k < s; k += 2) {
    const int64_t o = (((int64_t)h * s + k) * n + i) * 2;
    lohi[o] = row_lo(lead[k], mask[k], r0, t);
    lohi[o + 1] = row_hi(trail[k], mask[k], r0, t);
  }
}

// ---------------------------------------------------------------------------
// Reference kernel (VALU, fp32 arithmetic): one wave per query row at a time.
// Used for fp32 inputs and as an independent GPU formulation for bf16.
// Grid: one 256-thread workgroup per (head slot, batch, 128-row tile).
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ float load_elem(const T *p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float *p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t *p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
}
template <typename T>
__device__ __forceinline__ void store_elem(T *p, int64_t i, float v);
template <>
__device__ __forceinline__ void store_elem<float>(float *p, int64_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void store_elem<uint16_t>(uint16_t *p, int64_t i, float v) {
  p[i] = (uint16_t)f32_to_bf16_bits(v);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_valu_kernel(AttnArgs a, int causal) {
  extern __shared__ uint8_t smem[];
  const int s = a.s, n = a.n;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // per-wave scratch: lead, trail, mask, rlo, rhi [s]; qrow [D]; p [64]
  const size_t per_wave = (size_t)5 * s * 4 + D * 4 + 64 * 4;
  uint8_t *base = smem + wave * per_wave;
  int32_t *lead = (int32_t *)base;
  int32_t *trail = lead + s;
  uint32_t *mask = (uint32_t *)(trail + s);
  int32_t *rlo = (int32_t *)(mask + s);
  int32_t *rhi = rlo + s;
  float *qrow = (float *)(rhi + s);
  float *pj = qrow + D;

  const int unit = blockIdx.x / a.groups;
  const int g = blockIdx.x % a.groups;
  const int h = a.order[unit / a.batch];
  const int b = unit % a.batch;
  const int kvh = h / (a.heads / a.kv_heads);
  const int r0 = g * 128 + wave * 32;
  if (r0 >= n) return;

  const T *Q = (const T *)a.q + ((int64_t)b * a.heads + h) * n * D;
  const T *K = (const T *)a.k + ((int64_t)b * a.kv_heads + kvh) * n * D;
  const T *V = (const T *)a.v + ((int64_t)b * a.kv_heads + kvh) * n * D;
  T *O = (T *)a.out + ((int64_t)b * a.heads + h) * n * D;

  wave_setup(a.params + 2 * (int64_t)h * s, s, n, r0, lane, lead, trail, mask);
  wave_sync();

  constexpr int E = D / 64;
  for (int t = 0; t < 32 && r0 + t < n; ++t) {
    const int i = r0 + t;
    int ulo = n, uhi = 0;
    for (int k = lane; k < s; k += 64) {
      const int32_t lo = row_lo(lead[k], mask[k], r0, t);
      const int32_t hi = row_hi(trail[k], mask[k], r0, t);
      rlo[k] = lo;
      rhi[k] = hi;
      ulo = min(ulo, lo);
      uhi = max(uhi, hi);
    }
    for (int c = lane; c < D; c += 64) qrow[c] = load_elem(Q, (int64_t)i * D + c);
    ulo = wave_min_i(ulo);
    uhi = wave_max_i(uhi);
    if (causal) uhi = min(uhi, i + 1);
    wave_sync();

    float m = -INFINITY, l = 0.f, acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    for (int j0 = ulo; j0 < uhi; j0 += 64) {
      const int j = j0 + lane;
      const bool valid = j < uhi;
      float logit = 0.f;
      int c = 0;
      if (valid) {
        const int64_t kr = (int64_t)j * D;
        for (int dd = 0; dd < D; ++dd) logit = fmaf(qrow[dd], load_elem(K, kr + dd), logit);
        for (int kk = 0; kk < s; ++kk) c += (rlo[kk] <= j) & (j < rhi[kk]);
      }
      const bool use = valid && c > 0;
      const float mc = wave_max(use ? logit : -INFINITY);
      const float mn = fmaxf(m, mc);
      if (mn == -INFINITY) continue;
      const float alpha = (m == -INFINITY) ? 0.f : expf(m - mn);
      const float p = use ? (float)c * expf(logit - mn) : 0.f;
      l = l * alpha + wave_sum(p);
      pj[lane] = p;
      wave_sync();
      const int cnt = min(64, uhi - j0);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float sacc = 0.f;
        for (int jj = 0; jj < cnt; ++jj)
          sacc = fmaf(pj[jj], load_elem(V, (int64_t)(j0 + jj) * D + lane + 64 * e), sacc);
        acc[e] = acc[e] * alpha + sacc;
      }
      wave_sync();
      m = mn;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) store_elem(O, (int64_t)i * D + lane + 64 * e, acc[e] / l);
    wave_sync();
  }
}

// ---------------------------------------------------------------------------
// Sample-fused MFMA kernel (bf16 in, fp32 accumulate).
//
// Workgroup = 4 waves = 128 query rows of one (batch, head); each wave owns
// 32 rows.  Keys stream through LDS in stages of 64 (K row-major, V
// transposed); each wave consumes the 32-key tiles of its own union range.
// Per tile and wave:
//   S^T (32 keys x 32 queries) = K Q^T on v_mfma_f32_32x32x16_bf16, with the
//     key rows of the A operand permuted so that lane l holds query row
//     r0 + l % 32 and the 16 consecutive keys j0 + 16 (l / 32) + r in its
//     16 accumulators;
//   multiplicity c_ij from a per-row byte histogram of block edges in LDS
//     (prefix-summed four bytes at a time), or the row's running count when
//     no edge falls in the tile;
//   weighted online softmax in the log2 domain with a lazily raised running
//     max (only when a logit exceeds it by more than 2^8);
//   O^T (D x 32 queries) += V^T P^T on the same MFMA, P taken straight from
//     the accumulators (no cross-lane shuffle).
// Output O = acc / l is written once, rounded to bf16.
// ---------------------------------------------------------------------------
constexpr int kStageKeys = 64;

template <int D>
struct MfmaLds {
  static constexpr int kKStride = D + 8;            // bf16 per K row
  static constexpr int kVStride = kStageKeys + 8;   // bf16 per V^T row
  static constexpr int kHistStride = 20;            // dwords per histogram row
  alignas(16) uint16_t K[kStageKeys * kKStride];
  alignas(16) uint16_t Vt[D * kVStride];
  alignas(16) uint32_t hist[4][32 * kHistStride];
  int32_t range[4][2];
};

// key held by row a of the S^T accumulator block (see kernel comment)
__device__ __forceinline__ int key_of_row(int a) {
  return 16 * ((a >> 2) & 1) + 4 * (a >> 3) + (a & 3);
}

// prefix-sum 16 bytes held in 4 dwords (bytes never exceed 255)
__device__ __forceinline__ uint32_t prefix16(u32x4 &x) {
  uint32_t carry = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t y = x[w];
    y += y << 8;
    y += y << 16;
    y += carry * 0x01010101u;
    x[w] = y;
    carry = y >> 24;
  }
  return carry;  // total
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_mfma_kernel(AttnArgs a) {
  using L = MfmaLds<D>;
  __shared__ __attribute__((aligned(16))) L lds;
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  const int s = a.s, n = a.n;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t = lane & 31, hh = lane >> 5;
  int32_t *lead = (int32_t *)dyn + wave * 6 * s;
  int32_t *trail = lead + s;
  uint32_t *mask = (uint32_t *)(trail + s);
  int32_t *lord = (int32_t *)(mask + s);   // samples sorted by lead
  int32_t *tord = lord + s;                // samples sorted by trail
  int32_t *nzl = tord + s;                 // samples with a block edge inside the wave

  // ---- workgroup -> (head, batch, row tile): heavy heads first; on each of
  // the 8 XCDs (workgroups are dealt round-robin) a contiguous run of row
  // tiles of every (head, batch) unit, so neighbouring tiles share K/V in L2.
  const int G = a.groups;
  const int p = blockIdx.x;
  const int unit = p / G;
  const int tu = p - unit * G;
  const int xcd = p & 7;
  const int base_mod = (int)(((int64_t)unit * G) & 7);
  int start = 0, t0c = 0;
  for (int c = 0; c < 8; ++c) {
    const int t0 = (c - base_mod + 8) & 7;
    const int cnt = t0 < G ? (G - t0 + 7) / 8 : 0;
    if (c == xcd) { t0c = t0; break; }
    start += cnt;
  }
  const int g = start + (tu - t0c) / 8;
  const int h = a.order[unit / a.batch];
  const int b = unit % a.batch;
  const int kvh = h / (a.heads / a.kv_heads);
  const int r0 = g * 128 + wave * 32;
  const bool active = r0 < n;

  const uint16_t *Q = (const uint16_t *)a.q + ((int64_t)b * a.heads + h) * n * D;
  const uint16_t *K = (const uint16_t *)a.k + ((int64_t)b * a.kv_heads + kvh) * n * D;
  const uint16_t *V = (const uint16_t *)a.v + ((int64_t)b * a.kv_heads + kvh) * n * D;
  uint16_t *O = (uint16_t *)a.out + ((int64_t)b * a.heads + h) * n * D;

  // ---- a3: per-wave block intervals
  int U0w = INT32_MAX, U1w = INT32_MIN, nnz = 0;
  if (active) {
    wave_setup(a.params + 2 * (int64_t)h * s, s, n, r0, lane, lead, trail, mask);
    wave_sync();
    int mn = INT32_MAX, mx = INT32_MIN;
    for (int k = lane; k < s; k += 64) {
      mn = min(mn, lead[k]);
      mx = max(mx, trail[k]);
      // rank by (lead, k) and (trail, k)
      const int32_t lk = lead[k], tk = trail[k];
      int rl = 0, rt = 0;
      for (int k2 = 0; k2 < s; ++k2) {
        const int32_t l2 = lead[k2], t2 = trail[k2];
        rl += (l2 < lk) | ((l2 == lk) & (k2 < k));
        rt += (t2 < tk) | ((t2 == tk) & (k2 < k));
      }
      lord[rl] = k;
      tord[rt] = k;
    }
    // compact list of samples with a block edge inside the wave's rows
    for (int k0 = 0; k0 < s; k0 += 64) {
      const int k = k0 + lane;
      const bool nz = k < s && mask[k] != 0u;
      const uint64_t bal = __ballot(nz);
      if (nz) nzl[nnz + __popcll(bal & ((1ull << lane) - 1ull))] = k;
      nnz += __popcll(bal);
    }
    U0w = wave_min_i(mn) & ~31;
    U1w = CAUSAL ? r0 + 32 : ((wave_max_i(mx) + 31) & ~31);
    wave_sync();
  }
  if (lane == 0) {
    lds.range[wave][0] = U0w;
    lds.range[wave][1] = U1w;
  }
  // zero this wave's histogram rows
  for (int w = lane; w < 32 * L::kHistStride; w += 64) lds.hist[wave][w] = 0u;
  __syncthreads();
  int U0 = INT32_MAX, U1 = INT32_MIN;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    U0 = min(U0, lds.range[w][0]);
    U1 = max(U1, lds.range[w][1]);
  }
  U0 &= ~(kStageKeys - 1);
  const int nst = (U1 > U0) ? (U1 - U0 + kStageKeys - 1) / kStageKeys : 0;

  // ---- Q fragment (B operand of S^T = K Q^T): query r0 + t, dims 16c + 8hh + e
  constexpr int NC = D / 16;
  bf16x8 qf[NC];
  {
    const int i = r0 + t;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (active && i < n) raw = *(const u32x4 *)(Q + (int64_t)i * D + 16 * c + 8 * hh);
      qf[c] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // ---- running state
  constexpr int NDB = D / 32;
  floatx16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m2 = -INFINITY;  // running max, log2 units
  float lsum = 0.f;      // this lane's share of the row sum
  int base_up = 0, base_dn = 0, lp = 0, tp = 0;
  const uint32_t low_t = bits_1_to(t);
  const uint32_t high_t = ~((2u << t) - 1u);
  const int arow_key = key_of_row(lane & 31);

  // ---- K/V staging (register prefetch of the next stage)
  constexpr int KCH = kStageKeys * D / 8 / 256;   // 16-byte K chunks per thread
  constexpr int VIT = kStageKeys / 2 * D / 8 / 256;  // key-pair items per thread
  u32x4 kreg[KCH], vreg[VIT][2];
  auto load_stage = [&](int st) {
    const int kb = U0 + st * kStageKeys;
#pragma unroll
    for (int it = 0; it < KCH; ++it) {
      const int id = tid + 256 * it;
      const int key = id / (D / 8), part = id % (D / 8);
      const int j = kb + key;
      kreg[it] = (j >= 0 && j < n) ? *(const u32x4 *)(K + (int64_t)j * D + 8 * part)
                                   : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int id = tid + 256 * it;
      const int kp = id % (kStageKeys / 2), part = id / (kStageKeys / 2);
      const int j = kb + 2 * kp;
      vreg[it][0] = (j >= 0 && j < n) ? *(const u32x4 *)(V + (int64_t)j * D + 8 * part)
                                      : u32x4{0u, 0u, 0u, 0u};
      vreg[it][1] = (j + 1 >= 0 && j + 1 < n) ? *(const u32x4 *)(V + (int64_t)(j + 1) * D + 8 * part)
                                              : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_stage = [&]() {
#pragma unroll
    for (int it = 0; it < KCH; ++it) {
      const int id = tid + 256 * it;
      const int key = id / (D / 8), part = id % (D / 8);
      *(u32x4 *)(lds.K + key * L::kKStride + 8 * part) = kreg[it];
    }
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int id = tid + 256 * it;
      const int kp = id % (kStageKeys / 2), part = id / (kStageKeys / 2);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = vreg[it][0][w], y = vreg[it][1][w];
        const int dim = 8 * part + 2 * w;
        *(uint32_t *)(lds.Vt + dim * L::kVStride + 2 * kp) = (x & 0xFFFFu) | (y << 16);
        *(uint32_t *)(lds.Vt + (dim + 1) * L::kVStride + 2 * kp) = (x >> 16) | (y & 0xFFFF0000u);
      }
    }
  };

  if (nst > 0) load_stage(0);
  uint32_t *hrow = &lds.hist[wave][t * L::kHistStride];

  for (int st = 0; st < nst; ++st) {
    __syncthreads();
    store_stage();
    if (st + 1 < nst) load_stage(st + 1);
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int j0 = U0 + st * kStageKeys + 32 * tt;
      if (!active || j0 < U0w || j0 >= U1w) continue;

      // a5: S^T = K Q^T
      floatx16 sacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
      const uint16_t *krow = lds.K + (32 * tt + arow_key) * L::kKStride + 8 * hh;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, *(const u32x4 *)(krow + 16 * c));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[c], sacc, 0, 0, 0);
      }

      // a4: multiplicity c for keys j0 + 16 hh + r
      const bool diag = (j0 == r0);
      const int jend = j0 + 32;
      const bool up_in = (lp < s) && (lead[lord[lp]] < jend);
      const bool dn_in = !CAUSAL && (tp < s) && (trail[tord[tp]] < jend);
      float cf[16];
      if (!diag && !up_in && !dn_in) {
        const float cu = (float)(base_up - base_dn);
#pragma unroll
        for (int r = 0; r < 16; ++r) cf[r] = cu;
      } else {
        uint32_t *hup = hrow;
        uint32_t *hdn = hrow + 8;
        while (lp < s) {
          const int k = lord[lp];
          const int32_t pos = lead[k];
          if (pos >= jend) break;
          const int rel = pos - j0;
          if ((mask[k] & low_t) == 0u && (rel >> 4) == hh)
            atomicAdd(&hup[rel >> 2], 1u << (8 * (rel & 3)));
          ++lp;
        }
        if (diag) {
          for (int z = 0; z < nnz; ++z) {
            const uint32_t mk = mask[nzl[z]];
            const uint32_t ml = mk & low_t;
            if (ml) {
              const int rel = 31 - __builtin_clz(ml);
              if ((rel >> 4) == hh) atomicAdd(&hup[rel >> 2], 1u << (8 * (rel & 3)));
            }
            if (!CAUSAL) {
              const uint32_t mh = mk & high_t;
              if (mh) {
                const int rel = __builtin_ctz(mh);
                if ((rel >> 4) == hh) atomicAdd(&hdn[rel >> 2], 1u << (8 * (rel & 3)));
              }
            }
          }
        }
        if (!CAUSAL) {
          while (tp < s) {
            const int k = tord[tp];
            const int32_t pos = trail[k];
            if (pos >= jend) break;
            const int rel = pos - j0;
            if ((mask[k] & high_t) == 0u && (rel >> 4) == hh)
              atomicAdd(&hdn[rel >> 2], 1u << (8 * (rel & 3)));
            ++tp;
          }
        }
        wave_sync();
        u32x4 up = *(const u32x4 *)(hup + 4 * hh);
        const uint32_t tot_up = prefix16(up);
        const uint32_t oth_up = other_half(tot_up, lane);
        const uint32_t add_up = (uint32_t)base_up + (hh ? oth_up : 0u);
        base_up += (int)(tot_up + oth_up);
        u32x4 cnt;
#pragma unroll
        for (int w = 0; w < 4; ++w) cnt[w] = up[w] + add_up * 0x01010101u;
        if (!CAUSAL) {
          u32x4 dn = *(const u32x4 *)(hdn + 4 * hh);
          const uint32_t tot_dn = prefix16(dn);
          const uint32_t oth_dn = other_half(tot_dn, lane);
          const uint32_t add_dn = (uint32_t)base_dn + (hh ? oth_dn : 0u);
          base_dn += (int)(tot_dn + oth_dn);
#pragma unroll
          for (int w = 0; w < 4; ++w) cnt[w] -= dn[w] + add_dn * 0x01010101u;
          *(u32x4 *)(hdn + 4 * hh) = u32x4{0u, 0u, 0u, 0u};
        }
        *(u32x4 *)(hup + 4 * hh) = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int r = 0; r < 16; ++r) cf[r] = (float)((cnt[r >> 2] >> (8 * (r & 3))) & 0xFFu);
        if (CAUSAL && diag) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (16 * hh + r > t) cf[r] = 0.f;
        }
        wave_sync();
      }

      // a6: weighted online softmax (log2 domain, lazily raised max)
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[r] *= kLog2e;
        mx = fmaxf(mx, sacc[r]);
      }
      mx = fmaxf(mx, other_half_f(mx, lane));
      const bool need = mx > m2 + 8.0f;
      if (__any(need)) {
        const float mnew = need ? mx : m2;
        const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        m2 = mnew;
      }
      bf16x8 pk[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const __bf16 pb = (__bf16)(cf[r] * __builtin_amdgcn_exp2f(sacc[r] - m2));
        pk[r >> 3][r & 7] = pb;
        lsum += (float)pb;  // the row sum uses the same rounded weights as PV
      }

      // a7: O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const uint16_t *vp = lds.Vt + (32 * db + (lane & 31)) * L::kVStride + 32 * tt + 16 * hh + 8 * cc;
          const bf16x8 av = __builtin_bit_cast(bf16x8, *(const u32x4 *)vp);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pk[cc], oacc[db], 0, 0, 0);
        }
      }
    }
  }

  // a8: normalisation epilogue, one store per output element
  if (!active) return;
  const float ltot = lsum + other_half_f(lsum, lane);
  const float inv = 1.0f / ltot;
  const int i = r0 + t;
  if (i >= n) return;
  uint16_t *orow = O + (int64_t)i * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      u32x2 w2;
      w2[0] = f32_to_bf16_bits(oacc[db][4 * gq + 0] * inv) | (f32_to_bf16_bits(oacc[db][4 * gq + 1] * inv) << 16);
      w2[1] = f32_to_bf16_bits(oacc[db][4 * gq + 2] * inv) | (f32_to_bf16_bits(oacc[db][4 * gq + 3] * inv) << 16);
      *(u32x2 *)(orow + 32 * db + 8 * gq + 4 * hh) = w2;
    }
  }
}

}  // namespace dev

// ---------------------------------------------------------------------------
// Host launch code
// ---------------------------------------------------------------------------
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
  // heavy heads first: per-row work grows with sigma
  int idx[dev::kMaxHeadsArg];
  std::iota(idx, idx + heads, 0);
  std::stable_sort(idx, idx + heads, [&](int x, int y) { return sigma[x] > sigma[y]; });
  for (int i = 0; i < dev::kMaxHeadsArg; ++i) a.order[i] = i < heads ? idx[i] : 0;
}

plsh_status launch_check(const char *who) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PLSH_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return PLSH_OK;
}

plsh_status have_device(const char *who) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PLSH_ERR_HIP, "%s: no HIP device: %s", who, hipGetErrorString(e));
  }
  return PLSH_OK;
}

plsh_status launch_valu(const dev::AttnArgs &a, int d, plsh_dtype dtype, int causal, hipStream_t st,
                        const char *who) {
  const size_t per_wave = (size_t)5 * a.s * 4 + d * 4 + 64 * 4;
  const size_t shm = 4 * per_wave;
  const dim3 grid((unsigned)((int64_t)a.groups * a.batch * a.heads)), block(256);
  if (dtype == PLSH_F32) {
    if (d == 64) hipLaunchKernelGGL((dev::attn_valu_kernel<float, 64>), grid, block, shm, st, a, causal);
    else hipLaunchKernelGGL((dev::attn_valu_kernel<float, 128>), grid, block, shm, st, a, causal);
  } else {
    if (d == 64) hipLaunchKernelGGL((dev::attn_valu_kernel<uint16_t, 64>), grid, block, shm, st, a, causal);
    else hipLaunchKernelGGL((dev::attn_valu_kernel<uint16_t, 128>), grid, block, shm, st, a, causal);
  }
  return launch_check(who);
}

plsh_status launch_mfma(const dev::AttnArgs &a, int d, int causal, hipStream_t st, const char *who) {
  const size_t shm = (size_t)4 * 6 * a.s * 4;
  const dim3 grid((unsigned)((int64_t)a.groups * a.batch * a.heads)), block(256);
  if (d == 64) {
    if (causal) hipLaunchKernelGGL((dev::attn_mfma_kernel<64, true>), grid, block, shm, st, a);
    else hipLaunchKernelGGL((dev::attn_mfma_kernel<64, false>), grid, block, shm, st, a);
  } else {
    if (causal) hipLaunchKernelGGL((dev::attn_mfma_kernel<128, true>), grid, block, shm, st, a);
    else hipLaunchKernelGGL((dev::attn_mfma_kernel<128, false>), grid, block, shm, st, a);
  }
  return launch_check(who);
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
  if (dtype == PLSH_BF16) return launch_mfma(a, d, causal != 0, (hipStream_t)stream, who);
  return launch_valu(a, d, dtype, causal != 0, (hipStream_t)stream, who);
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
  const int groups = (bt->n + 31) / 32;
  const size_t shm = (size_t)3 * bt->s * 4;
  hipLaunchKernelGGL(dev::debug_intervals_kernel, dim3((unsigned)((int64_t)groups * bt->heads)), dim3(64), shm,
                     (hipStream_t)stream, bt->params, bt->n, bt->heads, bt->s, groups, lohi);
  return launch_check(who);
}
