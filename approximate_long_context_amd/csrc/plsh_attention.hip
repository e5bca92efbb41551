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

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <numeric>
#include <utility>
#include <vector>

#include "plsh_binning.h"
#include "plsh_device.h"
#include "plsh_fwd.h"
#include "plsh_internal.h"
#include "plsh_hip_status.h"

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
  // up to a multiple of 32 (rows n .. ns - 1 hold 0).  When stat_lse2 is set
  // the MFMA kernel writes these two arrays (stat_lse2, stat_dvec) instead of
  // out; the dQ and dK/dV kernels read them (lse2, dvec).
  const void *dout;
  const float *lse2;
  const float *dvec;
  float *stat_lse2;
  float *stat_dvec;
  // when set, the MFMA kernel writes lse2 ([batch, heads, ns], rows n .. ns - 1
  // hold 0) beside out: the statistic a later backward reads
  float *save_lse2;
  // backward from a saved forward: the dQ kernel forms D = dO . O from this
  // output ([batch, heads, n, d], bf16) itself and writes it to stat_dvec
  // (rows n .. ns - 1: 0) for the dK/dV kernel, instead of reading dvec
  const void *saved_out;
  int32_t order[kMaxHeadsArg];  // head processed in slot i, heaviest sigma first
};


// Per-wave block setup for rows [r0, r0 + 32) of one head (see file header),
// in LDS scratch of the wave.
struct WaveTab {
  double *prm;     // [2s] (delta, u) of the head, staged once
  int32_t *lead;   // [s]
  int32_t *trail;  // [s]
  uint32_t *mask;  // [s]
  int32_t *act;    // [s] samples with a block start inside the wave's rows
  u32x4 *lst;      // [64][2] operands of up to 64 listed samples: (delta, u), (1 / delta, k)
};

// bytes of LDS a WaveTab needs (16-byte multiple)
__host__ __device__ constexpr size_t wavetab_bytes(int s) {
  return (((size_t)16 * s + 16 * s + 15) & ~(size_t)15) + 64 * 32;
}

__device__ __forceinline__ WaveTab carve_wavetab(uint8_t *base, int s) {
  WaveTab w;
  w.prm = (double *)base;
  w.lead = (int32_t *)(base + 16 * (size_t)s);
  w.trail = w.lead + s;
  w.mask = (uint32_t *)(w.trail + s);
  w.act = (int32_t *)(w.mask + s);
  w.lst = (u32x4 *)(base + (((size_t)16 * s + 16 * s + 15) & ~(size_t)15));
  return w;
}

// Step 1: the two half-waves take samples k = k0 + t, t = lane % 32, and run
// the same instruction stream: the lower half finds the block of row r0 (its
// first position, the lead), the upper half the block of the wave's last row
// (one past its end, the trail), each as the first position whose bin reaches
// a target (bin, or bin + 1).  The lower half stages (delta, u) in LDS and
// lists the samples whose bins differ between those rows.  Returns the number
// of listed samples (the same in every lane).
__device__ int wave_ends(const double *prm, int s, int n, int r0, int lane, const WaveTab &w) {
  const int last = min(r0 + 31, n - 1);
  const int t = lane & 31, hh = lane >> 5;
  const int x = hh ? last : r0;
  const int lo = hh ? last + 1 : 0, hi = hh ? n : r0;
  int32_t *ends = hh ? w.trail : w.lead;
  int nact = 0;
  for (int k0 = 0; k0 < s; k0 += 32) {
    const int k = k0 + t;
    double b = 0.0;
    if (k < s) {
      const double dl = prm[2 * k], u = prm[2 * k + 1];
      if (hh == 0) {
        w.prm[2 * k] = dl;
        w.prm[2 * k + 1] = u;
        w.mask[k] = 0u;
      }
      const double ri = 1.0 / dl;
      b = bin_of_r(x, dl, u, ri);
      ends[k] = first_at_least(hh ? b + 1.0 : b, lo, hi, dl, u, ri);
    }
    // (the lane swap runs with every lane active, outside the condition)
    const double bo = other_half_d(b, lane);
    const bool cross = hh == 0 && k < s && b != bo;
    const uint64_t bal = __ballot(cross);
    if (cross) w.act[nact + __popcll(bal & ((1ull << lane) - 1ull))] = k;
    nact += __popcll(bal);
  }
  return nact;
}

// x from lane l - 1 (all 64 lanes in one DPP move per half of the double;
// lane 0 gets 0): the lane's left neighbour's value without an LDS round trip
__device__ __forceinline__ double from_left_lane(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, 0x138 /* wave_shr:1 */, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), 0x138, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Step 2: start masks of the listed samples.  The two half-waves take one
// sample each and lane t evaluates the bin of position r0 + t, so a start is
// a bin change between neighbouring lanes.
__device__ void wave_masks(int n, int r0, int lane, int nact, const WaveTab &w) {
  const int last = min(r0 + 31, n - 1);
  const int t = lane & 31, hh = lane >> 5;
  const int x = r0 + t;
  for (int c0 = 0; c0 < nact; c0 += 64) {
    // the chunk's listed samples, one per lane, staged as 32-byte operand
    // records; each half-wave then reads its sample's record with two
    // broadcast reads per step
    const int m = min(64, nact - c0);
    if (lane < m) {
      const int kc = w.act[c0 + lane];
      const double dlc = w.prm[2 * kc], uc = w.prm[2 * kc + 1];
      const double ric = 1.0 / dlc;
      const uint64_t bd = (uint64_t)__double_as_longlong(dlc), bu = (uint64_t)__double_as_longlong(uc);
      const uint64_t br = (uint64_t)__double_as_longlong(ric);
      w.lst[2 * lane] = u32x4{(uint32_t)bd, (uint32_t)(bd >> 32), (uint32_t)bu, (uint32_t)(bu >> 32)};
      w.lst[2 * lane + 1] = u32x4{(uint32_t)br, (uint32_t)(br >> 32), (uint32_t)kc, 0u};
    }
    wave_sync();
#pragma unroll 2
    for (int a0 = 0; a0 < m; a0 += 2) {
      // half-wave hh takes listed sample c0 + a0 + hh
      const int src = min(a0 + hh, m - 1);
      const u32x4 r0 = w.lst[2 * src], r1 = w.lst[2 * src + 1];
      const double dl = __longlong_as_double((long long)(((uint64_t)r0[1] << 32) | r0[0]));
      const double u = __longlong_as_double((long long)(((uint64_t)r0[3] << 32) | r0[2]));
      const double ri = __longlong_as_double((long long)(((uint64_t)r1[1] << 32) | r1[0]));
      const int k = (int)r1[2];
      const bool have = a0 + hh < m;
      const bool valid = have && x <= last;
      double b = 0.0;
      if (valid) b = bin_of_r(x, dl, u, ri);
      const double bp = from_left_lane(b);  // (lanes 0 and 32 have t == 0: unused)
      const uint64_t bal = __ballot(valid && t > 0 && b != bp);
      if (t == 0 && have) w.mask[k] = (uint32_t)(bal >> (32 * hh));
    }
    wave_sync();  // every read of the records before the next chunk's
  }
}

__device__ void wave_setup(const double *prm, int s, int n, int r0, int lane, const WaveTab &w) {
  const int nact = wave_ends(prm, s, n, r0, lane, w);
  wave_sync();
  wave_masks(n, r0, lane, nact, w);
  wave_sync();
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
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const WaveTab w = carve_wavetab(smem, s);
  const int32_t *lead = w.lead, *trail = w.trail;
  const uint32_t *mask = w.mask;
  const int lane = threadIdx.x;
  const int h = blockIdx.x / groups;
  const int r0 = (blockIdx.x % groups) * 32;
  if (h >= heads) return;
  wave_setup(params + 2 * (int64_t)h * s, s, n, r0, lane, w);
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
// Grid: one 256-thread workgroup per (head slot, batch, 32-row group); each
// of its four waves sets up the group's block intervals in its own scratch
// and takes eight of the rows.
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

__host__ __device__ constexpr size_t valu_wave_bytes(int s, int D) {
  return (wavetab_bytes(s) + (size_t)8 * s + 4 * D + 256 + 15) & ~(size_t)15;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_valu_kernel(AttnArgs a, int causal, int rpw) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int s = a.s, n = a.n;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // per-wave scratch: WaveTab; rlo, rhi [s]; qrow [D]; p [64]
  uint8_t *base = smem + wave * valu_wave_bytes(s, D);
  const WaveTab w = carve_wavetab(base, s);
  const int32_t *lead = w.lead, *trail = w.trail;
  const uint32_t *mask = w.mask;
  int32_t *rlo = (int32_t *)(base + wavetab_bytes(s));
  int32_t *rhi = rlo + s;
  float *qrow = (float *)(rhi + s);
  float *pj = qrow + D;

  // rpw rows per wave (1, 2, 4 or 8): 32 / (4 rpw) workgroups per 32-row group
  const int g32 = (n + 31) / 32;
  const int wgpg = 8 / rpw;
  const int unit = blockIdx.x / (g32 * wgpg);
  const int rem = blockIdx.x - unit * g32 * wgpg;
  const int g = rem / wgpg, sub = rem % wgpg;
  const int h = a.order[unit / a.batch];
  const int b = unit % a.batch;
  const int kvh = h / (a.heads / a.kv_heads);
  const int r0 = g * 32;                    // the group's first row
  const int t_lo = (4 * sub + wave) * rpw;  // this wave's rows r0 + t_lo .. + rpw - 1
  if (r0 + t_lo >= n) return;

  const T *Q = (const T *)a.q + ((int64_t)b * a.heads + h) * n * D;
  const T *K = (const T *)a.k + ((int64_t)b * a.kv_heads + kvh) * n * D;
  const T *V = (const T *)a.v + ((int64_t)b * a.kv_heads + kvh) * n * D;
  T *O = (T *)a.out + ((int64_t)b * a.heads + h) * n * D;

  wave_setup(a.params + 2 * (int64_t)h * a.pstride, s, n, r0, lane, w);

  constexpr int E = D / 64;
  for (int t = t_lo; t < t_lo + rpw && r0 + t < n; ++t) {
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
// Workgroup = 8 waves = 128 query rows of one (batch, head).  Wave w owns the
// 16 rows r0 = 128 g + 16 w: half w % 2 of the 32-row group w / 2 whose
// block-edge record the pre-pass wrote.  Keys stream through LDS in tiles of
// 32; each wave consumes the tiles of its group's union range.  Per tile:
//   S^T (32 keys x 16 queries) = K Q^T as two v_mfma_f32_16x16x32_bf16
//     accumulators: lane l holds query r0 + l % 16 and the keys
//     16 b + 4 (l / 16) + r of the tile (b = 0, 1; r = 0..3);
//   multiplicities c: on the diagonal tile the pre-pass table; on a tile
//     holding block edges, each edge adds its step to four byte counters per
//     accumulator (keys at or after the edge); otherwise the row's running
//     count, folded into the exponent;
//   weighted online softmax in the log2 domain with a lazily raised running
//     max (only when a logit exceeds it by more than 2^8);
//   O^T (D x 16 queries) += V^T P^T with P taken straight from the
//     accumulators: k-slot 8 (l / 16) + e of the contraction stands for key
//     16 (e / 4) + 4 (l / 16) + e % 4, and the transposing LDS reads deliver
//     V^T in that order.
// Output O = acc / l is written once, rounded to bf16.  16-row waves keep a
// wave near 128 VGPRs, so four waves share each SIMD and cover each other's
// LDS and matrix-core latency.
// Q and O pass through LDS (ring slots that are free at the time) so that
// every global access instruction covers whole rows: the address unit's time
// grows with the number of 64-byte segments each group of four lanes touches,
// and a row per lane (the MFMA operand layout) touches four per group, which
// measured as the kernel's dominant address-unit cost.
// ---------------------------------------------------------------------------
// K and V stream through a ring of kRing stages of 32 keys each, filled by
// direct global->LDS loads issued one pair of stages ahead.  Rows are stored
// whole (D bf16) with their 16-byte chunks XOR-swizzled by swz_key<D>(key) so
// that both operand reads are free of bank conflicts.  The LDS has 64 banks
// of 4 bytes, so 16 lanes of a 16-byte read, or 32 lanes of an 8-byte read,
// must cover 256 distinct bytes modulo 256:
//   K operand (16-byte reads): 16 lanes read 16 consecutive keys at one
//     chunk: swz_key is a bijection of the key's low four bits (D = 64: two
//     rows share 256 bytes, so bit 0 picks the half and bits 1..3 the chunk);
//   V operand (8-byte transposing reads): 32 lanes read chunks 2j, 2j + 1 of
//     8 consecutive keys: swz_key sends those keys to distinct chunk pairs.
constexpr int kTileKeys = 32;
constexpr int kRing = 4;  // (the tile loop below is written for 4 slots)
template <int Q>
struct SlotC {
  static constexpr int value = Q;
};
constexpr int kWaves = 8;  // waves per workgroup, 16 query rows each

template <int D>
struct MfmaLds {
  alignas(16) uint16_t kv[kRing][2][kTileKeys * D];
  // step[u][k]: byte r of word k is 1 when key 4 k + r of a tile is at or
  // after tile offset u (the keys an edge at offset u counts for)
  uint32_t step[kTileKeys][kTileKeys / 4];
};


template <int D>
__device__ __forceinline__ int swz_key(int key) {
  return D == 128 ? (((key & 7) << 1) | ((key >> 3) & 1)) : ((((key >> 1) & 3) << 1) | ((key >> 3) & 1));
}

// byte offset of 16-byte chunk c of row `key` inside a swizzled tile
template <int D>
__device__ __forceinline__ uint32_t swz(int key, int c) {
  return (uint32_t)(key * D * 2 + ((c ^ swz_key<D>(key)) << 4));
}

// The forward kernel's K tiles (and its staged Q rows, read the same way)
// use a swizzle of their own at D = 128.  Measured on gfx950 (bank-conflict
// counter over single read patterns): a 16-byte read serves in one cycle the
// lanes 0..7 of a 16-lane block together with lanes 8..15 of its neighbour
// (lanes 0-7 with 24-31, 8-15 with 16-23, and likewise in the upper half),
// whereas 8-byte reads serve 32 consecutive lanes.  The K operand read has
// lane (qc, gq) read key qc at chunk 4 c + gq, so keys 0..7 of block gq and
// keys 8..15 of block gq ^ 1 share a cycle; XOR with the key's low four bits
// keeps the two halves on disjoint chunk sets (bit 3 of the chunk stays that
// of the key, XOR 4 c permuting both sets alike).  The V operand's 8-byte
// transposing reads need the key's low three bits spread over chunk pairs
// instead, which swz_key provides, so V tiles keep it.
template <int D>
__device__ __forceinline__ int swz_key_k(int key) {
  return D == 128 ? (key & 15) : swz_key<D>(key);
}

template <int D>
__device__ __forceinline__ uint32_t swz_k(int key, int c) {
  return (uint32_t)(key * D * 2 + ((c ^ swz_key_k<D>(key)) << 4));
}

// The backward dQ kernel's K and V tiles at D = 128 are stored the same way,
// with K's chunk pairs swapped like V's (piece128): K is read there both as
// a 16-byte operand (key qc, chunk 4 c + gq) and through the transposing
// reads, and the conflict counter shows both free of conflicts in that
// layout; V is read as a 16-byte operand.
__device__ __forceinline__ uint32_t piece128(int key, int chunk) {
  return (uint32_t)((chunk >> 2) * 2048 + key * 64 + (((chunk & 3) ^ (((key >> 2) & 1) << 1)) << 4));
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

// ---------------------------------------------------------------------------
// Block-edge pre-pass: one record per (head, 32-row group), in a workspace
// (record format beside its constants in plsh_device.h).
// The fp64 block searches are latency-bound; as a kernel of their own they
// run at high occupancy instead of stalling the MFMA kernel.
// ---------------------------------------------------------------------------

// With CAUSAL false and ws_causal set, the same pass also writes the causal
// record of every group to ws_causal: the same sorted leads, the group's end
// as its key limit, and the diagonal table without the keys after the row
// (the block ends only count for those keys, so the rest is the same).
template <bool CAUSAL>
__global__ __launch_bounds__(256) void edges_kernel(const double *params, int pstride, int n, int heads, int s,
                                                    int g32, uint8_t *ws, uint8_t *ws_causal) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = lane & 31, hh = lane >> 5;
  const int item = blockIdx.x * 4 + wave;
  if (item >= heads * g32) return;
  const int h = item / g32, q = item % g32;
  const int r0 = 32 * q;
  uint8_t *wb = smem + wave * (wavetab_bytes(s) + 32 * 16 * 4);
  const WaveTab w = carve_wavetab(wb, s);
  uint32_t *hist = (uint32_t *)(wb + wavetab_bytes(s));  // [32 rows][16 dwords]: up 0..7, down 8..15
  for (int i = lane; i < 32 * 16; i += 64) hist[i] = 0u;
  // head h's s hashes are rows h * pstride .. + s - 1 of params
  const int nact = wave_ends(params + 2 * (int64_t)h * pstride, s, n, r0, lane, w);
  wave_sync();
  wave_masks(n, r0, lane, nact, w);
  wave_sync();
  uint8_t *rec = ws + (size_t)item * rec_bytes(s);
  u32x2 *evl = (u32x2 *)(rec + rec_evl_off());
  u32x2 *evt = (u32x2 *)(rec + rec_evt_off(s));
  uint8_t *rec_c = (!CAUSAL && ws_causal) ? ws_causal + (size_t)item * rec_bytes(s) : nullptr;
  u32x2 *evl_c = rec_c ? (u32x2 *)(rec_c + rec_evl_off()) : nullptr;
  int mn = INT32_MAX, mx = INT32_MIN;
  for (int k = lane; k < s; k += 64) {
    const int32_t lk = w.lead[k], tk = w.trail[k];
    const uint32_t mk = w.mask[k];
    mn = min(mn, lk);
    mx = max(mx, tk);
    int rl = 0, rt = 0;
#pragma unroll 4
    for (int k2 = 0; k2 < s; ++k2) {
      const int32_t l2 = w.lead[k2], t2 = w.trail[k2];
      rl += (l2 < lk) | ((l2 == lk) & (k2 < k));
      rt += (t2 < tk) | ((t2 == tk) & (k2 < k));
    }
    const uint32_t ml = mk & ~1u;  // starts inside rows r0 + 1 .. r0 + 31
    const uint32_t wl = ml ? ((1u << __builtin_ctz(ml)) - 1u) : 0xFFFFFFFFu;
    const uint32_t wt = mk ? ~((1u << (31 - __builtin_clz(mk))) - 1u) : 0xFFFFFFFFu;
    evl[rl] = u32x2{(uint32_t)lk, wl};
    if (!CAUSAL) evt[rt] = u32x2{(uint32_t)tk, wt};
    if (evl_c) evl_c[rl] = u32x2{(uint32_t)lk, wl};
  }
  if (lane < kSentinels) {
    evl[s + lane] = u32x2{0x7FFFFFFFu, 0u};
    if (!CAUSAL) evt[s + lane] = u32x2{0x7FFFFFFFu, 0u};
    if (evl_c) evl_c[s + lane] = u32x2{0x7FFFFFFFu, 0u};
  }
  const int U0w = wave_min_i(mn) & ~31;
  const int U1w = CAUSAL ? r0 + 32 : ((wave_max_i(mx) + 31) & ~31);
  if (lane == 0) *(int4 *)rec = make_int4(nact, U0w, U1w, 0);
  if (rec_c && lane == 0) *(int4 *)rec_c = make_int4(nact, U0w, r0 + 32, 0);

  // diagonal tile: row t's block starts inside the rows (highest mask bit <= t)
  // and, non-causal, its block ends inside them (lowest bit > t), as per-row
  // byte histograms; prefix sums give the counts
  const uint32_t low_t = bits_1_to(t), high_t = ~((2u << t) - 1u);
  uint32_t *hup = hist + 16 * t, *hdn = hup + 8;
  for (int z = 0; z < nact; ++z) {
    const uint32_t mk = w.mask[w.act[z]];
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
  wave_sync();
  u32x4 hu = *(const u32x4 *)(hup + 4 * hh);
  const uint32_t tu = prefix16(hu);
  const uint32_t ou = other_half(tu, lane);
  // samples whose block of row t starts at or before r0 count for every key
  const uint32_t before = (uint32_t)s - tu - ou;
  u32x4 c;
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = hu[i] + (before + (hh ? ou : 0u)) * 0x01010101u;
  if (!CAUSAL) {
    u32x4 hd = *(const u32x4 *)(hdn + 4 * hh);
    const uint32_t td = prefix16(hd);
    const uint32_t od = other_half(td, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] -= hd[i] + (hh ? od : 0u) * 0x01010101u;
  }
  const int last = min(r0 + 31, n - 1);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int u = 16 * hh + 4 * i + r;
      if ((CAUSAL && u > t) || r0 + u > last) c[i] &= ~(0xFFu << (8 * r));
    }
  *(u32x4 *)(rec + rec_diag_off(s) + 32 * t + 16 * hh) = c;
  if (rec_c) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (16 * hh + 4 * i + r > t) c[i] &= ~(0xFFu << (8 * r));
    *(u32x4 *)(rec_c + rec_diag_off(s) + 32 * t + 16 * hh) = c;
  }
}


template <int D, bool CAUSAL, bool WALK = false>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kWaves, 64 * kWaves), amdgpu_waves_per_eu(4, 4)))
void attn_mfma_kernel(AttnArgs a, const uint8_t *ws) {
  using L = MfmaLds<D>;
  __shared__ __attribute__((aligned(16))) L lds;
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  // WALK: the samples one by one (a.s of them), each through its own
  // single-sample records (0/1 masks); otherwise all samples fused, s = a.s
  const int s = WALK ? 1 : a.s, n = a.n;
  const int nwalk = WALK ? a.s : 1;
  // the wave index is wave-uniform; saying so keeps all per-wave control flow
  // on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int qc = lane & 15, gq = lane >> 4;
  // the step table, complete after the first stage's barrier
  if (threadIdx.x < kTileKeys * kTileKeys / 4) {
    const int u = threadIdx.x >> 3, k = threadIdx.x & 7;
    lds.step[u][k] = step4(u - 4 * k);
  }

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
  const int grp = wave >> 1, half = wave & 1;  // 32-row group of the workgroup, and which half
  const int rg = g * 128 + 32 * grp;           // the group's first row
  const int r0 = rg + 16 * half;               // this wave's first row
  const bool active = r0 < n;
  const int t32 = 16 * half + qc;              // the lane's row within its group
  const int g32 = (n + 31) / 32;
  const size_t rb = rec_bytes(s);

  const uint16_t *Q = (const uint16_t *)a.q + ((int64_t)b * a.heads + h) * n * D;
  const uint16_t *K = (const uint16_t *)a.k + ((int64_t)b * a.kv_heads + kvh) * n * D;
  const uint16_t *V = (const uint16_t *)a.v + ((int64_t)b * a.kv_heads + kvh) * n * D;
  uint16_t *O = (uint16_t *)a.out + ((int64_t)b * a.heads + h) * n * D;

  constexpr int NC = D / 32;
  // the Q fragment (B operand of S^T = K Q^T: query r0 + qc, dims 32 c +
  // 8 gq + e), read from LDS after the first wait (see below)
  bf16x8 qf[NC];
  constexpr int CPR_Q = D / 8;  // 16-byte chunks per query row
  constexpr int NDB = D / 16;   // 16-dim blocks of O^T
  floatx4 oacc[NDB];
  float m2;    // running max, log2 units
  float lsum;  // this lane's share of the row sum
  int nst = 0;
  for (int kk = 0; kk < nwalk; ++kk) {
    if (kk > 0) {
      // every wave is past the previous sample's tiles before its edge
      // lists and ring slots are refilled
      PLSH_WAIT_VM_LGKM0(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    const uint8_t *rec_wg = ws + ((size_t)(WALK ? h * nwalk + kk : h) * g32 + 4 * g) * rb;
    const uint8_t *rec = rec_wg + (size_t)grp * rb;
    // ---- the four groups' key ranges first (the K/V copies need them), then
    // the row's diagonal-tile multiplicities
    int U0 = INT32_MAX, U1 = INT32_MIN, U0w = INT32_MAX, U1w = INT32_MIN;
    {
      // all four headers in one round trip: groups past the end re-read the
      // last valid one (their ranges then add nothing)
      const int wlast = min(3, (n - 1 - g * 128) / 32);
      int4 hdr[4];
  #pragma unroll
      for (int w = 0; w < 4; ++w) hdr[w] = *(const int4 *)(rec_wg + (size_t)min(w, wlast) * rb);
  #pragma unroll
      for (int w = 0; w < 4; ++w) {
        U0 = min(U0, hdr[w].y);
        U1 = max(U1, hdr[w].z);
        if (w == grp) { U0w = hdr[w].y; U1w = hdr[w].z; }
      }
    }
    // bytes c(t32, 16 b + 4 gq + r), and (non-causal) c(t32, 31)
    uint32_t dg[2] = {0u, 0u};
    int dlast = 0;
    if (active) {
      const uint8_t *drow = rec + rec_diag_off(s) + 32 * t32;
      dg[0] = *(const uint32_t *)(drow + 4 * gq);
      dg[1] = *(const uint32_t *)(drow + 16 + 4 * gq);
      if (!CAUSAL) dlast = (int)(*(const uint32_t *)(drow + 28) >> 24);
    }
    // stage st covers keys [U0 + 32 st, U0 + 32 st + 32)
    nst = (U1 > U0) ? (U1 - U0) / kTileKeys : 0;
    // Everything loaded so far is needed before the first tile.  Waiting here,
    // before the first K/V copies are issued, measured faster than letting the
    // first stage waits cover these loads.
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)

    // the group's sorted edge lists, copied by its first wave into the group's
    // LDS slice (16 bytes = two edges per lane and instruction); they are
    // complete for both waves after the first stage's barrier
    const int nch = ev_count(s) / 2;
    u32x2 *evl = (u32x2 *)(dyn + (size_t)grp * ev_wave_bytes(s, CAUSAL));
    u32x2 *evt = evl + ev_count(s);
    if (active && half == 0) {
      for (int c0 = 0; c0 < nch; c0 += 64)
        if (c0 + lane < nch) dma16(rec + rec_evl_off() + 16 * (c0 + lane), lds_addr(evl + 2 * c0));
      if (!CAUSAL)
        for (int c0 = 0; c0 < nch; c0 += 64)
          if (c0 + lane < nch) dma16(rec + rec_evt_off(s) + 16 * (c0 + lane), lds_addr(evt + 2 * c0));
    }

    // ---- the wave's 16 query rows go to ring slots 2 and 3 (free until the
    // first pair has read them) in the swizzled layout of a K tile, so that
    // every copy instruction reads whole rows and the fragment reads are free of
    // bank conflicts (whole rows per instruction keep the address unit's work
    // per byte low; a row per lane would touch 16 rows per instruction)
    const uint32_t q_lds = lds_addr(&lds.kv[2][0][0]) + wave * 32 * D;
    if (active && kk == 0) {  // (staged once)
  #pragma unroll
      for (int c0 = 0; c0 < 16 * CPR_Q; c0 += 64) {
        const int row = (c0 + lane) / CPR_Q, ch = (c0 + lane) % CPR_Q;
        const int64_t off = (int64_t)min(r0 + row, n - 1) * (2 * D) + 16 * (ch ^ swz_key_k<D>(row));
        dma16((const char *)Q + off, q_lds + 16 * c0);
      }
    }

    // ---- K/V staging: a tile is 32 rows of D / 8 chunks, 4 D chunks per
    // matrix; wave w copies chunks [w CPW, (w + 1) CPW) with its first CPW
    // lanes.  Keys past the end read row n - 1, whose products get c = 0.
    constexpr int CPR = D / 8;            // chunks per row
    constexpr int CPW = 4 * D / kWaves;   // chunks per wave, stage and matrix (<= 64)
    constexpr int LPS = 2;                // loads per thread per stage (K and V)
    const char *Kb = (const char *)K, *Vb = (const char *)V;
    // the lane's chunk of every stage: row dkey of the tile, 16 bytes at
    // dofs_k (K tile) and dofs_v (V tile)
    const int dslot = wave * CPW + lane;
    const int dkey = dslot / CPR;
    const int dofs_k = 16 * ((dslot % CPR) ^ swz_key_k<D>(dkey));
    // V (D = 128): slot dslot holds key (dslot / 4) % 32, chunk 4 (dslot / 128)
    // + (dslot % 4 with its pair swapped by bit 2 of the key); else as K rows
    const int vkey = D == 128 ? (dslot >> 2) & 31 : dkey;
    const int dofs_v = D == 128 ? 16 * (4 * (dslot >> 7) + ((dslot & 3) ^ (((vkey >> 2) & 1) << 1)))
                                : 16 * ((dslot % CPR) ^ swz_key<D>(dkey));
    const uint32_t kv_lds = lds_addr(&lds.kv[0][0][0]) + wave * CPW * 16;
    auto issue_stage = [&](int st, int q) {  // q = st % kRing
      if (lane < CPW) {
        const int64_t row = (int64_t)min(U0 + kTileKeys * st + dkey, n - 1) * (2 * D);
        const int64_t vrow = (int64_t)min(U0 + kTileKeys * st + vkey, n - 1) * (2 * D);
        dma16(Kb + row + dofs_k, kv_lds + (uint32_t)(2 * q) * (kTileKeys * D * 2));
        dma16(Vb + vrow + dofs_v, kv_lds + (uint32_t)(2 * q + 1) * (kTileKeys * D * 2));
      }
    };
    // stages 0 and 1 now; the pair starting at stage st issues st + 2, st + 3
    if (nst > 0) issue_stage(0, 0);
    if (nst > 1) issue_stage(1, 1);

    // ---- running state
    if (kk == 0) {  // (over every sample when walking them)
  #pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] = floatx4{0.f, 0.f, 0.f, 0.f};
      m2 = -INFINITY;
      lsum = 0.f;
    }
    int base = 0;          // the row's multiplicity just before the current tile
    int lp = 0, tp = 0;    // next unconsumed lead / trail edge
    int pl = 0, pt = 0;    // their positions (wave-uniform)
    int lg_base = -1;      // the count whose log2 is lg
    float lg = 0.f;
    // edge positions read at a wave-uniform index are wave-uniform
    auto pos_at = [&](const u32x2 *ev, int i) { return (int32_t)__builtin_amdgcn_readfirstlane(ev[i][0]); };
    // K operand: key 16 b + qc, chunk 4 c + gq; b = 1 lies 16 rows further
    uint32_t kofs[NC];
  #pragma unroll
    for (int c = 0; c < NC; ++c) kofs[c] = swz_k<D>(qc, 4 * c + gq);
    // V operand (v_ds_read_b64_tr_b16): in each 16-lane group gq, lane r names
    // the row (key 4 gq + r / 4, dims 16 db + 4 (r % 4) .. + 3), and lane i
    // receives V[4 gq + e][16 db + i], e = 0..3; keys + 16 lie vhi bytes
    // further.  At D = 128 (vpiece128) the offsets of dim blocks db and
    // db + 2 differ by 2048: two bases, the rest immediates.
    uint32_t vofs[NDB];
    constexpr uint32_t vhi = D == 128 ? 16 * 64 : 16 * 2 * D;
    if constexpr (D == 128) {
      const int vk = 4 * gq + (qc >> 2);
      uint32_t vb[2];
  #pragma unroll
      for (int e = 0; e < 2; ++e) vb[e] = vpiece128(vk, 2 * e + ((qc >> 1) & 1)) + 8 * (qc & 1);
  #pragma unroll
      for (int db = 0; db < NDB; ++db) vofs[db] = vb[db & 1] + 2048 * (db >> 1);
    } else {
  #pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int dim = 16 * db + 4 * (qc & 3);
        vofs[db] = swz<D>(4 * gq + (qc >> 2), dim >> 3) + ((dim & 4) << 1);
      }
    }

    // this wave's tiles are the stages [sa, sb)
    const int sa = active ? (U0w - U0) / kTileKeys : 0;
    const int sb = active ? (U1w - U0) / kTileKeys : 0;

    // a5: S^T = K Q^T for the tile of stage st, keys 16 b + 4 gq + r
    floatx4 sacc[2];
    // (the ring slot is a compile-time constant, so that LDS operand offsets
    // become immediates of the reads)
    auto qk_tile = [&](auto slotc) {
      const char *kt = (const char *)lds.kv[decltype(slotc)::value][0];
  #pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        u32x4 kr[NC];
  #pragma unroll
        for (int c = 0; c < NC; ++c) kr[c] = *(const u32x4 *)(kt + kofs[c] + 32 * D * bb);
        sacc[bb] = floatx4{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
        for (int c = 0; c < NC; ++c)
          sacc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[c]), qf[c], sacc[bb], 0, 0, 0);
      }
    };

    // Visits, in order, the edges of a sorted list at positions < jend starting
    // at index ptr (position pp), and advances ptr / pp past them.  Lane l reads
    // edge ptr + l, so up to 64 edges are found with one LDS read and a ballot
    // (the list ends in 16 sentinels at INT32_MAX; reads stay inside it).
    const int ev_last = s + kSentinels - 1;
    auto edges_in_tile = [&](const u32x2 *ev, int &ptr, int &pp, int jend, auto &&visit) {
      while (pp < jend) {
        const u32x2 e = ev[min(ptr + lane, ev_last)];
        const int k = __popcll(__ballot((int32_t)e[0] < jend));  // a prefix of the lanes
        for (int i = 0; i < k; ++i)
          visit((int32_t)__builtin_amdgcn_readlane(e[0], i), __builtin_amdgcn_readlane(e[1], i));
        ptr += k;
        pp = k < 64 ? (int32_t)__builtin_amdgcn_readlane(e[0], k) : pos_at(ev, ptr);
      }
    };

    // a4, a6, a7 for the tile of stage st, whose logits are in sacc
    auto finish_tile = [&](int st, auto slotc) {
      const char *vt = (const char *)lds.kv[decltype(slotc)::value][1];
      const int j0 = U0 + kTileKeys * st;

      // a4: multiplicity c for keys j0 + 16 b + 4 gq + r.
      //  * diagonal tile: the row's bytes of the precomputed table;
      //  * a tile holding sample edges (lower block ends = leads on the left of
      //    the diagonal, upper ends = trails on the right; positions are
      //    wave-uniform): c = base +- sum over edges of w_e(row) [key >= pos_e],
      //    four keys per byte-counter word;
      //  * otherwise c = base for all keys of the tile.
      const int jend = j0 + kTileKeys;
      float cf[8];
      int kind;  // 0: one count for the tile, 1: per-key counts
      if (j0 == rg) {
        // (kept here: hoisted out of the loop, the conversion would wait for
        // the table load, and with it for every K/V copy issued after it)
        uint32_t d0 = dg[0], d1 = dg[1];
        asm volatile("" : "+v"(d0), "+v"(d1));
  #pragma unroll
        for (int r = 0; r < 8; ++r) cf[r] = (float)((((r >> 2) ? d1 : d0) >> (8 * (r & 3))) & 0xFFu);
        // the table already counts every edge at or before the tile's end
        edges_in_tile(evl, lp, pl, jend, [](int, uint32_t) {});
        if (!CAUSAL) {
          edges_in_tile(evt, tp, pt, jend, [](int, uint32_t) {});
          base = dlast;
        }
        kind = 1;
      } else if (pl < jend || (!CAUSAL && pt < jend)) {
        // the lane's keys are words gq and gq + 4 of the tile's step rows
        const uint32_t *srow = &lds.step[0][gq];
        uint32_t cw[2] = {(uint32_t)base * 0x01010101u, (uint32_t)base * 0x01010101u};
        // leads: the sample's block of the row starts at pos
        edges_in_tile(evl, lp, pl, jend, [&](int pos, uint32_t W) {
          const uint32_t w = (W >> t32) & 1u;
          const uint32_t *sr = srow + 8 * (pos - j0);
          cw[0] += w * sr[0];
          cw[1] += w * sr[4];
          base += (int)w;
        });
        // trails: the sample's block of the row ends before pos
        if (!CAUSAL)
          edges_in_tile(evt, tp, pt, jend, [&](int pos, uint32_t W) {
            const uint32_t w = (W >> t32) & 1u;
            const uint32_t *sr = srow + 8 * (pos - j0);
            cw[0] -= w * sr[0];
            cw[1] -= w * sr[4];
            base -= (int)w;
          });
  #pragma unroll
        for (int r = 0; r < 8; ++r) cf[r] = (float)((cw[r >> 2] >> (8 * (r & 3))) & 0xFFu);
        kind = 1;
      } else {
        cf[0] = (float)base;
        kind = 0;
      }

      // a6: weighted online softmax in the log2 domain.  The running max is
      // raised only when a logit exceeds it by more than 2^8 (the result does
      // not depend on the max used, and a rescale of the accumulators is then
      // rare).  A tile with one count per row folds log2(c) into the exponent
      // bias; otherwise P = c * 2^(...).  P is rounded to bf16 in pairs and the
      // row sum adds exactly the rounded weights that enter PV.
      // (raw v_max3_f32: one instruction per three finite logits)
      auto mx2 = [](float x, float y) { return max3f(x, y, y); };
      float mx = max3f(max3f(sacc[0][0], sacc[0][1], sacc[0][2]), max3f(sacc[0][3], sacc[1][0], sacc[1][1]),
                       max3f(sacc[1][2], sacc[1][3], sacc[1][3]));
      // the lane's own maximum decides whether any rescale is due; only then
      // is it combined over the four lanes of each query
      if (__any(mx * kLog2e > m2 + 8.0f)) {
        mx = mx2(mx, xor16_f(mx));
        mx = mx2(mx, other_half_f(mx, lane)) * kLog2e;
        const bool need = mx > m2 + 8.0f;
        const float mnew = need ? mx : m2;
        const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);
        lsum *= alpha;
  #pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
        m2 = mnew;
      }
      u32x4 pw;
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
      if (__builtin_amdgcn_readfirstlane(kind) == 0) {
        if (__any(base != lg_base)) {  // log2 of the running count, recomputed when it changes
          lg = __builtin_amdgcn_logf(cf[0]);
          lg_base = base;
        }
        const float bias = m2 - lg;  // c = 0 gives bias = +inf, P = 0
  #pragma unroll
        for (int r = 0; r < 8; r += 2) {
          const floatx2 pf = {__builtin_amdgcn_exp2f(fmaf(sacc[r >> 2][r & 3], kLog2e, -bias)),
                              __builtin_amdgcn_exp2f(fmaf(sacc[r >> 2][(r & 3) + 1], kLog2e, -bias))};
          const bf16x2 pb = __builtin_convertvector(pf, bf16x2);
          pw[r >> 1] = __builtin_bit_cast(uint32_t, pb);
          lsum = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, lsum, false);
        }
      } else {
  #pragma unroll
        for (int r = 0; r < 8; r += 2) {
          const floatx2 pf = {cf[r] * __builtin_amdgcn_exp2f(fmaf(sacc[r >> 2][r & 3], kLog2e, -m2)),
                              cf[r + 1] * __builtin_amdgcn_exp2f(fmaf(sacc[r >> 2][(r & 3) + 1], kLog2e, -m2))};
          const bf16x2 pb = __builtin_convertvector(pf, bf16x2);
          pw[r >> 1] = __builtin_bit_cast(uint32_t, pb);
          lsum = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, lsum, false);
        }
      }
      const bf16x8 pk = __builtin_bit_cast(bf16x8, pw);

      // a7: O^T += V^T P^T, the V operand read in two batches of 16-dim blocks
      constexpr int NB = NDB < 4 ? NDB : 4;
  #pragma unroll
      for (int d0 = 0; d0 < NDB; d0 += NB) {
        u32x4 vop[NB];
  #pragma unroll
        for (int j = 0; j < NB; ++j) {
          const char *va = vt + vofs[d0 + j];
          const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t *)va);
          const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t *)(va + vhi));
          vop[j] = u32x4{__builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1)),
                         __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3)),
                         __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1)),
                         __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3))};
        }
  #pragma unroll
        for (int j = 0; j < NB; ++j)
          oacc[d0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vop[j]), pk, oacc[d0 + j], 0, 0, 0);
      }
    };

    // Two stages per barrier (measured: the barrier, where every wave waits for
    // the slowest, costs more than the shorter look-ahead): the pair starting at
    // stage st waits for stages st, st + 1, then refills the ring slots of
    // stages st - 2, st - 1 (consumed by every wave before the barrier) with
    // stages st + 2, st + 3, and computes its two tiles.
    auto pair = [&](int st, auto s0, auto s1) {
      PLSH_WAIT_VM_LGKM0(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (st == 0 && kk == 0) {
        // the Q fragment from the wave's staged rows, then a barrier: every wave
        // has its fragment before slots 2, 3 take stages 2, 3
        const char *qt = (const char *)lds.kv[2][0] + wave * 32 * D;
  #pragma unroll
        for (int c = 0; c < NC; ++c) qf[c] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qt + swz_k<D>(qc, 4 * c + gq)));
        PLSH_WAIT_VM_LGKM0(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
      if (st + 2 < nst) issue_stage(st + 2, (decltype(s0)::value + 2) % kRing);
      if (st + 3 < nst) issue_stage(st + 3, (decltype(s1)::value + 2) % kRing);
      if (st == 0 && active) {  // the edge lists landed with stage 0
        pl = pos_at(evl, 0);
        if (!CAUSAL) pt = pos_at(evt, 0);
      }
      if (st >= sa && st < sb) {
        qk_tile(s0);
        finish_tile(st, s0);
      }
      if (st + 1 < nst && st + 1 >= sa && st + 1 < sb) {
        qk_tile(s1);
        finish_tile(st + 1, s1);
      }
    };
    for (int st0 = 0; st0 < nst; st0 += kRing) {
      pair(st0, SlotC<0>{}, SlotC<1>{});
      if (st0 + 2 < nst) pair(st0 + 2, SlotC<2>{}, SlotC<3>{});
    }
  }

  // a8: normalisation epilogue, one store per output element; the row sum
  // is spread over the four lanes qc + 16 gq
  // The wave's 16 x D output block is staged in LDS (in the two ring slots
  // the last pair does not use: every wave is past them), then written whole
  // rows per instruction.
  const int ns = (n + 31) & ~31;
  const int64_t srow = ((int64_t)b * a.heads + h) * ns + r0 + qc;
  if (!active) {
    if (a.stat_lse2 && r0 < ns && gq == 0) a.stat_lse2[srow] = a.stat_dvec[srow] = 0.f;
    if (a.save_lse2 && r0 < ns && gq == 0) a.save_lse2[srow] = 0.f;
    return;
  }
  float ltot = lsum + xor16_f(lsum);
  ltot += other_half_f(ltot, lane);
  const float inv = 1.0f / ltot;
  if (a.stat_lse2) {
    // backward statistics of the row: lse2 and D = dO . O (O in fp32, before
    // its rounding); the lane holds dims 16 db + 4 gq .. + 3
    const int io = r0 + qc;
    const uint16_t *dOr = (const uint16_t *)a.dout + (((int64_t)b * a.heads + h) * n + min(io, n - 1)) * D + 4 * gq;
    float acc = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const u32x2 raw = *(const u32x2 *)(dOr + 16 * db);
      acc = fmaf(__uint_as_float(raw[0] << 16), oacc[db][0], acc);
      acc = fmaf(__uint_as_float(raw[0] & 0xFFFF0000u), oacc[db][1], acc);
      acc = fmaf(__uint_as_float(raw[1] << 16), oacc[db][2], acc);
      acc = fmaf(__uint_as_float(raw[1] & 0xFFFF0000u), oacc[db][3], acc);
    }
    acc += xor16_f(acc);
    acc += other_half_f(acc, lane);
    if (gq == 0) {
      a.stat_lse2[srow] = io < n ? m2 + __log2f(ltot) : 0.f;
      a.stat_dvec[srow] = io < n ? acc * inv : 0.f;
    }
    return;
  }
  if (a.o32) {
    // fp32 partials for a log-sum-exp combine: O (normalised) and lse, in
    // natural-log units (the running max m2 is in log2 units)
    const int io = r0 + qc;
    if (io < n) {
      const int64_t row = ((int64_t)b * a.heads + h) * n + io;
      float *orow = a.o32 + row * D + 4 * gq;
#pragma unroll
      for (int db = 0; db < NDB; ++db) *(floatx4 *)(orow + 16 * db) = oacc[db] * inv;
      if (gq == 0) a.lse[row] = (m2 + __log2f(ltot)) * 0.6931471805599453f;
    }
    return;
  }
  if (a.save_lse2 && gq == 0) a.save_lse2[srow] = r0 + qc < n ? m2 + __log2f(ltot) : 0.f;
  const int free_slot = (((nst - 1) >> 1) & 1) ? 0 : 2;
  char *ob = (char *)lds.kv[free_slot][0] + wave * 32 * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const bf16x2 h0 = __builtin_convertvector((floatx2{oacc[db][0] * inv, oacc[db][1] * inv}), bf16x2);
    const bf16x2 h1 = __builtin_convertvector((floatx2{oacc[db][2] * inv, oacc[db][3] * inv}), bf16x2);
    // row qc, dims 16 db + 4 gq .. + 3: half (gq & 1) of 16-byte chunk 2 db + gq / 2
    *(u32x2 *)(ob + swz<D>(qc, 2 * db + (gq >> 1)) + 8 * (gq & 1)) =
        u32x2{__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1)};
  }
#pragma unroll
  for (int c0 = 0; c0 < 16 * CPR_Q; c0 += 64) {
    const int row = (c0 + lane) / CPR_Q, ch = (c0 + lane) % CPR_Q;
    const u32x4 val = *(const u32x4 *)(ob + swz<D>(row, ch));
    const int i = r0 + row;
    if (i < n) *(u32x4 *)(O + (int64_t)i * D + 8 * ch) = val;
  }
}

// ---------------------------------------------------------------------------
// Backward, dQ (gradients of the estimate for fixed tables; the pages train
// with the method, Experimental Validation).  The forward's structure -- the
// same records, multiplicities, ring and Q staging -- with the normaliser
// known (lse2 from a statistics pass) instead of an online softmax:
//   P_ij = c_ij 2^(q_i.k_j log2 e - lse2_i),  dP^T = V dO^T (MFMA),
//   dS = P o (dP - D_i),  dQ_i = sum_j dS_ij k_j  (dQ^T += K^T dS^T, MFMA,
//   the K tile read through the transposing LDS reads).
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kWaves, 64 * kWaves), amdgpu_waves_per_eu(4, 4)))
void attn_dq_kernel(AttnArgs a, const uint8_t *ws) {
  using L = MfmaLds<D>;
  __shared__ __attribute__((aligned(16))) L lds;
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  const int s = a.s, n = a.n;
  // the wave index is wave-uniform; saying so keeps all per-wave control flow
  // on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int qc = lane & 15, gq = lane >> 4;
  // the step table, complete after the first stage's barrier
  if (threadIdx.x < kTileKeys * kTileKeys / 4) {
    const int u = threadIdx.x >> 3, k = threadIdx.x & 7;
    lds.step[u][k] = step4(u - 4 * k);
  }

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
  const int grp = wave >> 1, half = wave & 1;  // 32-row group of the workgroup, and which half
  const int rg = g * 128 + 32 * grp;           // the group's first row
  const int r0 = rg + 16 * half;               // this wave's first row
  const bool active = r0 < n;
  const int t32 = 16 * half + qc;              // the lane's row within its group
  const int g32 = (n + 31) / 32;
  const size_t rb = rec_bytes(s);
  const uint8_t *rec_wg = ws + ((size_t)h * g32 + 4 * g) * rb;
  const uint8_t *rec = rec_wg + (size_t)grp * rb;

  const uint16_t *Q = (const uint16_t *)a.q + ((int64_t)b * a.heads + h) * n * D;
  const uint16_t *K = (const uint16_t *)a.k + ((int64_t)b * a.kv_heads + kvh) * n * D;
  const uint16_t *V = (const uint16_t *)a.v + ((int64_t)b * a.kv_heads + kvh) * n * D;
  uint16_t *O = (uint16_t *)a.out + ((int64_t)b * a.heads + h) * n * D;

  // ---- the four groups' key ranges first (the K/V copies need them), then
  // the row's diagonal-tile multiplicities
  int U0 = INT32_MAX, U1 = INT32_MIN, U0w = INT32_MAX, U1w = INT32_MIN;
  {
    // all four headers in one round trip: groups past the end re-read the
    // last valid one (their ranges then add nothing)
    const int wlast = min(3, (n - 1 - g * 128) / 32);
    int4 hdr[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) hdr[w] = *(const int4 *)(rec_wg + (size_t)min(w, wlast) * rb);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      U0 = min(U0, hdr[w].y);
      U1 = max(U1, hdr[w].z);
      if (w == grp) { U0w = hdr[w].y; U1w = hdr[w].z; }
    }
  }
  constexpr int NC = D / 32;
  // the Q fragment (B operand of S^T = K Q^T: query r0 + qc, dims 32 c +
  // 8 gq + e), read from LDS after the first wait (see below)
  bf16x8 qf[NC];
  // bytes c(t32, 16 b + 4 gq + r), and (non-causal) c(t32, 31)
  uint32_t dg[2] = {0u, 0u};
  int dlast = 0;
  if (active) {
    const uint8_t *drow = rec + rec_diag_off(s) + 32 * t32;
    dg[0] = *(const uint32_t *)(drow + 4 * gq);
    dg[1] = *(const uint32_t *)(drow + 16 + 4 * gq);
    if (!CAUSAL) dlast = (int)(*(const uint32_t *)(drow + 28) >> 24);
  }
  // stage st covers keys [U0 + 32 st, U0 + 32 st + 32)
  const int nst = (U1 > U0) ? (U1 - U0) / kTileKeys : 0;
  // the dO fragment (B operand of dP^T = V dO^T, laid out as the Q
  // fragment), the row's normaliser and D = dO . O
  const uint16_t *dOp = (const uint16_t *)a.dout + ((int64_t)b * a.heads + h) * n * D;
  bf16x8 dof[NC];
  float lse2r = 0.f, dvr = 0.f;
  {
    const int i = r0 + qc;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (active && i < n) raw = *(const u32x4 *)(dOp + (int64_t)i * D + 32 * c + 8 * gq);
      dof[c] = __builtin_bit_cast(bf16x8, raw);
    }
    const int ns = (n + 31) & ~31;
    const int64_t row = ((int64_t)b * a.heads + h) * ns + i;  // rows padded to 32
    if (active && i < n) {
      lse2r = a.lse2[row];
      if (!a.saved_out) dvr = a.dvec[row];
    }
    if (a.saved_out) {
      // D_i = dO_i . O_i from the saved output, in the dO fragment's layout:
      // the lane's 8 NC dims, then the sum over the row's four lanes
      const uint16_t *Op = (const uint16_t *)a.saved_out + ((int64_t)b * a.heads + h) * n * D;
      float acc = 0.f;
      if (active && i < n) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const u32x4 o = *(const u32x4 *)(Op + (int64_t)i * D + 32 * c + 8 * gq);
          const u32x4 g = __builtin_bit_cast(u32x4, dof[c]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc = fmaf(__uint_as_float(o[e] << 16), __uint_as_float(g[e] << 16), acc);
            acc = fmaf(__uint_as_float(o[e] & 0xFFFF0000u), __uint_as_float(g[e] & 0xFFFF0000u), acc);
          }
        }
      }
      acc += xor16_f(acc);
      acc += other_half_f(acc, lane);
      dvr = acc;
      if (gq == 0 && i < ns) a.stat_dvec[row] = i < n ? acc : 0.f;
    }
  }
  // Everything loaded so far is needed before the first tile.  Waiting here,
  // before the first K/V copies are issued, measured faster than letting the
  // first stage waits cover these loads.
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)

  // the group's sorted edge lists, copied by its first wave into the group's
  // LDS slice (16 bytes = two edges per lane and instruction); they are
  // complete for both waves after the first stage's barrier
  const int nch = ev_count(s) / 2;
  u32x2 *evl = (u32x2 *)(dyn + (size_t)grp * ev_wave_bytes(s, CAUSAL));
  u32x2 *evt = evl + ev_count(s);
  if (active && half == 0) {
    for (int c0 = 0; c0 < nch; c0 += 64)
      if (c0 + lane < nch) dma16(rec + rec_evl_off() + 16 * (c0 + lane), lds_addr(evl + 2 * c0));
    if (!CAUSAL)
      for (int c0 = 0; c0 < nch; c0 += 64)
        if (c0 + lane < nch) dma16(rec + rec_evt_off(s) + 16 * (c0 + lane), lds_addr(evt + 2 * c0));
  }

  // ---- the wave's 16 query rows go to ring slots 2 and 3 (free until the
  // first pair has read them) in the swizzled layout of a K tile, so that
  // every copy instruction reads whole rows and the fragment reads are free of
  // bank conflicts (whole rows per instruction keep the address unit's work
  // per byte low; a row per lane would touch 16 rows per instruction)
  constexpr int CPR_Q = D / 8;  // 16-byte chunks per row
  const uint32_t q_lds = lds_addr(&lds.kv[2][0][0]) + wave * 32 * D;
  if (active) {
#pragma unroll
    for (int c0 = 0; c0 < 16 * CPR_Q; c0 += 64) {
      const int row = (c0 + lane) / CPR_Q, ch = (c0 + lane) % CPR_Q;
      const int64_t off = (int64_t)min(r0 + row, n - 1) * (2 * D) + 16 * (ch ^ swz_key_k<D>(row));
      dma16((const char *)Q + off, q_lds + 16 * c0);
    }
  }

  // ---- K/V staging: a tile is 32 rows of D / 8 chunks, 4 D chunks per
  // matrix; wave w copies chunks [w CPW, (w + 1) CPW) with its first CPW
  // lanes.  Keys past the end read row n - 1, whose products get c = 0.
  constexpr int CPR = D / 8;            // chunks per row
  constexpr int CPW = 4 * D / kWaves;   // chunks per wave, stage and matrix (<= 64)
  constexpr int LPS = 2;                // loads per thread per stage (K and V)
  const char *Kb = (const char *)K, *Vb = (const char *)V;
  // the lane's chunk of every stage: row dkey of the tile, 16 bytes at dofs
  // (D = 128: slot dslot holds key (dslot / 4) % 32, chunk 4 (dslot / 128) +
  // (dslot % 4, its pair swapped by bit 2 of the key: piece128))
  const int dslot = wave * CPW + lane;
  const int dkey = D == 128 ? (dslot >> 2) & 31 : dslot / CPR;
  const int dofs = D == 128 ? 16 * (4 * (dslot >> 7) + ((dslot & 3) ^ (((dkey >> 2) & 1) << 1)))
                            : 16 * ((dslot % CPR) ^ swz_key<D>(dkey));
  const uint32_t kv_lds = lds_addr(&lds.kv[0][0][0]) + wave * CPW * 16;
  auto issue_stage = [&](int st, int q) {  // q = st % kRing
    if (lane < CPW) {
      const int64_t off = (int64_t)min(U0 + kTileKeys * st + dkey, n - 1) * (2 * D) + dofs;
      dma16(Kb + off, kv_lds + (uint32_t)(2 * q) * (kTileKeys * D * 2));
      dma16(Vb + off, kv_lds + (uint32_t)(2 * q + 1) * (kTileKeys * D * 2));
    }
  };
  // stages 0 and 1 now; the pair starting at stage st issues st + 2, st + 3
  if (nst > 0) issue_stage(0, 0);
  if (nst > 1) issue_stage(1, 1);

  // ---- running state
  constexpr int NDB = D / 16;  // 16-dim blocks of O^T
  floatx4 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m2 = -INFINITY;  // running max, log2 units
  float lsum = 0.f;      // this lane's share of the row sum
  int base = 0;          // the row's multiplicity just before the current tile
  int lp = 0, tp = 0;    // next unconsumed lead / trail edge
  int pl = 0, pt = 0;    // their positions (wave-uniform)
  int lg_base = -1;      // the count whose log2 is lg
  float lg = 0.f;
  // edge positions read at a wave-uniform index are wave-uniform
  auto pos_at = [&](const u32x2 *ev, int i) { return (int32_t)__builtin_amdgcn_readfirstlane(ev[i][0]); };
  // K operand: key 16 b + qc, chunk 4 c + gq; b = 1 lies khi bytes further
  uint32_t kofs[NC];
  constexpr uint32_t khi = D == 128 ? 16 * 64 : 16 * 2 * D;
#pragma unroll
  for (int c = 0; c < NC; ++c)  // (= piece128(qc, 4 c + gq) at D = 128)
    kofs[c] = D == 128 ? qc * 64 + ((gq ^ (((qc >> 2) & 1) << 1)) << 4) + 2048 * c : swz<D>(qc, 4 * c + gq);
  // transposing operand (v_ds_read_b64_tr_b16): in each 16-lane group gq,
  // lane r names the row (key 4 gq + r / 4, dims 16 db + 4 (r % 4) .. + 3),
  // and lane i receives X[4 gq + e][16 db + i], e = 0..3; keys + 16 lie khi
  // bytes further
  uint32_t vofs[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int dim = 16 * db + 4 * (qc & 3);
    vofs[db] = D == 128 ? piece128(4 * gq + (qc >> 2), dim >> 3) + ((dim & 4) << 1)
                        : swz<D>(4 * gq + (qc >> 2), dim >> 3) + ((dim & 4) << 1);
  }

  // this wave's tiles are the stages [sa, sb)
  const int sa = active ? (U0w - U0) / kTileKeys : 0;
  const int sb = active ? (U1w - U0) / kTileKeys : 0;

  // a5: S^T = K Q^T for the tile of stage st, keys 16 b + 4 gq + r
  floatx4 sacc[2];
  // (the ring slot is a compile-time constant, so that LDS operand offsets
  // become immediates of the reads)
  auto qk_tile = [&](auto slotc) {
    const char *kt = (const char *)lds.kv[decltype(slotc)::value][0];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      u32x4 kr[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) kr[c] = *(const u32x4 *)(kt + kofs[c] + khi * bb);
      sacc[bb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c)
        sacc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[c]), qf[c], sacc[bb], 0, 0, 0);
    }
  };

  // Visits, in order, the edges of a sorted list at positions < jend starting
  // at index ptr (position pp), and advances ptr / pp past them.  Lane l reads
  // edge ptr + l, so up to 64 edges are found with one LDS read and a ballot
  // (the list ends in 16 sentinels at INT32_MAX; reads stay inside it).
  const int ev_last = s + kSentinels - 1;
  auto edges_in_tile = [&](const u32x2 *ev, int &ptr, int &pp, int jend, auto &&visit) {
    while (pp < jend) {
      const u32x2 e = ev[min(ptr + lane, ev_last)];
      const int k = __popcll(__ballot((int32_t)e[0] < jend));  // a prefix of the lanes
      for (int i = 0; i < k; ++i)
        visit((int32_t)__builtin_amdgcn_readlane(e[0], i), __builtin_amdgcn_readlane(e[1], i));
      ptr += k;
      pp = k < 64 ? (int32_t)__builtin_amdgcn_readlane(e[0], k) : pos_at(ev, ptr);
    }
  };

  // a4, a6, a7 for the tile of stage st, whose logits are in sacc
  auto finish_tile = [&](int st, auto slotc) {
    const char *vt = (const char *)lds.kv[decltype(slotc)::value][1];
    const int j0 = U0 + kTileKeys * st;

    // a4: multiplicity c for keys j0 + 16 b + 4 gq + r.
    //  * diagonal tile: the row's bytes of the precomputed table;
    //  * a tile holding sample edges (lower block ends = leads on the left of
    //    the diagonal, upper ends = trails on the right; positions are
    //    wave-uniform): c = base +- sum over edges of w_e(row) [key >= pos_e],
    //    four keys per byte-counter word;
    //  * otherwise c = base for all keys of the tile.
    const int jend = j0 + kTileKeys;
    float cf[8];
    int kind;  // 0: one count for the tile, 1: per-key counts
    if (j0 == rg) {
      // (kept here: hoisted out of the loop, the conversion would wait for
      // the table load, and with it for every K/V copy issued after it)
      uint32_t d0 = dg[0], d1 = dg[1];
      asm volatile("" : "+v"(d0), "+v"(d1));
#pragma unroll
      for (int r = 0; r < 8; ++r) cf[r] = (float)((((r >> 2) ? d1 : d0) >> (8 * (r & 3))) & 0xFFu);
      // the table already counts every edge at or before the tile's end
      edges_in_tile(evl, lp, pl, jend, [](int, uint32_t) {});
      if (!CAUSAL) {
        edges_in_tile(evt, tp, pt, jend, [](int, uint32_t) {});
        base = dlast;
      }
      kind = 1;
    } else if (pl < jend || (!CAUSAL && pt < jend)) {
      // the lane's keys are words gq and gq + 4 of the tile's step rows
      const uint32_t *srow = &lds.step[0][gq];
      uint32_t cw[2] = {(uint32_t)base * 0x01010101u, (uint32_t)base * 0x01010101u};
      // leads: the sample's block of the row starts at pos
      edges_in_tile(evl, lp, pl, jend, [&](int pos, uint32_t W) {
        const uint32_t w = (W >> t32) & 1u;
        const uint32_t *sr = srow + 8 * (pos - j0);
        cw[0] += w * sr[0];
        cw[1] += w * sr[4];
        base += (int)w;
      });
      // trails: the sample's block of the row ends before pos
      if (!CAUSAL)
        edges_in_tile(evt, tp, pt, jend, [&](int pos, uint32_t W) {
          const uint32_t w = (W >> t32) & 1u;
          const uint32_t *sr = srow + 8 * (pos - j0);
          cw[0] -= w * sr[0];
          cw[1] -= w * sr[4];
          base -= (int)w;
        });
#pragma unroll
      for (int r = 0; r < 8; ++r) cf[r] = (float)((cw[r >> 2] >> (8 * (r & 3))) & 0xFFu);
      kind = 1;
    } else {
      cf[0] = (float)base;
      kind = 0;
    }

    // P = c 2^(s log2 e - lse2): the forward's normalised weights (a tile of
    // one count folds log2 c into the exponent, as in the forward)
    float pr[8];
    if (__builtin_amdgcn_readfirstlane(kind) == 0) {
      if (__any(base != lg_base)) {
        lg = __builtin_amdgcn_logf(cf[0]);
        lg_base = base;
      }
      const float bias = lse2r - lg;  // c = 0 gives bias = +inf, P = 0
#pragma unroll
      for (int r = 0; r < 8; ++r) pr[r] = __builtin_amdgcn_exp2f(fmaf(sacc[r >> 2][r & 3], kLog2e, -bias));
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) {  // (c = 0 selects 0: nothing bounds the exponent of an unweighted key)
        const float e2 = __builtin_amdgcn_exp2f(fmaf(sacc[r >> 2][r & 3], kLog2e, -lse2r));
        pr[r] = cf[r] == 0.f ? 0.f : cf[r] * e2;
      }
    }
    // dP^T = V dO^T: the V tile's rows as the A operand (read like K)
    floatx4 dpacc[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      u32x4 vr[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) vr[c] = *(const u32x4 *)(vt + kofs[c] + khi * bb);
      dpacc[bb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c)
        dpacc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vr[c]), dof[c], dpacc[bb], 0, 0, 0);
    }
    // dS = P (dP - D), rounded to bf16 pairs in the layout of P
    u32x4 sw;
#pragma unroll
    for (int r = 0; r < 8; r += 2) {
      const floatx2 sf = {pr[r] * (dpacc[r >> 2][r & 3] - dvr), pr[r + 1] * (dpacc[r >> 2][(r & 3) + 1] - dvr)};
      sw[r >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(sf, bf16x2));
    }
    const bf16x8 dsk = __builtin_bit_cast(bf16x8, sw);
    // dQ^T += K^T dS^T: the K tile through the transposing reads (K and V
    // tiles share one layout)
    const char *kt = (const char *)lds.kv[decltype(slotc)::value][0];
    constexpr int NB = NDB < 4 ? NDB : 4;
#pragma unroll
    for (int d0 = 0; d0 < NDB; d0 += NB) {
      u32x4 kop[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const char *ka = kt + vofs[d0 + j];
        const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t *)ka);
        const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t *)(ka + khi));
        kop[j] = u32x4{__builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1)),
                       __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3)),
                       __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1)),
                       __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3))};
      }
#pragma unroll
      for (int j = 0; j < NB; ++j)
        oacc[d0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kop[j]), dsk, oacc[d0 + j], 0, 0, 0);
    }
  };

  // Two stages per barrier (measured: the barrier, where every wave waits for
  // the slowest, costs more than the shorter look-ahead): the pair starting at
  // stage st waits for stages st, st + 1, then refills the ring slots of
  // stages st - 2, st - 1 (consumed by every wave before the barrier) with
  // stages st + 2, st + 3, and computes its two tiles.
  auto pair = [&](int st, auto s0, auto s1) {
    PLSH_WAIT_VM_LGKM0(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (st == 0) {
      // the Q fragment from the wave's staged rows, then a barrier: every wave
      // has its fragment before slots 2, 3 take stages 2, 3
      const char *qt = (const char *)lds.kv[2][0] + wave * 32 * D;
#pragma unroll
      for (int c = 0; c < NC; ++c) qf[c] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qt + swz_k<D>(qc, 4 * c + gq)));
      PLSH_WAIT_VM_LGKM0(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    if (st + 2 < nst) issue_stage(st + 2, (decltype(s0)::value + 2) % kRing);
    if (st + 3 < nst) issue_stage(st + 3, (decltype(s1)::value + 2) % kRing);
    if (st == 0 && active) {  // the edge lists landed with stage 0
      pl = pos_at(evl, 0);
      if (!CAUSAL) pt = pos_at(evt, 0);
    }
    if (st >= sa && st < sb) {
      qk_tile(s0);
      finish_tile(st, s0);
    }
    if (st + 1 < nst && st + 1 >= sa && st + 1 < sb) {
      qk_tile(s1);
      finish_tile(st + 1, s1);
    }
  };
  for (int st0 = 0; st0 < nst; st0 += kRing) {
    pair(st0, SlotC<0>{}, SlotC<1>{});
    if (st0 + 2 < nst) pair(st0 + 2, SlotC<2>{}, SlotC<3>{});
  }

  // a8: normalisation epilogue, one store per output element; the row sum
  // is spread over the four lanes qc + 16 gq
  // The wave's 16 x D output block is staged in LDS (in the two ring slots
  // the last pair does not use: every wave is past them), then written whole
  // rows per instruction.
  // dQ (accumulated in oacc) to a.out, staged like the forward's output
  if (!active) return;
  const float inv = 1.0f;
  const int free_slot = (((nst - 1) >> 1) & 1) ? 0 : 2;
  char *ob = (char *)lds.kv[free_slot][0] + wave * 32 * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const bf16x2 h0 = __builtin_convertvector((floatx2{oacc[db][0] * inv, oacc[db][1] * inv}), bf16x2);
    const bf16x2 h1 = __builtin_convertvector((floatx2{oacc[db][2] * inv, oacc[db][3] * inv}), bf16x2);
    // row qc, dims 16 db + 4 gq .. + 3: half (gq & 1) of 16-byte chunk 2 db + gq / 2
    *(u32x2 *)(ob + swz<D>(qc, 2 * db + (gq >> 1)) + 8 * (gq & 1)) =
        u32x2{__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1)};
  }
#pragma unroll
  for (int c0 = 0; c0 < 16 * CPR_Q; c0 += 64) {
    const int row = (c0 + lane) / CPR_Q, ch = (c0 + lane) % CPR_Q;
    const u32x4 val = *(const u32x4 *)(ob + swz<D>(row, ch));
    const int i = r0 + row;
    if (i < n) *(u32x4 *)(O + (int64_t)i * D + 8 * ch) = val;
  }
}

// ---------------------------------------------------------------------------
// Exact ALiBi attention (the dense comparator; Problem Statement, Methodology
// §1):  O_i = sum_j exp(q_i.k_j - |i - j| / sigma_h) v_j / sum_j exp(...),
// j <= i when causal.  The same machinery as the sample-fused kernel -- 128
// query rows per workgroup in 16-row waves, K/V through the LDS ring two
// 32-key stages per barrier, Q and O through free ring slots, MFMA for QK^T
// and PV, log2-domain online softmax with a lazily raised max -- with the
// multiplicity replaced by the bias, added to the logit in the exponent.
// Every key of [0, n) (causal: [0, i]) is visited: O(n^2) work.
// ---------------------------------------------------------------------------
struct ExactArgs {
  const void *q;
  const void *k;
  const void *v;
  void *out;
  int32_t batch, n, heads, kv_heads;
  int32_t groups;                 // query-row tiles per (batch, head)
  float slope2[kMaxHeadsArg];     // log2(e) / sigma_h
};

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kWaves, 64 * kWaves), amdgpu_waves_per_eu(4, 4)))
void exact_mfma_kernel(ExactArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t kv[kRing][2][kTileKeys * D];
  const int n = a.n;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int qc = lane & 15, gq = lane >> 4;

  // ---- workgroup -> (batch, head, row tile).  Causal: the tiles with the
  // most keys (largest row index) first.  Consecutive workgroups take
  // consecutive (batch, head) pairs, so each XCD (workgroups are dealt
  // round-robin) keeps a fixed subset of heads and their K/V in its L2.
  const int BH = a.batch * a.heads;
  const int p = blockIdx.x;
  const int bh = p % BH;
  const int g = CAUSAL ? a.groups - 1 - p / BH : p / BH;
  const int b = bh / a.heads, h = bh % a.heads;
  const int kvh = h / (a.heads / a.kv_heads);
  const int r0 = g * 128 + 16 * wave;  // this wave's first row
  const bool active = r0 < n;
  const float slope2 = a.slope2[h];

  const uint16_t *Q = (const uint16_t *)a.q + ((int64_t)b * a.heads + h) * n * D;
  const char *Kb = (const char *)((const uint16_t *)a.k + ((int64_t)b * a.kv_heads + kvh) * n * D);
  const char *Vb = (const char *)((const uint16_t *)a.v + ((int64_t)b * a.kv_heads + kvh) * n * D);
  uint16_t *O = (uint16_t *)a.out + ((int64_t)b * a.heads + h) * n * D;

  // keys [0, U1) for the workgroup; this wave's tiles are stages [0, sb)
  const int U1 = CAUSAL ? min(n, g * 128 + 128) : n;
  const int nst = (U1 + kTileKeys - 1) / kTileKeys;
  const int sb = !active ? 0 : CAUSAL ? min(r0 + 15, n - 1) / kTileKeys + 1 : nst;

  // ---- Q rows of the wave into ring slots 2, 3 (K-tile swizzle, whole rows
  // per copy instruction), read back after the first wait
  constexpr int NC = D / 32;
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  bf16x8 qf[NC];
  const uint32_t q_lds = lds_addr(&kv[2][0][0]) + wave * 32 * D;
  if (active) {
#pragma unroll
    for (int c0 = 0; c0 < 16 * CPR; c0 += 64) {
      const int row = (c0 + lane) / CPR, ch = (c0 + lane) % CPR;
      const int64_t off = (int64_t)min(r0 + row, n - 1) * (2 * D) + 16 * (ch ^ swz_key<D>(row));
      dma16((const char *)Q + off, q_lds + 16 * c0);
    }
  }

  // ---- K/V staging, as in the sample-fused kernel (keys past the end read
  // row n - 1 and are masked)
  constexpr int CPW = 4 * D / kWaves;
  const int dslot = wave * CPW + lane;
  const int dkey = dslot / CPR;
  const int dofs = 16 * ((dslot % CPR) ^ swz_key<D>(dkey));
  const uint32_t kv_lds = lds_addr(&kv[0][0][0]) + wave * CPW * 16;
  auto issue_stage = [&](int st, int q) {
    if (lane < CPW) {
      const int64_t off = (int64_t)min(kTileKeys * st + dkey, n - 1) * (2 * D) + dofs;
      dma16(Kb + off, kv_lds + (uint32_t)(2 * q) * (kTileKeys * D * 2));
      dma16(Vb + off, kv_lds + (uint32_t)(2 * q + 1) * (kTileKeys * D * 2));
    }
  };
  if (nst > 0) issue_stage(0, 0);
  if (nst > 1) issue_stage(1, 1);

  constexpr int NDB = D / 16;
  floatx4 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m2 = -INFINITY;  // running max, log2 units
  float lsum = 0.f;      // this lane's share of the row sum
  const int i = r0 + qc;  // the lane's query row
  // key offsets of the lane's accumulator entries within a tile
  float koff[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) koff[r] = (float)(16 * (r >> 2) + 4 * gq + (r & 3));
  uint32_t kofs[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) kofs[c] = swz<D>(qc, 4 * c + gq);
  uint32_t vofs[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int dim = 16 * db + 4 * (qc & 3);
    vofs[db] = swz<D>(4 * gq + (qc >> 2), dim >> 3) + ((dim & 4) << 1);
  }

  floatx4 sacc[2];
  auto qk_tile = [&](auto slotc) {
    const char *kt = (const char *)kv[decltype(slotc)::value][0];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      u32x4 kr[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) kr[c] = *(const u32x4 *)(kt + kofs[c] + 32 * D * bb);
      sacc[bb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c)
        sacc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[c]), qf[c], sacc[bb], 0, 0, 0);
    }
  };

  // softmax and PV of the tile of stage st, logits in sacc
  auto finish_tile = [&](int st, auto slotc) {
    const char *vt = (const char *)kv[decltype(slotc)::value][1];
    const int j0 = kTileKeys * st;
    // x = q.k log2(e) - |i - j| log2(e) / sigma, -inf for keys after the row
    // (causal) or past the end
    float x[8];
    const float d0 = (float)(j0 - i);
#pragma unroll
    for (int r = 0; r < 8; ++r) x[r] = fmaf(sacc[r >> 2][r & 3], kLog2e, -fabsf(d0 + koff[r]) * slope2);
    if ((CAUSAL && j0 + kTileKeys - 1 > r0) || j0 + kTileKeys > n) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int j = j0 + 16 * (r >> 2) + 4 * gq + (r & 3);
        if ((CAUSAL && j > i) || j >= n) x[r] = -INFINITY;
      }
    }
    auto mx2 = [](float u, float w) { return max3f(u, w, w); };
    float mx = max3f(max3f(x[0], x[1], x[2]), max3f(x[3], x[4], x[5]), max3f(x[6], x[7], x[7]));
    if (__any(mx > m2 + 8.0f)) {
      mx = mx2(mx, xor16_f(mx));
      mx = mx2(mx, other_half_f(mx, lane));
      const bool need = mx > m2 + 8.0f;
      const float mnew = need ? mx : m2;
      const float alpha = need ? __builtin_amdgcn_exp2f(m2 - mnew) : 1.0f;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      m2 = mnew;
    }
    u32x4 pw;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int r = 0; r < 8; r += 2) {
      const floatx2 pf = {__builtin_amdgcn_exp2f(x[r] - m2), __builtin_amdgcn_exp2f(x[r + 1] - m2)};
      const bf16x2 pb = __builtin_convertvector(pf, bf16x2);
      pw[r >> 1] = __builtin_bit_cast(uint32_t, pb);
      lsum = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, lsum, false);
    }
    const bf16x8 pk = __builtin_bit_cast(bf16x8, pw);
    constexpr int NB = NDB < 4 ? NDB : 4;
#pragma unroll
    for (int e0 = 0; e0 < NDB; e0 += NB) {
      u32x4 vop[NB];
#pragma unroll
      for (int jj = 0; jj < NB; ++jj) {
        const char *va = vt + vofs[e0 + jj];
        const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t *)va);
        const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t *)(va + 16 * 2 * D));
        vop[jj] = u32x4{__builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1)),
                        __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3)),
                        __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1)),
                        __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3))};
      }
#pragma unroll
      for (int jj = 0; jj < NB; ++jj)
        oacc[e0 + jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vop[jj]), pk, oacc[e0 + jj], 0, 0, 0);
    }
  };

  // two stages per barrier; the first pair also takes the Q fragment and
  // frees slots 2, 3 with a second barrier
  auto pair = [&](int st, auto s0, auto s1) {
    PLSH_WAIT_VM_LGKM0(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (st == 0) {
      const char *qt = (const char *)kv[2][0] + wave * 32 * D;
#pragma unroll
      for (int c = 0; c < NC; ++c) qf[c] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qt + swz<D>(qc, 4 * c + gq)));
      PLSH_WAIT_VM_LGKM0(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    if (st + 2 < nst) issue_stage(st + 2, (decltype(s0)::value + 2) % kRing);
    if (st + 3 < nst) issue_stage(st + 3, (decltype(s1)::value + 2) % kRing);
    if (st < sb) {
      qk_tile(s0);
      finish_tile(st, s0);
    }
    if (st + 1 < sb) {
      qk_tile(s1);
      finish_tile(st + 1, s1);
    }
  };
  for (int st0 = 0; st0 < nst; st0 += kRing) {
    pair(st0, SlotC<0>{}, SlotC<1>{});
    if (st0 + 2 < nst) pair(st0 + 2, SlotC<2>{}, SlotC<3>{});
  }

  // output through the two ring slots the last pair does not use
  if (!active) return;
  float ltot = lsum + xor16_f(lsum);
  ltot += other_half_f(ltot, lane);
  const float inv = 1.0f / ltot;
  const int free_slot = (((nst - 1) >> 1) & 1) ? 0 : 2;
  char *ob = (char *)kv[free_slot][0] + wave * 32 * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const bf16x2 h0 = __builtin_convertvector((floatx2{oacc[db][0] * inv, oacc[db][1] * inv}), bf16x2);
    const bf16x2 h1 = __builtin_convertvector((floatx2{oacc[db][2] * inv, oacc[db][3] * inv}), bf16x2);
    *(u32x2 *)(ob + swz<D>(qc, 2 * db + (gq >> 1)) + 8 * (gq & 1)) =
        u32x2{__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1)};
  }
#pragma unroll
  for (int c0 = 0; c0 < 16 * CPR; c0 += 64) {
    const int row = (c0 + lane) / CPR, ch = (c0 + lane) % CPR;
    const u32x4 val = *(const u32x4 *)(ob + swz<D>(row, ch));
    const int io = r0 + row;
    if (io < n) *(u32x4 *)(O + (int64_t)io * D + 8 * ch) = val;
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp combine of per-sample partials (the unfused form of
// Methodology §3: s short attentions, each normalised on its own, recombined
// into the one ratio of sums):
//   out_i = sum_k e^{lse_k,i} O_k,i / sum_k e^{lse_k,i}
// o32 [s][rows][D] and lse [s][rows] fp32; one wave per row, lane l holds
// dims l, l + 64.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const float *o32, const float *lse, int s, int64_t rows,
                                                      uint16_t *out) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  constexpr int E = D / 64;
  float mx = -INFINITY;
  for (int k = 0; k < s; ++k) mx = fmaxf(mx, lse[(int64_t)k * rows + row]);
  float acc[E], den = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int k = 0; k < s; ++k) {
    const float wk = expf(lse[(int64_t)k * rows + row] - mx);
    den += wk;
    const float *ok = o32 + ((int64_t)k * rows + row) * D;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(wk, ok[lane + 64 * e], acc[e]);
  }
  const float inv = 1.0f / den;
#pragma unroll
  for (int e = 0; e < E; ++e) out[row * D + lane + 64 * e] = (uint16_t)f32_to_bf16_bits(acc[e] * inv);
}

// ---------------------------------------------------------------------------
// Backward, dK and dV.  The same-bin count is symmetric (i and j share a
// block of hash k exactly when j and i do), so the roles of rows and keys can
// be swapped: a workgroup owns 128 key positions of one KV head, each wave
// 16 of them, and streams 32-row tiles of Q and dO (and those rows' lse2 and
// D) through the ring, with the multiplicities of its key positions taken
// from the non-causal records of their 32-position groups.  Causal: rows
// i >= j only (each wave starts at its group's diagonal tile, masked below
// the diagonal).  Per tile:
//   S^T = Q K^T,  P = c 2^(S log2 e - lse2_i),  dV^T += dO^T P,
//   dP^T = dO V^T,  dS = P o (dP - D_i),  dK^T += Q^T dS  (MFMA),
// for every query head of the workgroup's GQA group in turn, so the group's
// sum stays in registers.
// ---------------------------------------------------------------------------
template <int D>
struct BwdLds {
  alignas(16) uint16_t kv[kRing][2][kTileKeys * D];  // [0]: Q rows, [1]: dO rows of a stage
  uint32_t step[kTileKeys][kTileKeys / 4];
  alignas(16) float rs[kRing][2 * kTileKeys];         // the stage rows' lse2 [0, 32) and D [32, 64)
};

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kWaves, 64 * kWaves), amdgpu_waves_per_eu(2, 2)))
void attn_dkv_kernel(AttnArgs a, const uint8_t *ws, uint16_t *dk_out, uint16_t *dv_out) {
  using L = BwdLds<D>;
  __shared__ __attribute__((aligned(16))) L lds;
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  const int s = a.s, n = a.n;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int qc = lane & 15, gq = lane >> 4;
  if (threadIdx.x < kTileKeys * kTileKeys / 4) {
    const int u = threadIdx.x >> 3, k = threadIdx.x & 7;
    lds.step[u][k] = step4(u - 4 * k);
  }

  // ---- workgroup -> (batch, kv head, 128-position tile), the XCD-aware map
  // of the forward
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
  const int kvh = a.order[unit / a.batch];  // KV heads here, heaviest group first
  const int b = unit % a.batch;
  const int grpsz = a.heads / a.kv_heads;
  const int grp = wave >> 1, half = wave & 1;
  const int rg = g * 128 + 32 * grp;  // the group's first position
  const int r0 = rg + 16 * half;      // this wave's first key position
  const bool active = r0 < n;
  const int t32 = 16 * half + qc;     // the lane's key within its group
  const int g32 = (n + 31) / 32;
  const size_t rb = rec_bytes(s);
  constexpr int NC = D / 32, NDB = D / 16, CPR = D / 8, CPW = 4 * D / kWaves;

  // K and V fragments of the wave's keys (B operands, laid out as the
  // forward's Q fragment)
  bf16x8 kf[NC], vf[NC];
  {
    const uint16_t *Kh = (const uint16_t *)a.k + ((int64_t)b * a.kv_heads + kvh) * n * D;
    const uint16_t *Vh = (const uint16_t *)a.v + ((int64_t)b * a.kv_heads + kvh) * n * D;
    const int j = r0 + qc;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 rk = {0u, 0u, 0u, 0u}, rv = {0u, 0u, 0u, 0u};
      if (active && j < n) {
        rk = *(const u32x4 *)(Kh + (int64_t)j * D + 32 * c + 8 * gq);
        rv = *(const u32x4 *)(Vh + (int64_t)j * D + 32 * c + 8 * gq);
      }
      kf[c] = __builtin_bit_cast(bf16x8, rk);
      vf[c] = __builtin_bit_cast(bf16x8, rv);
    }
  }
  // tile operands (Q and dO tiles, D = 128: the piece layout of piece128,
  // whose rows + 16 lie khi bytes further): 16-byte reads at kofs, the
  // transposing reads at vofs
  uint32_t kofs[NC];
  constexpr uint32_t khi = D == 128 ? 16 * 64 : 16 * 2 * D;
#pragma unroll
  for (int c = 0; c < NC; ++c)  // (= piece128(qc, 4 c + gq) at D = 128)
    kofs[c] = D == 128 ? qc * 64 + ((gq ^ (((qc >> 2) & 1) << 1)) << 4) + 2048 * c : swz<D>(qc, 4 * c + gq);
  uint32_t vofs[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int dim = 16 * db + 4 * (qc & 3);
    vofs[db] = D == 128 ? piece128(4 * gq + (qc >> 2), dim >> 3) + ((dim & 4) << 1)
                        : swz<D>(4 * gq + (qc >> 2), dim >> 3) + ((dim & 4) << 1);
  }
  floatx4 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dkacc[db] = dvacc[db] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nch = ev_count(s) / 2;
  u32x2 *evl = (u32x2 *)(dyn + (size_t)grp * ev_wave_bytes(s, false));
  u32x2 *evt = evl + ev_count(s);
  const int dslot = wave * CPW + lane;
  // (D = 128: slot dslot holds row (dslot / 4) % 32, chunk 4 (dslot / 128) +
  // (dslot % 4, its pair swapped by bit 2 of the row: piece128))
  const int dkey = D == 128 ? (dslot >> 2) & 31 : dslot / CPR;
  const int dofs = D == 128 ? 16 * (4 * (dslot >> 7) + ((dslot & 3) ^ (((dkey >> 2) & 1) << 1)))
                            : 16 * ((dslot % CPR) ^ swz_key<D>(dkey));
  const uint32_t kv_lds = lds_addr(&lds.kv[0][0][0]) + wave * CPW * 16;
  const uint32_t rs_lds = lds_addr(&lds.rs[0][0]);
  auto pos_at = [&](const u32x2 *ev, int i) { return (int32_t)__builtin_amdgcn_readfirstlane(ev[i][0]); };
  const int ev_last = s + kSentinels - 1;
  auto edges_in_tile = [&](const u32x2 *ev, int &ptr, int &pp, int jend, auto &&visit) {
    while (pp < jend) {
      const u32x2 e = ev[min(ptr + lane, ev_last)];
      const int k = __popcll(__ballot((int32_t)e[0] < jend));
      for (int i = 0; i < k; ++i)
        visit((int32_t)__builtin_amdgcn_readlane(e[0], i), __builtin_amdgcn_readlane(e[1], i));
      ptr += k;
      pp = k < 64 ? (int32_t)__builtin_amdgcn_readlane(e[0], k) : pos_at(ev, ptr);
    }
  };

  int nst = 0;
  for (int hi = 0; hi < grpsz; ++hi) {
    const int h = kvh * grpsz + hi;
    const int64_t rowbase = ((int64_t)b * a.heads + h) * n;
    const int64_t statbase = ((int64_t)b * a.heads + h) * ((n + 31) & ~31);  // rows padded to 32
    const char *Qb = (const char *)((const uint16_t *)a.q + rowbase * D);
    const char *dOb = (const char *)((const uint16_t *)a.dout + rowbase * D);
    const uint8_t *rec_wg = ws + ((size_t)h * g32 + 4 * g) * rb;
    const uint8_t *rec = rec_wg + (size_t)grp * rb;
    int U0 = INT32_MAX, U1 = INT32_MIN, U0w = 0, U1w = 0;
    {
      const int wlast = min(3, (n - 1 - g * 128) / 32);
      int4 hdr[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) hdr[w] = *(const int4 *)(rec_wg + (size_t)min(w, wlast) * rb);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        U0 = min(U0, hdr[w].y);
        U1 = max(U1, hdr[w].z);
        if (w == grp) { U0w = hdr[w].y; U1w = hdr[w].z; }
      }
    }
    // rows i >= j (causal): nothing before the workgroup's first position
    if (CAUSAL) U0 = max(U0, g * 128);
    uint32_t dg[2] = {0u, 0u};
    int dlast = 0;
    if (active) {
      const uint8_t *drow = rec + rec_diag_off(s) + 32 * t32;
      dg[0] = *(const uint32_t *)(drow + 4 * gq);
      dg[1] = *(const uint32_t *)(drow + 16 + 4 * gq);
      dlast = (int)(*(const uint32_t *)(drow + 28) >> 24);
    }
    nst = (U1 > U0) ? (U1 - U0) / kTileKeys : 0;
    const int sa = active ? ((CAUSAL ? rg : U0w) - U0) / kTileKeys : 0;
    const int sb = active ? (U1w - U0) / kTileKeys : 0;
    // the previous head's tiles are done in every wave before its edge lists
    // and ring slots are refilled
    PLSH_WAIT_VM_LGKM0(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (active && half == 0) {
      for (int c0 = 0; c0 < nch; c0 += 64)
        if (c0 + lane < nch) dma16(rec + rec_evl_off() + 16 * (c0 + lane), lds_addr(evl + 2 * c0));
      for (int c0 = 0; c0 < nch; c0 += 64)
        if (c0 + lane < nch) dma16(rec + rec_evt_off(s) + 16 * (c0 + lane), lds_addr(evt + 2 * c0));
    }
    auto issue_stage = [&](int st, int q) {
      const int i0 = U0 + kTileKeys * st;
      if (lane < CPW) {
        const int64_t off = (int64_t)min(i0 + dkey, n - 1) * (2 * D) + dofs;
        dma16(Qb + off, kv_lds + (uint32_t)(2 * q) * (kTileKeys * D * 2));
        dma16(dOb + off, kv_lds + (uint32_t)(2 * q + 1) * (kTileKeys * D * 2));
      }
      // the rows' lse2 and D (a head's statistics are padded with zeros to a
      // multiple of 32 rows, which every stage lies within)
      if (wave == 0 && lane < 16) {
        const float *src = (lane < 8 ? a.lse2 : a.dvec) + statbase + i0 + 4 * (lane & 7);
        dma16(src, rs_lds + (uint32_t)q * (2 * kTileKeys * 4));
      }
    };
    if (nst > 0) issue_stage(0, 0);
    if (nst > 1) issue_stage(1, 1);
    int base = 0, lp = 0, tp = 0, pl = 0, pt = 0, lg_base = -1;
    float lg = 0.f;

    floatx4 sacc[2];
    auto s_tile = [&](auto slotc) {  // S^T = Q K^T: rows 16 b + 4 gq + r of the tile
      const char *qt = (const char *)lds.kv[decltype(slotc)::value][0];
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        u32x4 qr[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) qr[c] = *(const u32x4 *)(qt + kofs[c] + khi * bb);
        sacc[bb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c)
          sacc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qr[c]), kf[c], sacc[bb], 0, 0, 0);
      }
    };
    // A^T (D x 32 rows) B accumulated into acc, A a tile of the ring read
    // through the transposing reads
    auto tr_mfma = [&](const char *tile, const bf16x8 &bop, floatx4 *acc) {
      constexpr int NB = NDB < 4 ? NDB : 4;
#pragma unroll
      for (int d0 = 0; d0 < NDB; d0 += NB) {
        u32x4 op[NB];
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) {
          const char *ta = tile + vofs[d0 + jj];
          const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t *)ta);
          const short4_t hi2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t *)(ta + khi));
          op[jj] = u32x4{__builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1)),
                         __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3)),
                         __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi2, hi2, 0, 1)),
                         __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi2, hi2, 2, 3))};
        }
#pragma unroll
        for (int jj = 0; jj < NB; ++jj)
          acc[d0 + jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, op[jj]), bop, acc[d0 + jj], 0, 0, 0);
      }
    };
    auto finish_tile = [&](int st, auto slotc) {
      constexpr int Q = decltype(slotc)::value;
      const char *qt = (const char *)lds.kv[Q][0];
      const char *dot = (const char *)lds.kv[Q][1];
      const int j0 = U0 + kTileKeys * st;  // the tile's first row
      const int jend = j0 + kTileKeys;
      // multiplicities of (key t32, row 16 b + 4 gq + r) from the non-causal
      // record, exactly as the forward's for (row, key)
      float cf[8];
      int kind;
      if (j0 == rg) {
        uint32_t d0 = dg[0], d1 = dg[1];
        asm volatile("" : "+v"(d0), "+v"(d1));
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int u = 16 * (r >> 2) + 4 * gq + (r & 3);
          const float c = (float)((((r >> 2) ? d1 : d0) >> (8 * (r & 3))) & 0xFFu);
          cf[r] = (CAUSAL && u < t32) ? 0.f : c;  // causal: rows i >= j only
        }
        edges_in_tile(evl, lp, pl, jend, [](int, uint32_t) {});
        edges_in_tile(evt, tp, pt, jend, [](int, uint32_t) {});
        base = dlast;
        kind = 1;
      } else if (pl < jend || pt < jend) {
        const uint32_t *srow = &lds.step[0][gq];
        uint32_t cw[2] = {(uint32_t)base * 0x01010101u, (uint32_t)base * 0x01010101u};
        edges_in_tile(evl, lp, pl, jend, [&](int pos, uint32_t W) {
          const uint32_t w = (W >> t32) & 1u;
          const uint32_t *sr = srow + 8 * (pos - j0);
          cw[0] += w * sr[0];
          cw[1] += w * sr[4];
          base += (int)w;
        });
        edges_in_tile(evt, tp, pt, jend, [&](int pos, uint32_t W) {
          const uint32_t w = (W >> t32) & 1u;
          const uint32_t *sr = srow + 8 * (pos - j0);
          cw[0] -= w * sr[0];
          cw[1] -= w * sr[4];
          base -= (int)w;
        });
#pragma unroll
        for (int r = 0; r < 8; ++r) cf[r] = (float)((cw[r >> 2] >> (8 * (r & 3))) & 0xFFu);
        kind = 1;
      } else {
        cf[0] = (float)base;
        kind = 0;
      }
      // the rows' lse2 and D
      const float *rsq = lds.rs[Q];
      const floatx4 la = *(const floatx4 *)(rsq + 4 * gq), lb = *(const floatx4 *)(rsq + 16 + 4 * gq);
      const floatx4 da = *(const floatx4 *)(rsq + 32 + 4 * gq), dbv = *(const floatx4 *)(rsq + 48 + 4 * gq);
      float pr[8];
      if (__builtin_amdgcn_readfirstlane(kind) == 0) {
        if (__any(base != lg_base)) {
          lg = __builtin_amdgcn_logf(cf[0]);
          lg_base = base;
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float l2 = (r >> 2) ? lb[r & 3] : la[r & 3];
          pr[r] = __builtin_amdgcn_exp2f(fmaf(sacc[r >> 2][r & 3], kLog2e, lg - l2));  // c = 0: lg = -inf
        }
      } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float l2 = (r >> 2) ? lb[r & 3] : la[r & 3];
          const float e2 = __builtin_amdgcn_exp2f(fmaf(sacc[r >> 2][r & 3], kLog2e, -l2));
          pr[r] = cf[r] == 0.f ? 0.f : cf[r] * e2;
        }
      }
      u32x4 pw;
#pragma unroll
      for (int r = 0; r < 8; r += 2)
        pw[r >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2{pr[r], pr[r + 1]}), bf16x2));
      // dV^T += dO^T P
      tr_mfma(dot, __builtin_bit_cast(bf16x8, pw), dvacc);
      // dP^T = dO V^T (dO rows as the A operand)
      floatx4 dpacc[2];
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        u32x4 orr[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) orr[c] = *(const u32x4 *)(dot + kofs[c] + khi * bb);
        dpacc[bb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c)
          dpacc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, orr[c]), vf[c], dpacc[bb], 0, 0, 0);
      }
      // dS = P (dP - D), then dK^T += Q^T dS
      u32x4 sw;
#pragma unroll
      for (int r = 0; r < 8; r += 2) {
        const float dA = (r >> 2) ? dbv[r & 3] : da[r & 3];
        const float dB = (r >> 2) ? dbv[(r & 3) + 1] : da[(r & 3) + 1];
        const floatx2 sf = {pr[r] * (dpacc[r >> 2][r & 3] - dA), pr[r + 1] * (dpacc[r >> 2][(r & 3) + 1] - dB)};
        sw[r >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(sf, bf16x2));
      }
      tr_mfma(qt, __builtin_bit_cast(bf16x8, sw), dkacc);
    };
    auto pair = [&](int st, auto s0, auto s1) {
      PLSH_WAIT_VM_LGKM0(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (st + 2 < nst) issue_stage(st + 2, (decltype(s0)::value + 2) % kRing);
      if (st + 3 < nst) issue_stage(st + 3, (decltype(s1)::value + 2) % kRing);
      if (st == 0 && active) {
        pl = pos_at(evl, 0);
        pt = pos_at(evt, 0);
      }
      if (st >= sa && st < sb) {
        s_tile(s0);
        finish_tile(st, s0);
      }
      if (st + 1 < nst && st + 1 >= sa && st + 1 < sb) {
        s_tile(s1);
        finish_tile(st + 1, s1);
      }
    };
    for (int st0 = 0; st0 < nst; st0 += kRing) {
      pair(st0, SlotC<0>{}, SlotC<1>{});
      if (st0 + 2 < nst) pair(st0 + 2, SlotC<2>{}, SlotC<3>{});
    }
  }

  // dK, dV of the wave's 16 keys through the two ring slots the last pair
  // does not use (whole rows per store instruction)
  if (!active) return;
  const int free_slot = (((nst - 1) >> 1) & 1) ? 0 : 2;
  char *ob = (char *)lds.kv[free_slot][0] + wave * 32 * D;
  const int64_t kvrow = ((int64_t)b * a.kv_heads + kvh) * n;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const floatx4 *acc = which ? dvacc : dkacc;
    uint16_t *outp = (which ? dv_out : dk_out) + kvrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const bf16x2 h0 = __builtin_convertvector((floatx2{acc[db][0], acc[db][1]}), bf16x2);
      const bf16x2 h1 = __builtin_convertvector((floatx2{acc[db][2], acc[db][3]}), bf16x2);
      *(u32x2 *)(ob + swz<D>(qc, 2 * db + (gq >> 1)) + 8 * (gq & 1)) =
          u32x2{__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1)};
    }
#pragma unroll
    for (int c0 = 0; c0 < 16 * CPR; c0 += 64) {
      const int row = (c0 + lane) / CPR, ch = (c0 + lane) % CPR;
      const u32x4 val = *(const u32x4 *)(ob + swz<D>(row, ch));
      const int io = r0 + row;
      if (io < n) *(u32x4 *)(outp + (int64_t)io * D + 8 * ch) = val;
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
  a.pstride = s;
  a.o32 = nullptr;
  a.lse = nullptr;
  a.dout = nullptr;
  a.lse2 = nullptr;
  a.dvec = nullptr;
  a.stat_lse2 = nullptr;
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

// the event pair for the next timed launch, or nullptr when timing is off
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

// kernel launch, stamping the timer's events when tm is set
template <typename... Args, typename... P>
void launch_k(void (*kern)(Args...), dim3 grid, dim3 block, size_t shm, hipStream_t st,
              std::pair<hipEvent_t, hipEvent_t> *tm, P... p) {
  if (tm) hipExtLaunchKernelGGL(kern, grid, block, (uint32_t)shm, st, tm->first, tm->second, 0u, p...);
  else hipLaunchKernelGGL(kern, grid, block, shm, st, p...);
}

plsh_status launch_valu(const dev::AttnArgs &a, int d, plsh_dtype dtype, int causal, hipStream_t st,
                        const char *who) {
  const size_t shm = 4 * dev::valu_wave_bytes(a.s, d);
  // rows per wave: fewer for small problems, so that their rows spread over
  // the GPU's 256 compute units instead of running in sequence in few waves
  const int64_t groups = (int64_t)((a.n + 31) / 32) * a.batch * a.heads;
  const int rpw = groups <= 64 ? 1 : groups <= 256 ? 2 : groups <= 1024 ? 4 : 8;
  const dim3 grid((unsigned)(groups * (8 / rpw))), block(256);
  auto *tm = timer_slot();
  if (dtype == PLSH_F32) {
    if (d == 64) launch_k(dev::attn_valu_kernel<float, 64>, grid, block, shm, st, tm, a, causal, rpw);
    else launch_k(dev::attn_valu_kernel<float, 128>, grid, block, shm, st, tm, a, causal, rpw);
  } else {
    if (d == 64) launch_k(dev::attn_valu_kernel<uint16_t, 64>, grid, block, shm, st, tm, a, causal, rpw);
    else launch_k(dev::attn_valu_kernel<uint16_t, 128>, grid, block, shm, st, tm, a, causal, rpw);
  }
  return launch_check(who);
}

// bytes of the block-edge records of every (head, 32-row group)
size_t records_bytes(int n, int heads, int s) { return (size_t)heads * ((n + 31) / 32) * dev::rec_bytes(s); }

// The block-edge records of every (head, 32-row group), causal or not, into
// ws (records_bytes(a.n, a.heads, a.s) bytes, 16-byte aligned).
// (non-causal with ws_causal set: both record sets in one pass)
plsh_status launch_edges(const dev::AttnArgs &a, bool causal, hipStream_t st, const char *who, void *ws,
                         void *ws_causal = nullptr) {
  const int g32 = (a.n + 31) / 32;
  const int items = a.heads * g32;
  const dim3 egrid((unsigned)((items + 3) / 4)), eblock(256);
  const size_t eshm = 4 * (dev::wavetab_bytes(a.s) + 32 * 16 * 4);
  if (causal) hipLaunchKernelGGL(dev::edges_kernel<true>, egrid, eblock, eshm, st, a.params, a.pstride, a.n, a.heads, a.s, g32, (uint8_t *)ws, (uint8_t *)nullptr);
  else hipLaunchKernelGGL(dev::edges_kernel<false>, egrid, eblock, eshm, st, a.params, a.pstride, a.n, a.heads, a.s, g32, (uint8_t *)ws, (uint8_t *)ws_causal);
  return launch_check(who);
}

// The records into a workspace from the stream-ordered allocator (released by
// free_records).
plsh_status build_records(const dev::AttnArgs &a, bool causal, hipStream_t st, const char *who, void **ws) {
  const size_t ws_bytes = records_bytes(a.n, a.heads, a.s);
  *ws = nullptr;
  hipError_t e = hipMallocAsync(ws, ws_bytes, st);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    *ws = nullptr;
    return fail(PLSH_ERR_HIP, "%s: workspace allocation of %zu bytes failed: %s", who, ws_bytes,
                hipGetErrorString(e));
  }
  return launch_edges(a, causal, st, who, *ws);
}

// Causal and non-causal records in one pre-pass (the causal backward's two
// record sets), each in its own workspace from the stream-ordered allocator.
plsh_status build_record_pair(const dev::AttnArgs &a, hipStream_t st, const char *who, void **ws_causal,
                              void **ws_nc) {
  const size_t ws_bytes = records_bytes(a.n, a.heads, a.s);
  *ws_causal = *ws_nc = nullptr;
  for (void **p : {ws_causal, ws_nc}) {
    const hipError_t e = hipMallocAsync(p, ws_bytes, st);
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

// One MFMA kernel over records ws (causal records for modes 0, 1 and 3 of a
// causal call, non-causal ones otherwise).  mode 0: the estimator
// (attn_mfma_kernel); 1: its backward dQ (attn_dq_kernel); 2: its backward
// dK, dV into dk, dv (attn_dkv_kernel); 3: the estimator walking the samples
// one by one over single-sample records (attn_mfma_kernel<.., true>).
plsh_status launch_attn(const dev::AttnArgs &a, int d, int causal, hipStream_t st, const char *who, int mode,
                        const void *ws, void *dk = nullptr, void *dv = nullptr) {
  const int64_t units = mode == 2 ? (int64_t)a.batch * a.kv_heads : (int64_t)a.batch * a.heads;
  const dim3 grid((unsigned)(a.groups * units)), block(64 * dev::kWaves);
  const uint8_t *w8 = (const uint8_t *)ws;
  const size_t shm = 4 * dev::ev_wave_bytes(mode == 3 ? 1 : a.s, causal != 0 && mode != 2);
  auto *tm = timer_slot();
  if (mode == 2) {
    uint16_t *k16 = (uint16_t *)dk, *v16 = (uint16_t *)dv;
    if (d == 64) {
      if (causal) launch_k(dev::attn_dkv_kernel<64, true>, grid, block, shm, st, tm, a, w8, k16, v16);
      else launch_k(dev::attn_dkv_kernel<64, false>, grid, block, shm, st, tm, a, w8, k16, v16);
    } else {
      if (causal) launch_k(dev::attn_dkv_kernel<128, true>, grid, block, shm, st, tm, a, w8, k16, v16);
      else launch_k(dev::attn_dkv_kernel<128, false>, grid, block, shm, st, tm, a, w8, k16, v16);
    }
  } else if (mode == 3) {
    if (d == 64) {
      if (causal) launch_k(dev::attn_mfma_kernel<64, true, true>, grid, block, shm, st, tm, a, w8);
      else launch_k(dev::attn_mfma_kernel<64, false, true>, grid, block, shm, st, tm, a, w8);
    } else {
      if (causal) launch_k(dev::attn_mfma_kernel<128, true, true>, grid, block, shm, st, tm, a, w8);
      else launch_k(dev::attn_mfma_kernel<128, false, true>, grid, block, shm, st, tm, a, w8);
    }
  } else if (mode == 1) {
    if (d == 64) {
      if (causal) launch_k(dev::attn_dq_kernel<64, true>, grid, block, shm, st, tm, a, w8);
      else launch_k(dev::attn_dq_kernel<64, false>, grid, block, shm, st, tm, a, w8);
    } else {
      if (causal) launch_k(dev::attn_dq_kernel<128, true>, grid, block, shm, st, tm, a, w8);
      else launch_k(dev::attn_dq_kernel<128, false>, grid, block, shm, st, tm, a, w8);
    }
  } else if (d == 64) {
    if (causal) launch_k(dev::attn_mfma_kernel<64, true>, grid, block, shm, st, tm, a, w8);
    else launch_k(dev::attn_mfma_kernel<64, false>, grid, block, shm, st, tm, a, w8);
  } else {
    if (causal) launch_k(dev::attn_mfma_kernel<128, true>, grid, block, shm, st, tm, a, w8);
    else launch_k(dev::attn_mfma_kernel<128, false>, grid, block, shm, st, tm, a, w8);
  }
  return launch_check(who);
}

// The estimator: its records, then attn_mfma_kernel.  The records go to the
// caller's workspace when one is given, else to one from the stream-ordered
// allocator.
plsh_status launch_mfma(const dev::AttnArgs &a, const double *sigma, int d, int causal, hipStream_t st,
                        const char *who, void *caller_ws = nullptr) {
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
    plsh_status rc = launch_edges(a, causal != 0, st, who, caller_ws);
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

plsh_status launch_exact(const dev::ExactArgs &a, int d, int causal, hipStream_t st, const char *who) {
  const dim3 grid((unsigned)((int64_t)a.groups * a.batch * a.heads)), block(64 * dev::kWaves);
  auto *tm = timer_slot();
  if (d == 64) {
    if (causal) launch_k(dev::exact_mfma_kernel<64, true>, grid, block, 0, st, tm, a);
    else launch_k(dev::exact_mfma_kernel<64, false>, grid, block, 0, st, tm, a);
  } else {
    if (causal) launch_k(dev::exact_mfma_kernel<128, true>, grid, block, 0, st, tm, a);
    else launch_k(dev::exact_mfma_kernel<128, false>, grid, block, 0, st, tm, a);
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
  const int groups = (bt->n + 31) / 32;
  const size_t shm = dev::wavetab_bytes(bt->s);
  hipLaunchKernelGGL(dev::debug_intervals_kernel, dim3((unsigned)((int64_t)groups * bt->heads)), dim3(64), shm,
                     (hipStream_t)stream, bt->params, bt->n, bt->heads, bt->s, groups, lohi);
  return launch_check(who);
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
  hipError_t e = hipMallocAsync(&ws, bytes, hs);
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
  if (rc == PLSH_OK) {
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    if (d == 64) hipLaunchKernelGGL(dev::combine_kernel<64>, grid, block, 0, hs, o32, lse, s, rows, (uint16_t *)out);
    else hipLaunchKernelGGL(dev::combine_kernel<128>, grid, block, 0, hs, o32, lse, s, rows, (uint16_t *)out);
    rc = launch_check(who);
  }
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

// Gradients of the estimate for fixed tables (see include/plsh.h).
// The backward of the estimate for fixed tables.  With saved_out and
// saved_lse2 (the output and row statistics of plsh_alibi_attention_lse) the
// statistics pass is replaced by D = dO . O from the saved output.
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
  const size_t bytes = (saved ? 1 : 2) * (size_t)prows * sizeof(float);
  void *stats = nullptr;
  hipError_t e = hipMallocAsync(&stats, bytes, hs);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PLSH_ERR_HIP, "%s: statistics allocation of %zu bytes failed: %s", who, bytes, hipGetErrorString(e));
  }
  const float *lse2 = saved ? saved_lse2 : (const float *)stats;
  float *dvec = saved ? (float *)stats : (float *)stats + prows;
  dev::AttnArgs a;
  fill_args(a, q, k, v, dq, batch, n, heads, kv_heads, sigma, s, boundaries);
  a.dout = dout;
  plsh_status rc = PLSH_OK;
  // the records of the estimator serve its statistics pass and dQ; dK/dV
  // takes non-causal ones (the same records when the call is not causal;
  // a causal call gets both sets from one pre-pass)
  void *rec = nullptr, *rec_nc = nullptr;
  if (rc == PLSH_OK) {
    if (causal) rc = build_record_pair(a, hs, who, &rec, &rec_nc);
    else rc = build_records(a, false, hs, who, &rec);
  }
  if (rc == PLSH_OK && !saved) {
    // statistics: each row's normaliser and D = dO . O
    a.stat_lse2 = (float *)stats;
    a.stat_dvec = dvec;
    rc = launch_attn(a, d, causal != 0, hs, who, 0, rec);
  }
  if (rc == PLSH_OK) {
    // dQ; from a saved forward it also forms D = dO . O into dvec
    a.stat_lse2 = nullptr;
    a.stat_dvec = saved ? dvec : nullptr;
    a.saved_out = saved ? saved_out : nullptr;
    a.lse2 = lse2;
    a.dvec = saved ? nullptr : dvec;
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
