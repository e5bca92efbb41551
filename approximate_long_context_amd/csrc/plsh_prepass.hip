// plsh_prepass.hip -- block intervals on the device: the block-edge pre-pass,
// the interval dump and the one-row-per-wave VALU kernel (gfx950).
// Built without contraction of multiply-adds: the bins here must equal the
// host table's bit for bit (plsh_binning.h).
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

#include "plsh_binning.h"
#include "plsh_hip_status.h"
#include "plsh_kernels.h"

namespace plsh {
namespace dev {

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
  // ranks of the edges (ties by sample index): with s <= 32, J = 64 / s lane
  // groups split the comparisons of sample k (lane k + s j takes the samples
  // k2 = j mod J) and add their partial ranks in LDS (the operand records of
  // the mask step are free by now)
  const int J = s <= 32 ? 64 / s : 1;
  int *rk = (int *)w.lst;  // [2][s]: lead ranks, trail ranks
  if (J > 1) {
    for (int i = lane; i < 2 * s; i += 64) rk[i] = 0;
    wave_sync();
    const int k = lane % s, j = lane / s;
    if (j < J) {
      const int32_t lk = w.lead[k], tk = w.trail[k];
      int rl = 0, rt = 0;
      for (int k2 = j; k2 < s; k2 += J) {
        const int32_t l2 = w.lead[k2], t2 = w.trail[k2];
        rl += (l2 < lk) | ((l2 == lk) & (k2 < k));
        rt += (t2 < tk) | ((t2 == tk) & (k2 < k));
      }
      atomicAdd(&rk[k], rl);
      if (!CAUSAL) atomicAdd(&rk[s + k], rt);
    }
    wave_sync();
  }
  int mn = INT32_MAX, mx = INT32_MIN;
  for (int k = lane; k < s; k += 64) {
    const int32_t lk = w.lead[k], tk = w.trail[k];
    const uint32_t mk = w.mask[k];
    mn = min(mn, lk);
    mx = max(mx, tk);
    int rl = 0, rt = 0;
    if (J > 1) {
      rl = rk[k];
      if (!CAUSAL) rt = rk[s + k];
    } else {
#pragma unroll 4
      for (int k2 = 0; k2 < s; ++k2) {
        const int32_t l2 = w.lead[k2], t2 = w.trail[k2];
        rl += (l2 < lk) | ((l2 == lk) & (k2 < k));
        rt += (t2 < tk) | ((t2 == tk) & (k2 < k));
      }
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
  // (the two half-waves take alternate listed samples, every key of the row)
  for (int z = hh; z < nact; z += 2) {
    const uint32_t mk = w.mask[w.act[z]];
    const uint32_t ml = mk & low_t;
    if (ml) {
      const int rel = 31 - __builtin_clz(ml);
      atomicAdd(&hup[rel >> 2], 1u << (8 * (rel & 3)));
    }
    if (!CAUSAL) {
      const uint32_t mh = mk & high_t;
      if (mh) {
        const int rel = __builtin_ctz(mh);
        atomicAdd(&hdn[rel >> 2], 1u << (8 * (rel & 3)));
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
  // keep the bytes of keys u <= lim (u < n; causal: u <= t): byte r of word
  // i is key 16 hh + 4 i + r
  auto keep = [&](int lim, int i) {
    const int e = lim - 16 * hh - 4 * i;  // last kept byte of the word
    return e >= 3 ? 0xFFFFFFFFu : (e < 0 ? 0u : (0xFFFFFFFFu >> (24 - 8 * e)));
  };
  const int lim_n = min(31, n - 1 - r0);
  const int lim = CAUSAL ? min(t, lim_n) : lim_n;
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] &= keep(lim, i);
  *(u32x4 *)(rec + rec_diag_off(s) + 32 * t + 16 * hh) = c;
  if (rec_c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] &= keep(min(t, lim_n), i);
    *(u32x4 *)(rec_c + rec_diag_off(s) + 32 * t + 16 * hh) = c;
  }
}

}  // namespace dev

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


// The block-edge records of every (head, 32-row group), causal or not, into
// ws (records_bytes(a.n, a.heads, a.s) bytes, 16-byte aligned).
// (non-causal with ws_causal set: both record sets in one pass)
plsh_status launch_edges(const dev::AttnArgs &a, bool causal, hipStream_t st, const char *who, void *ws,
                         void *ws_causal) {
  const int g32 = (a.n + 31) / 32;
  const int items = a.heads * g32;
  const dim3 egrid((unsigned)((items + 3) / 4)), eblock(256);
  const size_t eshm = 4 * (dev::wavetab_bytes(a.s) + 32 * 16 * 4);
  if (causal) hipLaunchKernelGGL(dev::edges_kernel<true>, egrid, eblock, eshm, st, a.params, a.pstride, a.n, a.heads, a.s, g32, (uint8_t *)ws, (uint8_t *)nullptr);
  else hipLaunchKernelGGL(dev::edges_kernel<false>, egrid, eblock, eshm, st, a.params, a.pstride, a.n, a.heads, a.s, g32, (uint8_t *)ws, (uint8_t *)ws_causal);
  return launch_check(who);
}

plsh_status launch_debug_intervals(const plsh_tables *bt, int32_t *lohi, hipStream_t st, const char *who) {
  const int groups = (bt->n + 31) / 32;
  const size_t shm = dev::wavetab_bytes(bt->s);
  hipLaunchKernelGGL(dev::debug_intervals_kernel, dim3((unsigned)((int64_t)groups * bt->heads)), dim3(64), shm, st,
                     bt->params, bt->n, bt->heads, bt->s, groups, lohi);
  return launch_check(who);
}

}  // namespace plsh
