// plsh_mfma16.hip -- the kernels with 16-row waves (gfx950): the estimator
// as the unfused form's fp32 partials and as the per-sample walk, the
// backward's dQ and dK/dV, and the log-sum-exp combine.
//
// "Positional LSH: Binary Block Matrix Approximation for Attention with Linear
// Biases", Methodology §3 (Theorem 2.2): the ratio-of-sums estimator
//   T~_i = sum_j c_ij e^{q_i.k_j} v_j / sum_j c_ij e^{q_i.k_j},
//   c_ij = #{k : j in B_k(i)}  (times the causal mask),
// over the block-edge records of the pre-pass (plsh_prepass.hip; format in
// plsh_device.h).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "plsh_hip_status.h"
#include "plsh_kernels.h"
#include "plsh_mfma16.h"

namespace plsh {
namespace dev {


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
  if (!active) return;
  float ltot = lsum + xor16_f(lsum);
  ltot += other_half_f(ltot, lane);
  const float inv = 1.0f / ltot;
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
// known (lse2 from the forward) instead of an online softmax:
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
  // fragment), the row's normaliser and D = dO . O from the forward's output
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
    if (active && i < n) lse2r = a.lse2[row];
    // D_i = dO_i . O_i in the dO fragment's layout: the lane's 8 NC dims,
    // then the sum over the row's four lanes; written for the dK/dV kernel
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

// One MFMA kernel over records ws (causal records for modes 0, 1 and 3 of a
// causal call, non-causal ones otherwise).  mode 0: the estimator
// (attn_mfma_kernel); 1: its backward dQ (attn_dq_kernel); 2: its backward
// dK, dV into dk, dv (attn_dkv_kernel); 3: the estimator walking the samples
// one by one over single-sample records (attn_mfma_kernel<.., true>).
plsh_status launch_attn(const dev::AttnArgs &a, int d, int causal, hipStream_t st, const char *who, int mode,
                        const void *ws, void *dk, void *dv) {
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

plsh_status launch_combine(const float *o32, const float *lse, int s, int64_t rows, int d, void *out,
                           hipStream_t st, const char *who) {
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (d == 64) hipLaunchKernelGGL(dev::combine_kernel<64>, grid, block, 0, st, o32, lse, s, rows, (uint16_t *)out);
  else hipLaunchKernelGGL(dev::combine_kernel<128>, grid, block, 0, st, o32, lse, s, rows, (uint16_t *)out);
  return launch_check(who);
}

}  // namespace plsh
