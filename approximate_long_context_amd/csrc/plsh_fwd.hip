// plsh_fwd.hip -- the estimator's forward kernel for gfx950 with 32-row
// waves on 32 x 32 x 16 bf16 matrix ops.
//
// "Positional LSH: Binary Block Matrix Approximation for Attention with Linear
// Biases", Methodology §3 (Theorem 2.2): ALiBi attention as s randomized
// short-context attentions without positional bias, here fused over the
// samples as one ratio of sums per row,
//   T~_i = sum_j c_ij e^{q_i.k_j} v_j / sum_j c_ij e^{q_i.k_j},
//   c_ij = #{k : j in B_k(i)}  (times the causal mask),
// each in-block pair evaluated once with its multiplicity c_ij (the union of
// the s blocks holding i is one interval, Methodology §1: every block holds
// i).  The multiplicities come from the block-edge records of the pre-pass
// (format in plsh_device.h): per 32-row group, the samples' block starts
// left of the group (leads), ends right of it (trails) and the diagonal
// tile's counts.
//
// Layout of the work.  A wave owns one 32-row group of one head (the rows of
// one record).  A workgroup is four waves sharing one K/V stream: either four
// consecutive row groups of one head, or, for light heads (small sigma:
// short blocks), the same row group of up to four query heads of one GQA
// group, which read the same K/V head and need nearly the same short key
// range, so each K/V stage is staged once for all of them.
//
// Per 32-key stage a wave computes S^T = K Q^T (32 keys x 32 queries) with
// eight v_mfma_f32_32x32x16_bf16 (D = 128): lane l holds query l % 32 and
// keys 8 (r / 4) + 4 (l / 32) + r % 4 in accumulator r, so a row's softmax
// statistics need one exchange between lanes l and l ^ 32.  O^T (D x 32
// queries) += V^T P^T takes P straight from those accumulators: contraction
// slot 8 (l / 32) + i of 16-key chunk c stands for key 16 c + 8 (i / 4) +
// 4 (l / 32) + i % 4, and the transposing LDS reads (ds_read_b64_tr_b16)
// deliver V^T in that order.  Each K and V fragment read from LDS feeds a
// 32-query product, half the LDS bytes per pair of 16-query tiles.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <numeric>
#include <vector>

#include "plsh_device.h"
#include "plsh_fwd.h"
#include "plsh_hip_status.h"

namespace plsh {
namespace dev {

constexpr int kFwdWaves = 4;   // waves per workgroup, one 32-row group each
// K/V ring stages: 4 (two stages per barrier) for D = 64 and for launches
// with split row groups; 3 (one stage per barrier) for D = 128 otherwise,
// which keeps a workgroup within a third of the compute unit's LDS
template <int D, bool SPLIT>
constexpr int kFwdRing = (D == 128 && !SPLIT) ? 3 : 4;
constexpr int kKeys = 32;      // keys per stage
// Waves per SIMD the register allocation is held to: D = 64 fits four
// (116 registers; four workgroups of 34 KB of LDS per compute unit); D = 128
// three with the three-stage ring (168 registers, 50 KB), two with the
// four-stage one (188 registers, 66.5 KB).  Against two at D = 64: the
// n = 16384 Mistral-shaped layer at d = 64 takes 0.060 instead of 0.086 ms
// (three: 0.066).
template <int D, bool SPLIT>
constexpr int kFwdWavesPerEu = D == 64 ? 4 : (kFwdRing<D, SPLIT> == 3 ? 3 : 2);
constexpr int kMaxUnits = 128;

struct FwdArgs {
  const uint16_t *q, *k, *v;
  uint16_t *out;
  float *save_lse2;
  const uint8_t *ws;
  int32_t batch, n, heads, kv_heads, s, g32;
  int32_t nunits;
  // unit u = a set of hw consecutive query heads from head (one GQA group),
  // unit_info[u] = head | log2(hw) << 8 | log2(sp) << 10, hw in {1, 2, 4},
  // sp in {1, 2} waves per row group (sp = 2 only with hw = 1: the two
  // waves of a group take alternate stages of its key range and merge their
  // partial sums at the end); its workgroups are unit_start[u] ..
  // unit_start[u+1]-1, batch * ceil(g32 / (4 / (hw sp))) of them; units
  // heaviest first (words, so that the kernel reads them with scalar loads)
  int32_t unit_start[kMaxUnits + 1];
  int32_t unit_info[kMaxUnits];
};

template <int D, int RING>
struct FwdLds {
  alignas(16) uint16_t kv[RING][2][kKeys * D];
  // step[u][4 hf + i]: word 2 i + hf of the byte counters of a tile (keys
  // 4 w .. 4 w + 3 in word w) with 1 in every key at or after offset u
  alignas(16) uint32_t step[kKeys][8];
};

template <int Q>
struct Slot {
  static constexpr int value = Q;
};

// 16-byte chunk swizzle of K rows (and of the staged Q and O rows): the
// operand reads have lanes 0..31 read keys 0..31 at one chunk, and a 16-byte
// read serves lanes 0-7 with 24-31 and 8-15 with 16-23 per cycle, which this
// XOR keeps on 16 distinct chunk positions (D = 64: two keys per 256 bytes).
template <int D>
__device__ __forceinline__ int kswz(int key) {
  return D == 128 ? (key & 15) : ((key >> 1) & 7);
}
template <int D>
__device__ __forceinline__ uint32_t kpos(int key, int chunk) {
  return (uint32_t)(key * 2 * D + ((chunk ^ kswz<D>(key)) << 4));
}

// SPLIT: the launch has units with two waves per row group (the other
// instantiation keeps that code out of the tile loop).
template <int D, bool CAUSAL, bool SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kFwdWaves, 64 * kFwdWaves),
                          amdgpu_waves_per_eu(kFwdWavesPerEu<D, SPLIT>, kFwdWavesPerEu<D, SPLIT>)))
void attn_fwd_kernel(FwdArgs a) {
  constexpr int RING = kFwdRing<D, SPLIT>;
  using L = FwdLds<D, RING>;
  __shared__ __attribute__((aligned(16))) L lds;
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  const int s = a.s, n = a.n;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int t = lane & 31, hf = lane >> 5;
  {
    const int u = threadIdx.x >> 3, e = threadIdx.x & 7;  // 256 threads: 32 x 8 entries
    lds.step[u][e] = step4(u - 4 * (2 * (e & 3) + (e >> 2)));
  }

  // ---- workgroup -> (unit, batch, row block); XCD-aware: workgroups are
  // dealt to the 8 XCDs round-robin, and each XCD takes a contiguous run of
  // the unit's row blocks, so neighbouring blocks share K/V in its L2
  const int p = blockIdx.x;
  int unit = 0;
  {
    int hi = a.nunits - 1;
    while (unit < hi) {
      const int mid = (unit + hi + 1) >> 1;
      if (a.unit_start[mid] <= p) unit = mid; else hi = mid - 1;
    }
  }
  const int ustart = a.unit_start[unit];
  const int G = a.unit_start[unit + 1] - ustart;
  const int tu = p - ustart;
  const int xcd = p & 7, base_mod = ustart & 7;
  int start = 0, t0c = 0;
  for (int c = 0; c < 8; ++c) {
    const int t0 = (c - base_mod + 8) & 7;
    const int cnt = t0 < G ? (G - t0 + 7) / 8 : 0;
    if (c == xcd) { t0c = t0; break; }
    start += cnt;
  }
  const int gidx = start + (tu - t0c) / 8;
  const int info = a.unit_info[unit];
  // wave bits, high to low: head in the set (lhw), row group (lgw), part (lsp)
  const int lhw = (info >> 8) & 3, lsp = SPLIT ? (info >> 10) & 1 : 0, lgw = 2 - lhw - lsp;
  const int gw = 1 << lgw;
  const int nblk = (a.g32 + gw - 1) >> lgw;
  const int b = gidx / nblk, blk = gidx - b * nblk;
  const int h0 = info & 0xFF;
  const bool split = lsp != 0;
  const int part = wave & lsp;            // which alternate stages (split only)
  const int wg_grp = (wave >> lsp) & (gw - 1);  // the wave's row group in the workgroup
  const int h = h0 + (wave >> (lsp + lgw));
  const int grp = (blk << lgw) + wg_grp;
  const int r0 = 32 * grp;
  const bool active = grp < a.g32;
  const int kvh = h / (a.heads / a.kv_heads);
  const size_t rb = rec_bytes(s);
  const uint8_t *rec = a.ws + ((size_t)h * a.g32 + min(grp, a.g32 - 1)) * rb;

  const uint16_t *Q = a.q + ((int64_t)b * a.heads + h) * n * D;
  const char *Kb = (const char *)(a.k + ((int64_t)b * a.kv_heads + kvh) * n * D);
  const char *Vb = (const char *)(a.v + ((int64_t)b * a.kv_heads + kvh) * n * D);

  // ---- the record headers of the four waves' groups (scalar loads, issued
  // before the copies below so that they may read through the scalar cache)
  int4 hdr[kFwdWaves];
#pragma unroll
  for (int w = 0; w < kFwdWaves; ++w) {
    const int g2 = min((blk << lgw) + ((w >> lsp) & (gw - 1)), a.g32 - 1);
    hdr[w] = *(const int4 *)(a.ws + ((size_t)(h0 + (w >> (lsp + lgw))) * a.g32 + g2) * rb);
  }
  // ---- then the loads that need only the wave's own record and rows: the
  // lane's row of the diagonal table, the sorted edge lists (into the wave's
  // LDS slice, 16 bytes = two edges per lane) and the 32 query rows; all
  // land by the first stage's wait.  The query rows go straight to the
  // lane's Q fragments (B operand: query t, dims 16 c + 8 hf .. + 7) with the
  // three-stage ring, whose slots are all taken by K/V from the start, and
  // else through ring slots 2, 3 (free until the first stages have been
  // read; whole rows per copy instruction, K-row swizzle).
  constexpr int NC = D / 16;  // QK^T products per stage
  bf16x8 qf[NC];
  if (RING == 3 && active) {
    const uint16_t *qrow = Q + (int64_t)min(r0 + t, n - 1) * D + 8 * hf;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = *(const bf16x8 *)(qrow + 16 * c);
  }
  // (of the row's eight table words, the lane's are 2 i + hf, i = 0..3;
  // non-causal, the last byte too: the count after the diagonal tile)
  uint32_t dw[4] = {0u, 0u, 0u, 0u}, dlast = 0u;
  if (active) {
    const uint32_t *drow = (const uint32_t *)(rec + rec_diag_off(s) + 32 * t);
#pragma unroll
    for (int i = 0; i < 4; ++i) dw[i] = drow[2 * i + hf];
    if (!CAUSAL) dlast = drow[7] >> 24;
  }
  const int nch = ev_count(s) / 2;
  u32x2 *evl = (u32x2 *)(dyn + (size_t)wave * ev_wave_bytes(s, CAUSAL));
  u32x2 *evt = evl + ev_count(s);
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  const uint32_t q_lds = lds_addr(&lds.kv[2][0][0]) + wave * 32 * D * 2;
  if (active) {
    for (int c0 = 0; c0 < nch; c0 += 64)
      if (c0 + lane < nch) dma16(rec + rec_evl_off() + 16 * (c0 + lane), lds_addr(evl + 2 * c0));
    if (!CAUSAL)
      for (int c0 = 0; c0 < nch; c0 += 64)
        if (c0 + lane < nch) dma16(rec + rec_evt_off(s) + 16 * (c0 + lane), lds_addr(evt + 2 * c0));
    if (RING == 4) {
#pragma unroll
      for (int c0 = 0; c0 < 32 * CPR; c0 += 64) {
        const int row = (c0 + lane) / CPR, ch = (c0 + lane) % CPR;
        const int64_t off = (int64_t)min(r0 + row, n - 1) * (2 * D) + 16 * (ch ^ kswz<D>(row));
        dma16((const char *)Q + off, q_lds + 16 * c0);
      }
    }
  }

  // ---- key ranges of the four waves' groups (only the scalar header loads
  // are waited for here), the union is the workgroup's stream
  int U0 = INT32_MAX, U1 = INT32_MIN, U0w = 0, U1w = 0;
  {
#pragma unroll
    for (int w = 0; w < kFwdWaves; ++w) {
      if ((blk << lgw) + ((w >> lsp) & (gw - 1)) < a.g32) {
        U0 = min(U0, hdr[w].y);
        U1 = max(U1, hdr[w].z);
      }
      if (w == wave) { U0w = hdr[w].y; U1w = hdr[w].z; }
    }
  }
  // (a record always holds 0 <= U0 < U1 <= 32 g32; the clamp keeps every
  // address inside the tensors even for a workspace that holds no records)
  U0 = min(max(U0, 0), 32 * a.g32);
  U1 = min(U1, 32 * a.g32);
  const int nst = (U1 > U0) ? (U1 - U0) / kKeys : 0;

  // ---- K/V staging: a K tile is 32 whole rows (K-row swizzle), a V tile 32
  // keys x D as 64-byte pieces per 32 dims (vpiece128); each tile is 4 D
  // 16-byte chunks, wave w copies chunks [w D, (w + 1) D).  The copies go
  // through buffer resources over the head's K and V rows: the lane's offset
  // inside a tile is fixed, the tile's start is a scalar offset, and keys
  // past the end read as zeros, whose products get c = 0.
  constexpr int NCW = D / 64;  // copy instructions per wave, tile and stage
  const uint32_t kv_lds = lds_addr(&lds.kv[0][0][0]);
  const i32x4 krs = buffer_rsrc(Kb, (uint32_t)n * (2 * D)), vrs = buffer_rsrc(Vb, (uint32_t)n * (2 * D));
  uint32_t ck_off[NCW], cv_off[NCW];
#pragma unroll
  for (int j = 0; j < NCW; ++j) {
    const int ci = wave * D + 64 * j + lane;  // the lane's chunk position in the tile
    ck_off[j] = (uint32_t)((ci / CPR) * (2 * D) + 16 * ((ci % CPR) ^ kswz<D>(ci / CPR)));
    const int P = 16 * ci;
    const int vkey = (P >> 6) & 31;
    cv_off[j] = (uint32_t)(vkey * (2 * D) + 16 * (4 * (P >> 11) + (((P >> 4) & 3) ^ (((vkey >> 2) & 1) << 1))));
  }
  auto issue_stage = [&](int st, int q) {  // q = st % kFwdRing
    const uint32_t soff = (uint32_t)(U0 + kKeys * st) * (2 * D);
#pragma unroll
    for (int j = 0; j < NCW; ++j) {
      const uint32_t dst = kv_lds + (uint32_t)(2 * q) * (kKeys * D * 2) + 16 * (wave * D + 64 * j);
      dma16_buf(krs, ck_off[j], soff, dst);
      dma16_buf(vrs, cv_off[j], soff, dst + kKeys * D * 2);
    }
  };
  if (nst > 0) issue_stage(0, 0);
  if (nst > 1) issue_stage(1, 1);

  // ---- running state of the lane's row
  constexpr int NB = D / 32;  // 32-dim blocks of O^T
  floatx16 oacc[NB];
#pragma unroll
  for (int db = 0; db < NB; ++db) oacc[db] = floatx16{};
  float m2 = -INFINITY;  // running max, log2 units
  float lsum = 0.f;      // this lane's share of the row sum
  int base = 0;          // the row's multiplicity just before the current tile
  int lp = 0, tp = 0;    // next unconsumed lead / trail edge
  int pl = 0, pt = 0;    // their positions (wave-uniform)
  int lg_base = -1;      // the count whose log2 is lg
  float lg = 0.f;
  auto pos_at = [&](const u32x2 *ev, int i) { return (int32_t)__builtin_amdgcn_readfirstlane(ev[i][0]); };

  // K operand of product c: key t, chunk 2 c + hf
  uint32_t kofs[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) kofs[c] = kpos<D>(t, 2 * c + hf);
  // V operand (transposing reads): lane (g = l / 16, r = l % 16) names key
  // 4 (g / 2) + r / 4 (+ 16 c + 8 e) at dims 32 b + 16 (g % 2) + 4 (r % 4);
  // every read of a stage is this address plus an immediate
  uint32_t vofs;
  {
    const int g = lane >> 4, r = lane & 15;
    const int kk = 4 * (g >> 1) + (r >> 2);
    const int x = 2 * (g & 1) + ((r & 3) >> 1);  // 16-byte chunk inside the 64-byte piece
    vofs = (uint32_t)(kk * 64 + ((x ^ (((kk >> 2) & 1) << 1)) << 4) + 8 * (r & 1));
  }
  const int sa = active ? (U0w - U0) / kKeys : 0;
  const int sb = active ? (U1w - U0) / kKeys : 0;

  // a5: S^T = K Q^T for the stage in ring slot Q0: the K fragment reads of
  // a group are issued first, then its products (one group; two with the
  // three-stage ring, whose register budget holds half the fragments)
  auto qk_tile = [&](auto s0, floatx16 &SA) {
    const char *ka = (const char *)lds.kv[decltype(s0)::value][0];
    constexpr int KG = RING == 3 ? NC / 2 : NC;  // fragments per group
    SA = floatx16{};
#pragma unroll
    for (int g0 = 0; g0 < NC; g0 += KG) {
      u32x4 kra[KG];
#pragma unroll
      for (int c = 0; c < KG; ++c) kra[c] = *(const u32x4 *)(ka + kofs[g0 + c]);
#pragma unroll
      for (int c = 0; c < KG; ++c)
        SA = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kra[c]), qf[g0 + c], SA, 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, KG, 0);  // the group's K reads
      __builtin_amdgcn_sched_group_barrier(0x008, KG, 0);  // then its products
    }
  };

  // Visits, in order, the edges of a sorted list at positions < jend from
  // index ptr (position pp) and advances both: lane l reads edge ptr + l, so up
  // to 64 edges are found with one LDS read and a ballot (the list ends in 16
  // sentinels at INT32_MAX, so ptr stops at the first of them).  Reads are
  // clamped to the list, and a full ballot at or past its last entry ends the
  // walk, so even a list that is not sorted stays inside itself and ends.
  const int ev_last = s + kSentinels - 1;
  auto edges_in_tile = [&](const u32x2 *ev, int &ptr, int &pp, int jend, auto &&visit) {
    while (pp < jend) {
      const u32x2 e = ev[min(ptr + lane, ev_last)];
      const int k = __popcll(__ballot((int32_t)e[0] < jend));  // a prefix of the lanes
      for (int i = 0; i < k; ++i)
        visit((int32_t)__builtin_amdgcn_readlane(e[0], i), __builtin_amdgcn_readlane(e[1], i));
      ptr += k;
      pp = k < 64 ? (int32_t)__builtin_amdgcn_readlane(e[0], k) : (ptr >= ev_last ? INT32_MAX : pos_at(ev, ptr));
    }
  };

  // a4, a6, a7 for the stage in ring slot Q, whose logits are in sacc
  auto finish_tile = [&](int st, auto slotc, const floatx16 &sacc_in) {
    floatx16 sacc = sacc_in;
    const char *vt = (const char *)lds.kv[decltype(slotc)::value][1];
    const int j0 = U0 + kKeys * st;
    const int jend = j0 + kKeys;
    // a4: multiplicity of keys j0 + 8 (r / 4) + 4 hf + r % 4, byte r % 4 of
    // counter word r / 4 (tile word 2 (r / 4) + hf):
    //  * diagonal tile: the row's bytes of the record's table;
    //  * a tile holding edges (leads left of the diagonal, trails right of it;
    //    positions wave-uniform): base +- sum over edges of [row's block
    //    starts / ends there] [key >= edge];
    //  * otherwise one count, base, for every key of the tile.
    float cf[16];
    int kind;  // 0: one count for the tile, 1: per-key counts
    if (j0 == r0) {
      // the lane's words 2 i + hf of its row of the record's table (loaded
      // in the prologue; landed by the first stage's wait)
      uint32_t d0 = dw[0], d1 = dw[1], d2 = dw[2], d3 = dw[3];
      asm volatile("" : "+v"(d0), "+v"(d1), "+v"(d2), "+v"(d3));
      const uint32_t dd[4] = {d0, d1, d2, d3};
#pragma unroll
      for (int r = 0; r < 16; ++r) cf[r] = (float)((dd[r >> 2] >> (8 * (r & 3))) & 0xFFu);
      // keys of the tile outside the row's blocks (causal: the keys after
      // the row) leave the running max and the weights: their logits, which
      // may be far above the row's own, would otherwise raise the max until
      // the row's weights underflow.  The row's own key always counts s, so
      // the max stays finite.
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = cf[r] > 0.f ? sacc[r] : -INFINITY;
      // the table already counts every edge up to the tile's end
      edges_in_tile(evl, lp, pl, jend, [](int, uint32_t) {});
      if (!CAUSAL) {
        edges_in_tile(evt, tp, pt, jend, [](int, uint32_t) {});
        base = (int)dlast;  // c(row, r0 + 31): the count after the diagonal tile
      }
      kind = 1;
    } else if (pl < jend || (!CAUSAL && pt < jend)) {
      const uint32_t b4 = (uint32_t)base * 0x01010101u;
      uint32_t cw[4] = {b4, b4, b4, b4};
      const uint32_t *srow = &lds.step[0][4 * hf];
      // (an edge visited here lies in the tile, pos - j0 in [0, 32), for any
      // list the pre-pass wrote; for any other the read stays an LDS read,
      // which the hardware range-checks against the workgroup's allocation)
      auto step_at = [&](int pos) { return *(const u32x4 *)(srow + 8 * (pos - j0)); };
      edges_in_tile(evl, lp, pl, jend, [&](int pos, uint32_t W) {
        const uint32_t w = (W >> t) & 1u;
        const u32x4 sr = step_at(pos);
#pragma unroll
        for (int i = 0; i < 4; ++i) cw[i] += w * sr[i];
        base += (int)w;
      });
      if (!CAUSAL)
        edges_in_tile(evt, tp, pt, jend, [&](int pos, uint32_t W) {
          const uint32_t w = (W >> t) & 1u;
          const u32x4 sr = step_at(pos);
#pragma unroll
          for (int i = 0; i < 4; ++i) cw[i] -= w * sr[i];
          base -= (int)w;
        });
#pragma unroll
      for (int r = 0; r < 16; ++r) cf[r] = (float)((cw[r >> 2] >> (8 * (r & 3))) & 0xFFu);
      kind = 1;
    } else {
      cf[0] = (float)base;
      kind = 0;
    }

    // a6: weighted online softmax in the log2 domain; the running max is
    // raised only when a logit exceeds it by more than 2^8 (the result does
    // not depend on the max used), and then for both lanes of the row
    float mx = max3f(max3f(sacc[0], sacc[1], sacc[2]), max3f(sacc[3], sacc[4], sacc[5]),
                     max3f(sacc[6], sacc[7], sacc[8]));
    mx = max3f(mx, max3f(sacc[9], sacc[10], sacc[11]), max3f(sacc[12], sacc[13], sacc[14]));
    mx = max3f(mx, sacc[15], sacc[15]);
    if (__any(mx * kLog2e > m2 + 8.0f)) {
      mx = max3f(mx, other_half_f(mx, lane), mx) * kLog2e;
      const bool need = mx > m2 + 8.0f;
      const float mnew = need ? mx : m2;
      const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NB; ++db) oacc[db] *= alpha;
      m2 = mnew;
    }
    // P = c 2^(x - m2), rounded to bf16 in pairs; the row sum adds exactly
    // the rounded weights that enter PV.  A tile with one count folds
    // log2 c into the exponent bias (c = 0: bias +inf, P = 0).
    u32x4 pw[2];
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    if (__builtin_amdgcn_readfirstlane(kind) == 0) {
      if (__any(base != lg_base)) {
        lg = __builtin_amdgcn_logf(cf[0]);
        lg_base = base;
      }
      const float bias = m2 - lg;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const floatx2 pf = {__builtin_amdgcn_exp2f(fmaf(sacc[r], kLog2e, -bias)),
                            __builtin_amdgcn_exp2f(fmaf(sacc[r + 1], kLog2e, -bias))};
        const bf16x2 pb = __builtin_convertvector(pf, bf16x2);
        pw[r >> 3][(r & 7) >> 1] = __builtin_bit_cast(uint32_t, pb);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, lsum, false);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const floatx2 pf = {cf[r] * __builtin_amdgcn_exp2f(fmaf(sacc[r], kLog2e, -m2)),
                            cf[r + 1] * __builtin_amdgcn_exp2f(fmaf(sacc[r + 1], kLog2e, -m2))};
        const bf16x2 pb = __builtin_convertvector(pf, bf16x2);
        pw[r >> 3][(r & 7) >> 1] = __builtin_bit_cast(uint32_t, pb);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, lsum, false);
      }
    }

    // a7: O^T += V^T P^T, two 16-key chunks, V^T by transposing reads (each
    // chunk's reads issued together ahead of its products)
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      u32x4 vop[NB];
#pragma unroll
      for (int db = 0; db < NB; ++db) {
        const char *va = vt + vofs + db * 2048 + cc * 1024;
        const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t *)va);
        const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t *)(va + 512));
        vop[db] = u32x4{__builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1)),
                        __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3)),
                        __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1)),
                        __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3))};
      }
#pragma unroll
      for (int db = 0; db < NB; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vop[db]),
                                                           __builtin_bit_cast(bf16x8, pw[cc]), oacc[db], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * NB, 0);  // the chunk's reads
      __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);      // then its products
    }
  };

  // Split row groups: the edges of a stage the other wave of the group
  // computes still move this wave's running count past it (the diagonal
  // tile's table already counts every edge up to its end; after it, the
  // count of the row's last key is the base, non-causal)
  auto skip_tile = [&](int st) {
    const int j0 = U0 + kKeys * st;
    const int jend = j0 + kKeys;
    if (j0 == r0) {
      edges_in_tile(evl, lp, pl, jend, [](int, uint32_t) {});
      if (!CAUSAL) {
        edges_in_tile(evt, tp, pt, jend, [](int, uint32_t) {});
        base = (int)dlast;
      }
    } else {
      edges_in_tile(evl, lp, pl, jend, [&](int, uint32_t W) { base += (int)((W >> t) & 1u); });
      if (!CAUSAL) edges_in_tile(evt, tp, pt, jend, [&](int, uint32_t W) { base -= (int)((W >> t) & 1u); });
    }
  };

  // Two stages per barrier: the pair starting at stage st waits for stages
  // st, st + 1, refills the slots of stages st - 2, st - 1 (every wave is
  // past them) with st + 2, st + 3, and computes its two tiles.
  auto pair = [&](int st, auto s0, auto s1) {
    PLSH_WAIT_VM_LGKM0(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (st == 0) {
      // the Q fragment (B operand: query t, dims 16 c + 8 hf .. + 7), then a
      // barrier: every wave has its fragment before slots 2, 3 take stages 2, 3
      const char *qt = (const char *)lds.kv[2][0] + wave * 32 * D * 2;
#pragma unroll
      for (int c = 0; c < NC; ++c) qf[c] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qt + kpos<D>(t, 2 * c + hf)));
      PLSH_WAIT_VM_LGKM0(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (active) {  // the edge lists landed with stage 0
        pl = pos_at(evl, 0);
        if (!CAUSAL) pt = pos_at(evt, 0);
      }
    }
    if (st + 2 < nst) issue_stage(st + 2, (decltype(s0)::value + 2) % RING);
    if (st + 3 < nst) issue_stage(st + 3, (decltype(s1)::value + 2) % RING);
    // (split groups: part 0 computes stage st, part 1 stage st + 1, and each
    // moves its count past the other's)
    const bool ra = st >= sa && st < sb;
    const bool rb = st + 1 < nst && st + 1 >= sa && st + 1 < sb;
    const bool ta = ra && part == 0, tb = rb && (!split || part == 1);
    floatx16 SA;
    if (ra && part == 1) skip_tile(st);
    if (ta) {
      qk_tile(s0, SA);
      finish_tile(st, s0, SA);
    }
    if (rb && split && part == 0) skip_tile(st + 1);
    if (tb) {
      qk_tile(s1, SA);
      finish_tile(st + 1, s1, SA);
    }
  };
  // One stage per barrier (three-stage ring): stage st waits for its own
  // copies only (those of st + 1, issued after them, may still be in
  // flight: copies complete in issue order), refills the slot of stage
  // st - 1 (every wave is past it) with st + 2, and computes its tile.
  auto single = [&](int st, auto s0) {
    if (st + 1 < nst) PLSH_WAIT_VM_LGKM0(2 * NCW);
    else PLSH_WAIT_VM_LGKM0(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (st == 0 && active) {  // the edge lists landed before stage 0
      pl = pos_at(evl, 0);
      if (!CAUSAL) pt = pos_at(evt, 0);
    }
    if (st + 2 < nst) issue_stage(st + 2, (decltype(s0)::value + 2) % RING);
    if (st >= sa && st < sb) {
      floatx16 SA;
      qk_tile(s0, SA);
      finish_tile(st, s0, SA);
    }
  };
  if constexpr (RING == 3) {
    // the first stage's wait, and with it the Q fragments and the table
    // words, ahead of the loop: the compiler, which does not see the
    // copies, then counts those loads as done inside it (else it waits on
    // them at every tile, and with them on the later stages' copies)
    if (nst > 1) PLSH_WAIT_VM_LGKM0(2 * NCW);
    else PLSH_WAIT_VM_LGKM0(0);
#pragma unroll
    for (int c = 0; c < NC; ++c) asm volatile("" : "+v"(qf[c]));
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(dw[i]));
    asm volatile("" : "+v"(dlast));
    for (int st0 = 0; st0 < nst; st0 += 3) {
      single(st0, Slot<0>{});
      if (st0 + 1 < nst) single(st0 + 1, Slot<1>{});
      if (st0 + 2 < nst) single(st0 + 2, Slot<2>{});
    }
  } else {
    for (int st0 = 0; st0 < nst; st0 += 4) {
      pair(st0, Slot<0>{}, Slot<1>{});
      if (st0 + 2 < nst) pair(st0 + 2, Slot<2>{}, Slot<3>{});
    }
  }

  // ---- split row groups: the part-1 wave hands its partial sums (running
  // max, row-sum share, O^T accumulators, lane by lane) to the part-0 wave
  // through LDS, every ring slot being free once all waves have passed the
  // barrier; the part-0 wave merges them into its own, each side scaled by
  // 2^(m_p - max(m_0, m_1)), and writes the rows
  if (split) {
    PLSH_WAIT_VM_LGKM0(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    u32x4 *pacc = (u32x4 *)lds.kv[0][0] + wg_grp * (4 * NB * 64);  // [4 NB][64 lanes] 16-byte words
    float *pml = (float *)&lds.step[0][0] + wg_grp * 128;            // [2][64 lanes]
    if (part == 1 && active) {
#pragma unroll
      for (int db = 0; db < NB; ++db)
#pragma unroll
        for (int r = 0; r < 16; r += 4)
          pacc[(4 * db + r / 4) * 64 + lane] =
              u32x4{__float_as_uint(oacc[db][r]), __float_as_uint(oacc[db][r + 1]), __float_as_uint(oacc[db][r + 2]),
                    __float_as_uint(oacc[db][r + 3])};
      pml[lane] = m2;
      pml[64 + lane] = lsum;
    }
    PLSH_WAIT_VM_LGKM0(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (part == 1) return;
    if (active) {
      const float m1 = pml[lane], l1 = pml[64 + lane];
      const float mm = fmaxf(m2, m1);
      const float a0 = __builtin_amdgcn_exp2f(m2 - mm), a1 = __builtin_amdgcn_exp2f(m1 - mm);
      lsum = lsum * a0 + l1 * a1;
#pragma unroll
      for (int db = 0; db < NB; ++db)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          const u32x4 o1 = pacc[(4 * db + r / 4) * 64 + lane];
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[db][r + i] = oacc[db][r + i] * a0 + __uint_as_float(o1[i]) * a1;
        }
      m2 = mm;
    }
  }

  // ---- a8: O = acc / l, rounded to bf16, staged in two ring slots no wave
  // still reads (four stages: the two the last pair does not use; three: those
  // of the last stage's two predecessors, every wave being past both; split
  // groups: slots 2, 3, past the merge's barrier) and stored whole rows per
  // instruction
  if (!active) return;
  const float ltot = lsum + other_half_f(lsum, lane);
  const float inv = 1.0f / ltot;
  const int ns = 32 * a.g32;
  if (a.save_lse2 && hf == 0)
    a.save_lse2[((int64_t)b * a.heads + h) * ns + r0 + t] = r0 + t < n ? m2 + __log2f(ltot) : 0.f;
  char *ob;
  if constexpr (RING == 3) {
    const int last = nst > 0 ? (nst - 1) % 3 : 2;
    ob = (char *)lds.kv[(last + 1 + (wave >> 1)) % 3][0] + (wave & 1) * 32 * D * 2;
  } else {
    const int free_slot = split ? 2 : ((((nst - 1) >> 1) & 1) ? 0 : 2);
    ob = (char *)lds.kv[free_slot][0] + (split ? wg_grp : wave) * 32 * D * 2;
  }
#pragma unroll
  for (int db = 0; db < NB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // dims 32 db + 8 j + 4 hf .. + 3: half hf of chunk 4 db + j
      const bf16x2 h0 = __builtin_convertvector((floatx2{oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv}), bf16x2);
      const bf16x2 h1 =
          __builtin_convertvector((floatx2{oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv}), bf16x2);
      *(u32x2 *)(ob + kpos<D>(t, 4 * db + j) + 8 * hf) =
          u32x2{__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1)};
    }
  wave_sync();
  uint16_t *O = a.out + ((int64_t)b * a.heads + h) * n * D;
#pragma unroll
  for (int c0 = 0; c0 < 32 * CPR; c0 += 64) {
    const int row = (c0 + lane) / CPR, ch = (c0 + lane) % CPR;
    const u32x4 val = *(const u32x4 *)(ob + kpos<D>(row, ch));
    const int i = r0 + row;
    if (i < n) *(u32x4 *)(O + (int64_t)i * D + 8 * ch) = val;
  }
}

}  // namespace dev

// Compute units of the current device (2 resident workgroups each), cached
// per device; 256 if the query fails.
static int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) {
    (void)hipGetLastError();
    v = 256;
  }
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// Waves per row group for each unit (1, or 2 for single-head units whose
// workgroups would otherwise set the kernel's length).  Work estimate per
// 32-row group in 32-key stages: the union of a row's s blocks reaches
// about 1.55 sigma ln s keys back (causal; twice that, both sides, when not),
// fitted to sampled tables for sigma 2..256 and s 10..40.  A workgroup of
// four groups computes about (stages + 3) tiles per wave; split into two
// groups of two waves, each wave computes about half of its group's stages
// plus a merge, with one tile per barrier instead of two.  Only when a
// launch has fewer than two workgroups per resident slot (2 per CU) is the
// tail not filled by later workgroups, so only then are heads split, and
// only those whose workgroups exceed 1.5 times both the average load per
// slot and the average workgroup's load: a split wave has one tile per
// barrier to cover the next stages' copies, so splitting heads of equal
// weight measured slower (sigma = 256 everywhere, n = 4096: 80 -> 92 us),
// while splitting the few heaviest of unequal heads shortens the tail
// (sigma = 2 .. 256, n = 4096: 59 -> 43 us).  The rule
// counts one batch element, every head as its own unit, and never splits a
// light head (sigma <= kSharedKvSigma): a batch and each of its slices, and
// a GQA layout and the same heads with repeated K/V, take the same
// decisions and so give the same bits.
template <class HW, class KEY>
static std::vector<int> split_units(const FwdCall &c, size_t nunits, HW hw_of, KEY sigma_of) {
  std::vector<int> sp(nunits, 1);
  const int g32 = (c.n + 31) / 32;
  const double slots = 2.0 * device_cus();
  const double lns = std::log((double)std::max(c.s, 2));
  const double reach = c.causal ? 0.5 * c.n : (double)c.n;
  auto load_of = [&](double sigma) {
    const double keys = c.causal ? 48.0 + 1.55 * sigma * lns : 64.0 + 3.1 * sigma * lns;
    return std::min(keys, reach) / 32.0 + 3.0;
  };
  const double nwg = (double)((g32 + 3) / 4);  // per head and batch element, four groups per workgroup
  double load = 0.0;
  for (int h = 0; h < c.heads; ++h) load += nwg * load_of(c.sigma[h]);
  if (nwg * c.heads >= 2.0 * slots) return sp;
  const double bar = 1.5 * std::max(load / slots, load / (nwg * c.heads));
  for (size_t u = 0; u < nunits; ++u)
    if (hw_of(u) == 1 && sigma_of(u) > kSharedKvSigma && load_of(sigma_of(u)) > bar) sp[u] = 2;
  return sp;
}

plsh_status launch_fwd(const FwdCall &c, hipStream_t st, std::pair<hipEvent_t, hipEvent_t> *timer,
                       const char *who) {
  // (a head's K or V rows, up to the last tile's end, are addressed through
  // 32-bit buffer offsets)
  if (((int64_t)c.n + 31) * 2 * c.d >= ((int64_t)1 << 32))
    return fail(PLSH_ERR_UNSUPPORTED, "%s: n = %d exceeds %lld at d = %d", who, c.n,
                (long long)(((int64_t)1 << 32) / (2 * c.d) - 32), c.d);
  if (c.heads > dev::kMaxUnits) return fail(PLSH_ERR_UNSUPPORTED, "%s: heads = %d exceeds %d", who, c.heads, dev::kMaxUnits);
  dev::FwdArgs a;
  a.q = (const uint16_t *)c.q;
  a.k = (const uint16_t *)c.k;
  a.v = (const uint16_t *)c.v;
  a.out = (uint16_t *)c.out;
  a.save_lse2 = c.save_lse2;
  a.ws = (const uint8_t *)c.ws;
  a.batch = c.batch;
  a.n = c.n;
  a.heads = c.heads;
  a.kv_heads = c.kv_heads;
  a.s = c.s;
  a.g32 = (c.n + 31) / 32;
  // head sets: within each GQA group, sets of hw consecutive heads, hw the
  // largest of 4, 2 that divides the group size when every head of the group
  // is light (sigma <= kSharedKvSigma), else single heads; heaviest set first
  const int grp = c.heads / c.kv_heads;
  struct U { int head, hw; double key; };
  std::vector<U> units;
  for (int g0 = 0; g0 < c.heads; g0 += grp) {
    double smax = 0.0;
    for (int h = g0; h < g0 + grp; ++h) smax = std::max(smax, c.sigma[h]);
    const int hw = smax <= kSharedKvSigma ? (grp % 4 == 0 ? 4 : grp % 2 == 0 ? 2 : 1) : 1;
    for (int h = g0; h < g0 + grp; h += hw) {
      double key = 0.0;
      for (int x = h; x < h + hw; ++x) key = std::max(key, c.sigma[x]);
      units.push_back({h, hw, key});
    }
  }
  std::stable_sort(units.begin(), units.end(), [](const U &x, const U &y) { return x.key > y.key; });
  const std::vector<int> sp = split_units(c, units.size(), [&](size_t u) { return units[u].hw; },
                                          [&](size_t u) { return units[u].key; });
  a.nunits = (int32_t)units.size();
  int64_t total = 0;
  for (size_t u = 0; u < units.size(); ++u) {
    a.unit_start[u] = (int32_t)total;
    a.unit_info[u] =
        units[u].head | ((units[u].hw == 4 ? 2 : units[u].hw == 2 ? 1 : 0) << 8) | ((sp[u] == 2 ? 1 : 0) << 10);
    const int gw = 4 / (units[u].hw * sp[u]);
    total += (int64_t)c.batch * ((a.g32 + gw - 1) / gw);
    if (total >= ((int64_t)1 << 31)) return fail(PLSH_ERR_UNSUPPORTED, "%s: too many workgroups", who);
  }
  a.unit_start[units.size()] = (int32_t)total;
  for (size_t u = units.size() + 1; u <= (size_t)dev::kMaxUnits; ++u) a.unit_start[u] = (int32_t)total;
  const dim3 grid((unsigned)total), block(64 * dev::kFwdWaves);
  const size_t shm = dev::kFwdWaves * dev::ev_wave_bytes(c.s, c.causal);
  auto go = [&](auto kern) {
    if (timer) hipExtLaunchKernelGGL(kern, grid, block, (uint32_t)shm, st, timer->first, timer->second, 0u, a);
    else hipLaunchKernelGGL(kern, grid, block, shm, st, a);
  };
  const bool any_split = std::find(sp.begin(), sp.end(), 2) != sp.end();
  if (c.d == 64) {
    if (c.causal) any_split ? go(dev::attn_fwd_kernel<64, true, true>) : go(dev::attn_fwd_kernel<64, true, false>);
    else any_split ? go(dev::attn_fwd_kernel<64, false, true>) : go(dev::attn_fwd_kernel<64, false, false>);
  } else {
    if (c.causal) any_split ? go(dev::attn_fwd_kernel<128, true, true>) : go(dev::attn_fwd_kernel<128, true, false>);
    else any_split ? go(dev::attn_fwd_kernel<128, false, true>) : go(dev::attn_fwd_kernel<128, false, false>);
  }
  return launch_check(who);
}

}  // namespace plsh
