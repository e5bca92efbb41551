// plsh_exact.hip -- dense exact-ALiBi attention (the comparator) for gfx950,
// with 32-row waves on 32 x 32 x 16 bf16 matrix ops.
//
// Exact ALiBi attention (Problem Statement; Methodology §1 of "Positional
// LSH: Binary Block Matrix Approximation for Attention with Linear Biases"):
//   O_i = sum_j e^{q_i.k_j - |i - j| / sigma_h} v_j / sum_j e^{...},
// j <= i when causal.  Every key of [0, n) (causal: [0, i]) is visited: the
// O(n^2) work the estimator avoids.
//
// Layout of the work.  A workgroup is four waves, each owning 32 consecutive
// query rows of one head (128 rows); the waves share one stream of 32-key
// K/V stages through a three-slot LDS ring (one stage per barrier, copies
// straight from global memory into LDS through buffer resources).  Per stage
// a wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16: lane l holds
// query row l % 32 and keys 8 (r / 4) + 4 (l / 32) + r % 4 of the stage in
// accumulator r, so a row's softmax statistics need one exchange between
// lanes l and l ^ 32; O^T += V^T P^T takes P from those accumulators with V^T
// from transposing LDS reads.
//
// The bias.  Softmax is unchanged by a per-row constant, so row i = r0 + t
// of a wave whose rows start at r0 may use the logit shifted by t / sigma:
//   keys left of the wave's rows (j < r0):  q.k + (j - r0) / sigma,
// in log2 units log2(e) (q.k + koff / sigma) + log2(e) (j0 - r0) / sigma for
// key j = j0 + koff of a stage starting at j0.  The first term comes out of
// the matrix op itself, whose accumulator starts at koff / sigma (a register
// constant of the lane) instead of zero; the second is one number per stage,
// folded into the exponent's offset.  Such a stage then costs the softmax no
// more than an unbiased one.  The diagonal stage (j0 = r0) and, without the
// causal mask, the stages right of it (j > i: q.k - (j - i) / sigma, shifted
// by t / sigma: q.k - (j - r0) / sigma + 2 t / sigma) add a per-key term, as
// does the mask of keys past the end.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "plsh_device.h"
#include "plsh_hip_status.h"
#include "plsh_kernels.h"

namespace plsh {
namespace dev {

namespace {

constexpr int kExWaves = 4;  // waves per workgroup, 32 rows each
constexpr int kExRing = 3;   // K/V ring stages
constexpr int kExKeys = 32;  // keys per stage
// register budget: three waves per SIMD at D = 128 (168 registers, 48 KB of
// LDS per workgroup), four at D = 64
template <int D>
constexpr int kExWavesPerEu = D == 64 ? 4 : 3;

template <int Q>
struct ExSlot {
  static constexpr int value = Q;
};

// 16-byte chunk swizzle of K rows (and of the staged O rows): the operand
// reads have lanes 0..31 read keys 0..31 at one chunk, and this XOR keeps the
// lanes that share an LDS cycle on distinct banks
template <int D>
__device__ __forceinline__ int ex_kswz(int key) {
  return D == 128 ? (key & 15) : ((key >> 1) & 7);
}
template <int D>
__device__ __forceinline__ uint32_t ex_kpos(int key, int chunk) {
  return (uint32_t)(key * 2 * D + ((chunk ^ ex_kswz<D>(key)) << 4));
}

}  // namespace

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kExWaves, 64 * kExWaves),
                          amdgpu_waves_per_eu(kExWavesPerEu<D>, kExWavesPerEu<D>)))
void exact_fwd_kernel(ExactArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t kv[kExRing][2][kExKeys * D];
  const int n = a.n;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int t = lane & 31, hf = lane >> 5;

  // ---- workgroup -> (batch, head, 128-row block).  Causal: the blocks with
  // the most keys first.  Workgroups are dealt to the 8 XCDs round-robin;
  // when the (batch, KV head) pairs split evenly over them, each XCD takes
  // whole pairs and runs the query heads of a pair's GQA group next to each
  // other, so the workgroups resident on an XCD stream the same K/V rows
  // through its L2.  Otherwise consecutive workgroups take consecutive
  // (batch, head) pairs.
  const int grp = a.heads / a.kv_heads;
  const int BKV = a.batch * a.kv_heads;
  const int p = blockIdx.x;
  int bkv, hq, gi;
  if ((BKV & 7) == 0) {
    const int m = p >> 3, per = BKV >> 3;
    hq = m % grp;
    const int mp = m / grp;
    bkv = (p & 7) + 8 * (mp % per);
    gi = mp / per;
  } else {
    const int BH = a.batch * a.heads;
    const int bh = p % BH;
    gi = p / BH;
    bkv = bh / grp;
    hq = bh % grp;
  }
  const int g = CAUSAL ? a.groups - 1 - gi : gi;
  const int b = bkv / a.kv_heads, kvh = bkv % a.kv_heads;
  const int h = kvh * grp + hq;
  const int r0 = g * 128 + 32 * wave;  // this wave's first row
  const bool active = r0 < n;
  const float slope2 = a.slope2[h];              // log2(e) / sigma
  const float slope = slope2 * 0.69314718056f;   // 1 / sigma

  const uint16_t *Q = (const uint16_t *)a.q + ((int64_t)b * a.heads + h) * n * D;
  const char *Kb = (const char *)((const uint16_t *)a.k + ((int64_t)b * a.kv_heads + kvh) * n * D);
  const char *Vb = (const char *)((const uint16_t *)a.v + ((int64_t)b * a.kv_heads + kvh) * n * D);

  // ---- the lane's Q fragments (B operand: query t, dims 16 c + 8 hf .. + 7)
  // straight from global memory; they land by the first stage's wait
  constexpr int NC = D / 16;  // QK^T products per stage
  bf16x8 qf[NC];
  if (active) {
    const uint16_t *qrow = Q + (int64_t)min(r0 + t, n - 1) * D + 8 * hf;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = *(const bf16x8 *)(qrow + 16 * c);
  }

  // ---- K/V stages [0, nst): keys [0, U1) for the workgroup; this wave
  // computes stages [sa, sb).  A K tile is 32 whole rows (K-row swizzle), a V
  // tile 32 keys x D as 64-byte pieces per 32 dims (vpiece128); wave w copies
  // the tile's 16-byte chunks [w D, (w + 1) D).  Keys past the end read as
  // zeros through the buffer resource and are masked.
  const int U1 = CAUSAL ? min(n, g * 128 + 128) : n;
  const int nst = (U1 + kExKeys - 1) / kExKeys;
  // The bias is largest at a row's own key, so the stream starts at the
  // workgroup's last diagonal tile dt and runs down to key 0 (causal: the
  // whole stream; a wave's tiles are stages [sa, nst)), then, without the
  // causal mask, on from dt + 1 to the end: each row meets its largest
  // biases within its first stages and the running max rarely rises later.
  const int dt = min(g * 4 + 3, nst - 1);
  auto key_tile = [&](int st) { return st <= dt ? dt - st : st; };
  const int sa = !active ? nst : CAUSAL ? nst - 1 - r0 / kExKeys : 0;
  const int sb = !active ? 0 : nst;
  constexpr int CPR = D / 8;   // 16-byte chunks per row
  constexpr int NCW = D / 64;  // copy instructions per wave, tile and stage
  const uint32_t kv_lds = lds_addr(&kv[0][0][0]);
  const i32x4 krs = buffer_rsrc(Kb, (uint32_t)n * (2 * D)), vrs = buffer_rsrc(Vb, (uint32_t)n * (2 * D));
  uint32_t ck_off[NCW], cv_off[NCW];
#pragma unroll
  for (int j = 0; j < NCW; ++j) {
    const int ci = wave * D + 64 * j + lane;  // the lane's chunk position in the tile
    ck_off[j] = (uint32_t)((ci / CPR) * (2 * D) + 16 * ((ci % CPR) ^ ex_kswz<D>(ci / CPR)));
    const int P = 16 * ci;
    const int vkey = (P >> 6) & 31;
    cv_off[j] = (uint32_t)(vkey * (2 * D) + 16 * (4 * (P >> 11) + (((P >> 4) & 3) ^ (((vkey >> 2) & 1) << 1))));
  }
  auto issue_stage = [&](int st, int q) {  // q = st % kExRing
    const uint32_t soff = (uint32_t)(kExKeys * key_tile(st)) * (2 * D);
#pragma unroll
    for (int j = 0; j < NCW; ++j) {
      const uint32_t dst = kv_lds + (uint32_t)(2 * q) * (kExKeys * D * 2) + 16 * (wave * D + 64 * j);
      dma16_buf(krs, ck_off[j], soff, dst);
      dma16_buf(vrs, cv_off[j], soff, dst + kExKeys * D * 2);
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
  // key offset of accumulator r inside a stage, and the accumulators' start
  auto koff = [&](int r) { return 8 * (r >> 2) + 4 * hf + (r & 3); };
  floatx16 kinit;
#pragma unroll
  for (int r = 0; r < 16; ++r) kinit[r] = slope * (float)koff(r);

  // diagonal stage: bit r set when key offset koff(r) is at or before the
  // lane's row
  uint32_t dmask = 0u;
#pragma unroll
  for (int r = 0; r < 16; ++r) dmask |= (uint32_t)(koff(r) <= t) << r;
  // K operand of product c: key t, chunk 2 c + hf
  uint32_t kofs[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) kofs[c] = ex_kpos<D>(t, 2 * c + hf);
  // V operand (transposing reads): lane (g = l / 16, r = l % 16) names key
  // 4 (g / 2) + r / 4 (+ 16 c + 8 e) at dims 32 b + 16 (g % 2) + 4 (r % 4);
  // every read of a stage is this address plus an immediate
  uint32_t vofs;
  {
    const int gg = lane >> 4, rr = lane & 15;
    const int kk = 4 * (gg >> 1) + (rr >> 2);
    const int x = 2 * (gg & 1) + ((rr & 3) >> 1);  // 16-byte chunk inside the 64-byte piece
    vofs = (uint32_t)(kk * 64 + ((x ^ (((kk >> 2) & 1) << 1)) << 4) + 8 * (rr & 1));
  }

  // S^T + koff / sigma for the stage in ring slot Q0 (the K fragment reads of
  // each half issued ahead of its products)
  auto qk_tile = [&](auto s0, floatx16 &SA) {
    const char *ka = (const char *)kv[decltype(s0)::value][0];
    constexpr int KG = NC / 2;  // fragments per group
    SA = kinit;
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

  // raises the running max when the tile's largest logit (log2 units, for
  // the lane: mx) exceeds it by more than 2^8 (the result does not depend on
  // the max used), for both lanes of the row
  auto raise_max = [&](float mx) {
    if (__any(mx > m2 + 8.0f)) {
      mx = max3f(mx, other_half_f(mx, lane), mx);
      const bool need = mx > m2 + 8.0f;
      const float mnew = need ? mx : m2;
      const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NB; ++db) oacc[db] *= alpha;
      m2 = mnew;
    }
  };

  // softmax and PV of stage st (ring slot slotc), logits in SA
  auto finish_tile = [&](int st, auto slotc, const floatx16 &SA) {
    const char *vt = (const char *)kv[decltype(slotc)::value][1];
    const int j0 = kExKeys * key_tile(st);
    const bool plain = j0 < r0 && j0 + kExKeys <= n;
    // the tile's logits in log2 units are fma(x, sc, off)
    floatx16 x = SA;
    float sc, off;
    const float tb = slope2 * (float)(j0 - r0);
    if (__builtin_amdgcn_readfirstlane(plain)) {
      // keys left of the wave's rows: log2(e) SA + slope2 (j0 - r0)
      sc = kLog2e;
      off = tb;
    } else {
      // the diagonal stage, the stages right of it (no causal mask) and the
      // last stage (keys past the end): a term per key.  Key offset koff(r)
      // is c_r + 4 hf with c_r a constant of r; keys after the row (no causal
      // mask) take -tb + 2 slope2 (t - koff)
      const float eb = -tb + 2.0f * slope2 * (float)(t - 4 * hf), s2 = 2.0f * slope2;
      auto right = [&](int r) { return fmaf(-(float)(8 * (r >> 2) + (r & 3)), s2, eb); };
      if (j0 == r0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool left = (dmask >> r) & 1u;
          x[r] = fmaf(x[r], kLog2e, left ? tb : CAUSAL ? -INFINITY : right(r));
        }
      } else if (CAUSAL || j0 < r0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = fmaf(x[r], kLog2e, tb);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = fmaf(x[r], kLog2e, right(r));
      }
      if (!CAUSAL && j0 + kExKeys > n) {
        const int lim = n - j0 - 4 * hf;  // c_r >= lim: the key is past the end
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = 8 * (r >> 2) + (r & 3) >= lim ? -INFINITY : x[r];
      }
      sc = 1.0f;
      off = 0.0f;
    }
    float mx = max3f(max3f(x[0], x[1], x[2]), max3f(x[3], x[4], x[5]), max3f(x[6], x[7], x[8]));
    mx = max3f(mx, max3f(x[9], x[10], x[11]), max3f(x[12], x[13], x[14]));
    mx = max3f(mx, x[15], x[15]);
    raise_max(fmaf(mx, sc, off));
    // P = 2^(logit - m2), rounded to bf16 in pairs; the row sum adds exactly
    // the rounded weights that enter PV
    const float o2 = off - m2;
    u32x4 pw[2];
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const floatx2 pf = {__builtin_amdgcn_exp2f(fmaf(x[r], sc, o2)), __builtin_amdgcn_exp2f(fmaf(x[r + 1], sc, o2))};
      const bf16x2 pb = __builtin_convertvector(pf, bf16x2);
      pw[r >> 3][(r & 7) >> 1] = __builtin_bit_cast(uint32_t, pb);
      lsum = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, lsum, false);
    }

    // O^T += V^T P^T, two 16-key chunks, V^T by transposing reads (each
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

  // One stage per barrier: stage st waits for its own copies only (those of
  // st + 1, issued after them, may still be in flight: copies complete in
  // issue order), refills the slot of stage st - 1 (every wave is past it)
  // with st + 2, and computes its tile.
  auto single = [&](int st, auto s0) {
    if (st + 1 < nst) PLSH_WAIT_VM_LGKM0(2 * NCW);
    else PLSH_WAIT_VM_LGKM0(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (st + 2 < nst) issue_stage(st + 2, (decltype(s0)::value + 2) % kExRing);
    if (st >= sa && st < sb) {
      floatx16 SA;
      qk_tile(s0, SA);
      finish_tile(st, s0, SA);
    }
  };
  // the first stage's wait, and with it the Q fragments, ahead of the loop:
  // the compiler, which does not see the copies, then counts those loads as
  // done inside it (else it waits on them at every tile, and with them on
  // the later stages' copies)
  if (nst > 1) PLSH_WAIT_VM_LGKM0(2 * NCW);
  else PLSH_WAIT_VM_LGKM0(0);
#pragma unroll
  for (int c = 0; c < NC; ++c) asm volatile("" : "+v"(qf[c]));
  for (int st0 = 0; st0 < nst; st0 += 3) {
    single(st0, ExSlot<0>{});
    if (st0 + 1 < nst) single(st0 + 1, ExSlot<1>{});
    if (st0 + 2 < nst) single(st0 + 2, ExSlot<2>{});
  }

  // ---- O = acc / l, rounded to bf16, staged in the two ring slots of the
  // last stage's predecessors (every wave is past both) and stored whole rows
  // per instruction
  if (!active) return;
  const float ltot = lsum + other_half_f(lsum, lane);
  const float inv = 1.0f / ltot;
  const int last = nst > 0 ? (nst - 1) % 3 : 2;
  char *ob = (char *)kv[(last + 1 + (wave >> 1)) % 3][0] + (wave & 1) * 32 * D * 2;
#pragma unroll
  for (int db = 0; db < NB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // dims 32 db + 8 j + 4 hf .. + 3: half hf of chunk 4 db + j
      const bf16x2 h0 = __builtin_convertvector((floatx2{oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv}), bf16x2);
      const bf16x2 h1 =
          __builtin_convertvector((floatx2{oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv}), bf16x2);
      *(u32x2 *)(ob + ex_kpos<D>(t, 4 * db + j) + 8 * hf) =
          u32x2{__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1)};
    }
  wave_sync();
  uint16_t *O = (uint16_t *)a.out + ((int64_t)b * a.heads + h) * n * D;
#pragma unroll
  for (int c0 = 0; c0 < 32 * CPR; c0 += 64) {
    const int row = (c0 + lane) / CPR, ch = (c0 + lane) % CPR;
    const u32x4 val = *(const u32x4 *)(ob + ex_kpos<D>(row, ch));
    const int i = r0 + row;
    if (i < n) *(u32x4 *)(O + (int64_t)i * D + 8 * ch) = val;
  }
}

}  // namespace dev

plsh_status launch_exact(const dev::ExactArgs &a, int d, int causal, hipStream_t st, const char *who) {
  const dim3 grid((unsigned)((int64_t)a.groups * a.batch * a.heads)), block(64 * 4);
  auto *tm = timer_slot();
  if (d == 64) {
    if (causal) launch_k(dev::exact_fwd_kernel<64, true>, grid, block, 0, st, tm, a);
    else launch_k(dev::exact_fwd_kernel<64, false>, grid, block, 0, st, tm, a);
  } else {
    if (causal) launch_k(dev::exact_fwd_kernel<128, true>, grid, block, 0, st, tm, a);
    else launch_k(dev::exact_fwd_kernel<128, false>, grid, block, 0, st, tm, a);
  }
  return launch_check(who);
}

}  // namespace plsh
