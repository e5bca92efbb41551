// plsh_exact.hip -- dense exact-ALiBi attention (the comparator) for gfx950.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "plsh_hip_status.h"
#include "plsh_kernels.h"
#include "plsh_mfma16.h"

namespace plsh {
namespace dev {


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

}  // namespace dev

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

}  // namespace plsh
