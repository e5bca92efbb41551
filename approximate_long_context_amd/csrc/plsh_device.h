// plsh_device.h -- device helpers and the block-edge record format shared by
// the attention kernels of libplsh (plsh_attention.hip, plsh_fwd.hip).
//
// "Positional LSH: Binary Block Matrix Approximation for Attention with Linear
// Biases", Methodology §1 (blocks of a random-binning hash) and §3 (Theorem
// 2.2: the estimator as s block-local attentions fused into one ratio of sums).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace plsh {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

constexpr int kMaxHeadsArg = 128;
constexpr float kLog2e = 1.4426950408889634f;

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
__device__ __forceinline__ double other_half_d(double x, int lane) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint64_t lo = other_half((uint32_t)b, lane), hi = other_half((uint32_t)(b >> 32), lane);
  return __longlong_as_double((long long)(lo | (hi << 32)));
}

// bits 1..t of a 32-bit mask (t in [0, 31])
__device__ __forceinline__ uint32_t bits_1_to(int t) {
  return t == 0 ? 0u : ((0xFFFFFFFFu >> (31 - t)) & ~1u);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

// V tiles (the estimator's forward kernels) are not stored row by row: the
// 64-byte piece of key `key` holding dims 32 m .. 32 m + 31 (chunks 4 m ..
// 4 m + 3) lies at m * 2048 + key * 64, its chunk pairs swapped when bit 2 of
// the key is set.  Each group of four copy lanes still reads one 64-byte
// segment of a row; the transposing 8-byte reads of a 16-dim block (32
// lanes: keys 0..7, two chunks, two halves) cover 256 distinct bytes; and
// the reads of all eight dim blocks differ by immediate offsets, so they need
// two address registers instead of eight (with eight, the compiler recycled
// the operand registers and serialised every read behind a matrix op).
__device__ __forceinline__ uint32_t vpiece128(int key, int chunk) {
  return (uint32_t)((chunk >> 2) * 2048 + key * 64 + (((chunk & 3) ^ (((key >> 2) & 1) << 1)) << 4));
}

// LDS address of a pointer into LDS (the generic-to-LDS cast; on static
// shared variables it folds to a constant)
__device__ __forceinline__ uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)(lds_void_t *)p; }

// Direct global->LDS copy of 16 bytes per lane: lane l's bytes land at LDS
// address lds_base + 16 l (lds_base wave-uniform).  Issued as inline assembly so that
// the ring's only ordering is the explicit vmcnt wait + barrier of each stage
// (the compiler would otherwise wait for every outstanding copy before any
// LDS read, since it cannot tell which ring stage a copy targets).
__device__ __forceinline__ void dma16(const void *gsrc, uint32_t lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "s"(m0)
               : "memory", "m0");
}

// Buffer resource (gfx9 descriptor) for `bytes` bytes from `base`: raw
// addressing, no stride; reads at offsets past the end return zeros.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 buffer_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int32_t)((uint32_t)(a >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane((int32_t)bytes);
  r[3] = 0x00020000;  // 32-bit data format, the untyped loads ignore it
  return r;
}

// The same copy as dma16 through a buffer resource: lane l's 16 bytes at
// offset voff (lane) + soff (wave-uniform) of the resource land at
// lds_base + 16 l; offsets past the resource's end give zeros.  Only the
// scalar offset changes between the stages of a ring, so a stage's copies
// take no vector address arithmetic.
__device__ __forceinline__ void dma16_buf(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "s"(m0)
               : "memory", "m0");
}

// s_waitcnt with vmcnt <= v and lgkmcnt == 0 (gfx9 encoding)
#define PLSH_WAIT_VM_LGKM0(v) __builtin_amdgcn_s_waitcnt(((v) & 15) | (((v) >> 4) << 14) | (7 << 4))

// ---------------------------------------------------------------------------
// Block-edge records: one per (head, 32-row group), written by the pre-pass.
//   [0, 16)              int32 nnz, U0w, U1w, 0: number of samples with a block
//                        start inside the group's rows; the group's key range
//                        [U0w, U1w) (32-aligned)
//   [16, +8 E)           (lead, W) of every sample sorted by (lead, k), then
//                        16 sentinels (0x7FFFFFFF, 0); E = s + 16 rounded up
//                        to even, so that each list is whole 16-byte chunks;
//                        bit t of W is set when row r0 + t's block of that
//                        sample starts at the lead (no block start in rows
//                        r0 + 1 .. r0 + t)
//   [.., +8 E)           (trail, W) sorted by (trail, k), 16 sentinels
//                        (written by the non-causal pass only); bit t of W is
//                        set when row r0 + t's block ends at the trail (no
//                        block start in rows r0 + t + 1 .. r0 + 31)
//   [.., +1024)          multiplicity of the diagonal tile: byte [t][u] is
//                        c(r0 + t, r0 + u), zero where j > i (causal) or j >= n
// ---------------------------------------------------------------------------
constexpr int kSentinels = 16;
__host__ __device__ constexpr int ev_count(int s) { return (s + kSentinels + 1) & ~1; }
__host__ __device__ constexpr size_t rec_evl_off() { return 16; }
__host__ __device__ constexpr size_t rec_evt_off(int s) { return 16 + (size_t)8 * ev_count(s); }
__host__ __device__ constexpr size_t rec_diag_off(int s) { return 16 + (size_t)16 * ev_count(s); }
__host__ __device__ constexpr size_t rec_bytes(int s) { return rec_diag_off(s) + 1024; }
// samples per head of the MFMA paths: the forward kernel (byte counters and
// per-wave edge lists up to 255) and the backward kernels (124)
constexpr int kMaxFwdSamples = 255;
constexpr int kMaxMfmaSamples = 124;

// max of three finite floats in one instruction (the compiler's max of
// floats first quiets each operand's NaN payload, one extra instruction per
// operand; logits are never NaN)
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// x from lane l ^ 16 (within each 32-lane half; ds_swizzle bit mode, no
// memory access)
__device__ __forceinline__ float xor16_f(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
}

// four byte counters for keys k, k + 1, k + 2, k + 3: 1 in byte r when
// r >= d, i.e. the keys at or after an edge d keys past k
__device__ __forceinline__ uint32_t step4(int d) {
  const int dc = min(max(d, 0), 4);
  return dc < 4 ? (0x01010101u << (8 * dc)) : 0u;
}

__host__ __device__ constexpr size_t ev_wave_bytes(int s, bool causal) {
  return (size_t)(causal ? 8 : 16) * ev_count(s);
}

}  // namespace dev
}  // namespace plsh
