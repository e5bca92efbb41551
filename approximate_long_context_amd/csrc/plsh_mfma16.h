// plsh_mfma16.h -- the LDS ring, swizzles and tile constants of the kernels
// with 16-row waves (plsh_mfma16.hip, plsh_exact.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plsh_device.h"

namespace plsh {
namespace dev {

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


}  // namespace dev
}  // namespace plsh
