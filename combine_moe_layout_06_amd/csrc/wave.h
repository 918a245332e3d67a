// Wave-level helpers for gfx950 (CDNA4): 64-lane wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_WAVE 64

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Number of set bits of `mask` in lanes below the calling lane.
__device__ __forceinline__ int count_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t wave_ballot(bool p) {
  return __builtin_amdgcn_ballot_w64(p);
}

// Lanes whose `key` equals the calling lane's key, among lanes where
// `active` holds. Keys are compared on their low `nbits` bits through one
// ballot per bit; the result is identical in every lane of a peer group.
__device__ __forceinline__ uint64_t peer_mask(uint32_t key, bool active, int nbits) {
  uint64_t peers = wave_ballot(active);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1u;
    const uint64_t ones = wave_ballot(bit);
    peers &= bit ? ones : ~ones;
  }
  return active ? peers : 0ull;
}

// Uniform value of lane `src` (src must be wave-uniform).
__device__ __forceinline__ int read_lane(int v, int src) {
  return __builtin_amdgcn_readlane(v, src);
}
__device__ __forceinline__ float read_lane(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

__device__ __forceinline__ int ceil_log2(int n) {
  int b = 0;
  while ((1 << b) < n) ++b;
  return b;
}
