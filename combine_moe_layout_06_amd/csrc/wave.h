// Wave-level helpers for gfx950 (CDNA4): 64-lane wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_WAVE 64

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Streaming accesses: data touched once per call bypass the caches' normal
// retention (nontemporal hint) unless built with MOE_TEMPORAL_ROWS.
template <typename V>
__device__ __forceinline__ V stream_load(const V* p) {
#ifdef MOE_TEMPORAL_ROWS
  return *p;
#else
  return __builtin_nontemporal_load(p);
#endif
}
template <typename V>
__device__ __forceinline__ void stream_store(V v, V* p) {
#ifdef MOE_TEMPORAL_ROWS
  *p = v;
#else
  __builtin_nontemporal_store(v, p);
#endif
}

// Two fp32 values rounded to bf16 (nearest, ties to even) and packed, `lo`
// in the low half, with gfx950's packed convert (v_cvt_pk_bf16_f32). On the
// device it gives the integer rounding to nearest even of the fp32 pattern
// for every non-NaN value, infinities, overflow and subnormals included, and
// a NaN for a NaN (tests/hip/convert_sweep.hip compares all 2^32 patterns).
typedef __bf16 moe_bf16x2 __attribute__((ext_vector_type(2)));
typedef float moe_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const moe_f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, moe_bf16x2));
}

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

// DPP lane moves inside 16-lane rows (gfx9 DPP controls):
//   0xB1 quad_perm(1,0,3,2)   0x4E quad_perm(2,3,0,1)
//   0x141 row_half_mirror     0x140 row_mirror
// Applying an associative, commutative op after each of the four moves in
// that order leaves the op over the whole row in every lane of the row.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = dpp_u32<CTRL>((uint32_t)v);
  const uint32_t hi = dpp_u32<CTRL>((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  return __longlong_as_double((long long)dpp_u64<CTRL>((uint64_t)__double_as_longlong(v)));
}

// Value of lane (l ^ 16) and of lane (l ^ 32), with gfx950's row and half
// swaps (checked on the device: permlane16_swap(v, v) returns v of the lane
// itself and of the neighbouring row, in an order that depends on the row's
// parity; permlane32_swap likewise for the two halves of the wave).
// Keep the explicit select of the partner's element: a commutative op
// applied directly to the two results (e.g. r[0] + r[1]) was compiled into
// r[0] + r[0] by this toolchain when both operands are the same value.
__device__ __forceinline__ uint32_t xor16_u32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return (lane_id() & 16) ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t xor32_u32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (lane_id() & 32) ? r[0] : r[1];
}
__device__ __forceinline__ float xor16_f32(float v) { return __uint_as_float(xor16_u32(__float_as_uint(v))); }
__device__ __forceinline__ float xor32_f32(float v) { return __uint_as_float(xor32_u32(__float_as_uint(v))); }
__device__ __forceinline__ uint64_t xor16_u64(uint64_t v) {
  return ((uint64_t)xor16_u32((uint32_t)(v >> 32)) << 32) | xor16_u32((uint32_t)v);
}
__device__ __forceinline__ uint64_t xor32_u64(uint64_t v) {
  return ((uint64_t)xor32_u32((uint32_t)(v >> 32)) << 32) | xor32_u32((uint32_t)v);
}
__device__ __forceinline__ double xor16_f64(double v) {
  return __longlong_as_double((long long)xor16_u64((uint64_t)__double_as_longlong(v)));
}
__device__ __forceinline__ double xor32_f64(double v) {
  return __longlong_as_double((long long)xor32_u64((uint64_t)__double_as_longlong(v)));
}

// Wave-wide reductions, all in vector registers: four DPP steps inside each
// 16-lane row, then the row and half swaps. Every lane gets the result.
__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  v = fmaxf(v, xor16_f32(v));
  return fmaxf(v, xor32_f32(v));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  v += xor16_f32(v);
  return v + xor32_f32(v);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  v += dpp_f64<0x141>(v);
  v += dpp_f64<0x140>(v);
  v += xor16_f64(v);
  return v + xor32_f64(v);
}
