// Combine on gfx950: bring each token's k expert outputs back and sum them,
// weighted by the router scores.
//
// Source: glossary "Expert Parallelism" (polydesk.ai), "Le pattern de
// communication all-to-all", Phase 2 (results return to the token's origin
// and are summed with the router weights); hyper.ai story on Hybrid-EP (the
// combine operator reduces the returned expert outputs).
//
//   out[t, :] = bf16( fma chain over j = 0..k-1 of w[t,j] * y[dst_row[t,j], :] )
//
// One 64-lane wave per (token, column part). For a compile-time k the wave
// issues the loads of all k rows (16 bytes per lane each) before the first
// FMA, so k x 1 KiB per wave are in flight; the fp32 accumulators are
// rounded once to bf16 (nearest even) and stored with one 16-byte store.

#include "kernels.h"
#include "wave.h"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;

#ifndef MOE_COMBINE_U8
#define MOE_COMBINE_U8 2   // 16-byte chunks per lane per step when k = 8
#endif

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;  // NaN
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void fma_row(float (&acc)[8], float w, const u32x4& v) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc[2 * q] = __builtin_fmaf(w, bf16_lo(v[q]), acc[2 * q]);
    acc[2 * q + 1] = __builtin_fmaf(w, bf16_hi(v[q]), acc[2 * q + 1]);
  }
}

__device__ __forceinline__ u32x4 pack_row(const float (&acc)[8]) {
  u32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = bf16_rne(acc[2 * q]) | (bf16_rne(acc[2 * q + 1]) << 16);
  return r;
}

// K > 0: compile-time top-k; all K rows are loaded before accumulating.
template <int K, int U>
__global__ __launch_bounds__(256) void combine_kernel(
    int T, int nch, int parts, int cpp, int num_rows, const u32x4* __restrict__ y,
    const int32_t* __restrict__ dst_row, const float* __restrict__ w,
    u32x4* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (gw >= T * parts) return;
  const int t = gw / parts;
  const int c0 = (gw - t * parts) * cpp;
  const int cnt = min(cpp, nch - c0);
  const int my_dst = lane < K ? dst_row[(size_t)t * K + lane] : -1;
  const float my_w = lane < K ? w[(size_t)t * K + lane] : 0.0f;

  int d[K];
  float wj[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    d[j] = read_lane(my_dst, j);
    wj[j] = read_lane(my_w, j);
    if (d[j] >= num_rows) d[j] = -1;
  }
  u32x4* dst = out + (size_t)t * nch + c0;

  for (int base = 0; base < cnt; base += MOE_WAVE * U) {
    u32x4 v[K][U];
#pragma unroll
    for (int j = 0; j < K; ++j) {
#pragma unroll
      for (int u = 0; u < U; ++u) v[j][u] = u32x4{0u, 0u, 0u, 0u};
      const u32x4* row = y + (size_t)(d[j] < 0 ? 0 : d[j]) * nch + c0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = base + u * MOE_WAVE + lane;
        if (d[j] >= 0 && c < cnt) v[j][u] = stream_load(row + c);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = base + u * MOE_WAVE + lane;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < K; ++j)
        if (d[j] >= 0) fma_row(acc, wj[j], v[j][u]);
      if (c < cnt) stream_store(pack_row(acc), dst + c);
    }
  }
}

// Any k: rows are loaded one slot at a time.
__global__ __launch_bounds__(256) void combine_kernel_any_k(
    int T, int k, int nch, int parts, int cpp, int num_rows, const u32x4* __restrict__ y,
    const int32_t* __restrict__ dst_row, const float* __restrict__ w,
    u32x4* __restrict__ out) {
  constexpr int U = 4;
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (gw >= T * parts) return;
  const int t = gw / parts;
  const int c0 = (gw - t * parts) * cpp;
  const int cnt = min(cpp, nch - c0);
  const int my_dst = lane < k ? dst_row[(size_t)t * k + lane] : -1;
  const float my_w = lane < k ? w[(size_t)t * k + lane] : 0.0f;
  u32x4* dst = out + (size_t)t * nch + c0;

  for (int base = 0; base < cnt; base += MOE_WAVE * U) {
    float acc[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[u][q] = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int d = read_lane(my_dst, j);
      const float wj = read_lane(my_w, j);
      if (d < 0 || d >= num_rows) continue;
      const u32x4* row = y + (size_t)d * nch + c0;
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = base + u * MOE_WAVE + lane;
        v[u] = u32x4{0u, 0u, 0u, 0u};
        if (c < cnt) v[u] = stream_load(row + c);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) fma_row(acc[u], wj, v[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = base + u * MOE_WAVE + lane;
      if (c < cnt) stream_store(pack_row(acc[u]), dst + c);
    }
  }
}

template <int K, int U>
void launch_fixed(dim3 grid, hipStream_t stream, int T, int nch, int parts, int cpp,
                  int num_rows, const void* y, const int32_t* dst_row, const float* w,
                  void* out) {
  hipLaunchKernelGGL((combine_kernel<K, U>), grid, dim3(256), 0, stream, T, nch, parts, cpp,
                     num_rows, static_cast<const u32x4*>(y), dst_row, w,
                     static_cast<u32x4*>(out));
}

}  // namespace

hipError_t launch_combine(int T, int H, int k, int num_rows, const void* y,
                          const int32_t* dst_row, const float* w, void* out,
                          hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int nch = H / 8;
  int parts = T > 0 ? (kTargetWaves + T - 1) / T : 1;
  parts = max(1, min(parts, nch / MOE_WAVE));
  int cpp = (nch + parts - 1) / parts;
  cpp = (cpp + MOE_WAVE - 1) / MOE_WAVE * MOE_WAVE;
  parts = (nch + cpp - 1) / cpp;
  const dim3 grid((T * parts + kWavesPerBlock - 1) / kWavesPerBlock);
  switch (k) {
    case 1: launch_fixed<1, 4>(grid, stream, T, nch, parts, cpp, num_rows, y, dst_row, w, out); break;
    case 2: launch_fixed<2, 4>(grid, stream, T, nch, parts, cpp, num_rows, y, dst_row, w, out); break;
    case 4: launch_fixed<4, 2>(grid, stream, T, nch, parts, cpp, num_rows, y, dst_row, w, out); break;
    case 6: launch_fixed<6, 1>(grid, stream, T, nch, parts, cpp, num_rows, y, dst_row, w, out); break;
    case 8: launch_fixed<8, MOE_COMBINE_U8>(grid, stream, T, nch, parts, cpp, num_rows, y, dst_row, w, out); break;
    default:
      hipLaunchKernelGGL(combine_kernel_any_k, grid, dim3(256), 0, stream, T, k, nch, parts,
                         cpp, num_rows, static_cast<const u32x4*>(y), dst_row, w,
                         static_cast<u32x4*>(out));
  }
  return hipGetLastError();
}

}  // namespace moe
