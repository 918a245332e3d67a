// Top-k and group-limited top-k routing on gfx950.
//
// One 64-lane wave per token; lane l holds experts l, l+64, l+128, ...
// Sources: hyper.ai story on NVIDIA Hybrid-EP (each token activates only k
// experts); DeepEP article (ai-master.dev), section "Group-limited gating
// algorithm" (the choice is restricted to a few expert groups); glossary
// "Expert Parallelism" (polydesk.ai), "Le pattern de communication
// all-to-all", Phase 2 (outputs are weighted by the router scores).
//
// Precision: sigmoid and exp run in fp64 and each result is rounded once to
// fp32; selection keys are fp32; weight sums run in fp64.

#include "kernels.h"
#include "wave.h"

namespace moe {
namespace {

constexpr int kRouteWaves = 4;  // tokens per 256-thread block

// Monotone map fp32 -> uint32 (larger float -> larger integer); -0 and +0
// compare equal, as they do as floats.
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  uint32_t b = __float_as_uint(v);
  if ((b & 0x7FFFFFFFu) == 0u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Candidate (key desc, expert asc) packed so that a larger integer wins.
// Zero means "no candidate": every finite key maps above it.
__device__ __forceinline__ uint64_t candidate(float key, int e) {
  return ((uint64_t)ordered_bits(key) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = __shfl_xor((unsigned long long)v, off);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(
    int T, int E, int k, const float* __restrict__ logits,
    const float* __restrict__ bias, int sigmoid, int G, int kg,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  __shared__ float s_key[kRouteWaves][MOE_MAX_EXPERTS];
  __shared__ float s_gscore[kRouteWaves][MOE_MAX_GROUPS];
  __shared__ int s_gkeep[kRouteWaves][MOE_MAX_GROUPS];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRouteWaves + wave;
  const bool live = t < T;

  float key[VPL], score[VPL];
  bool ok[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    ok[i] = live && e < E;
    const float l = ok[i] ? logits[(size_t)t * E + e] : 0.0f;
    const float s = sigmoid ? (float)(1.0 / (1.0 + exp(-(double)l))) : l;
    score[i] = s;
    key[i] = (bias != nullptr && ok[i]) ? s + bias[e] : s;
  }

  if (G > 1) {  // G is uniform over the block: the barriers below are safe
    const int gs = E / G;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (ok[i]) s_key[wave][lane + 64 * i] = key[i];
    __syncthreads();
    if (live && lane < G) {
      // group score: sum of the two largest keys, largest first
      float m1 = -INFINITY, m2 = -INFINITY;
      for (int q = 0; q < gs; ++q) {
        const float v = s_key[wave][lane * gs + q];
        if (v > m1) { m2 = m1; m1 = v; }
        else if (v > m2) { m2 = v; }
      }
      s_gscore[wave][lane] = gs == 1 ? m1 : m1 + m2;
    }
    __syncthreads();
    if (live && lane < G) {
      const float mine = s_gscore[wave][lane];
      int rank = 0;
      for (int q = 0; q < G; ++q) {
        const float o = s_gscore[wave][q];
        rank += (o > mine) || (o == mine && q < lane);
      }
      s_gkeep[wave][lane] = rank < kg;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (ok[i]) ok[i] = s_gkeep[wave][(lane + 64 * i) / gs] != 0;
  }
  if (!live) return;  // whole wave; no barrier follows

  int my_e = -1;
  float my_score = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
    float best_score = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      if (!ok[i]) continue;
      const uint64_t c = candidate(key[i], lane + 64 * i);
      if (c > best) { best = c; best_score = score[i]; }
    }
    const uint64_t win = wave_max_u64(best);
    const int e_win = (int)(0xFFFFFFFFu - (uint32_t)win);
    const int owner = e_win & 63;
    const float s_win = read_lane(best_score, owner);
    if (lane == owner) {
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (lane + 64 * i == e_win) ok[i] = false;
    }
    if (lane == j) { my_e = e_win; my_score = s_win; }
  }

  double u;
  if (sigmoid) {
    u = lane < k ? (double)my_score : 0.0;
  } else {
    const float m = wave_max_f32(lane < k ? my_score : -INFINITY);
    u = lane < k ? exp((double)my_score - (double)m) : 0.0;
  }
  const double total = wave_sum_f64(u);
  if (lane < k) {
    idx_out[(size_t)t * k + lane] = my_e;
    w_out[(size_t)t * k + lane] = (float)(u / total);
  }
}

}  // namespace

hipError_t launch_route(int T, int E, int k, const float* logits, const float* bias,
                        int sigmoid, int G, int kg, int32_t* idx_out, float* w_out,
                        hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + kRouteWaves - 1) / kRouteWaves), block(256);
  if (E <= 64)
    hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, stream, T, E, k, logits, bias, sigmoid, G, kg, idx_out, w_out);
  else if (E <= 128)
    hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, stream, T, E, k, logits, bias, sigmoid, G, kg, idx_out, w_out);
  else if (E <= 256)
    hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, stream, T, E, k, logits, bias, sigmoid, G, kg, idx_out, w_out);
  else
    hipLaunchKernelGGL(route_kernel<8>, grid, block, 0, stream, T, E, k, logits, bias, sigmoid, G, kg, idx_out, w_out);
  return hipGetLastError();
}

}  // namespace moe
