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

// Wave max of a 32-bit value, in every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));
  v = max(v, dpp_u32<0x4E>(v));
  v = max(v, dpp_u32<0x141>(v));
  v = max(v, dpp_u32<0x140>(v));
  v = max(v, xor16_u32(v));
  return max(v, xor32_u32(v));
}

// Top-2 merge of (largest, second largest) pairs.
__device__ __forceinline__ void merge_top2(float& m1, float& m2, float o1, float o2) {
  const float hi = fmaxf(m1, o1), lo = fminf(m1, o1);
  m2 = fmaxf(lo, fmaxf(m2, o2));
  m1 = hi;
}

template <int CTRL>
__device__ __forceinline__ void dpp_top2(float& m1, float& m2) {
  merge_top2(m1, m2, dpp_f32<CTRL>(m1), dpp_f32<CTRL>(m2));
}

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(
    int T, int E, int k, const float* __restrict__ logits,
    const float* __restrict__ bias, int sigmoid, int G, int kg,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  __shared__ float s_key[kRouteWaves][MOE_MAX_EXPERTS];

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
    float gscore = 0.0f;                // lane g < G: score of group g
    if (gs == 16 || gs == 32 || gs == 64) {
      // groups cover whole rows of one slot: top-2 per row with DPP, then
      // the row and half swaps merge the rows of a group (16: none, 32: one
      // swap, 64: two). Group scores are then spread so that lane g < G
      // holds the score of group g.
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        float m1 = ok[i] ? key[i] : -INFINITY, m2 = -INFINITY;
        dpp_top2<0xB1>(m1, m2);
        dpp_top2<0x4E>(m1, m2);
        dpp_top2<0x141>(m1, m2);
        dpp_top2<0x140>(m1, m2);
        if (gs >= 32) merge_top2(m1, m2, xor16_f32(m1), xor16_f32(m2));
        if (gs == 64) merge_top2(m1, m2, xor32_f32(m1), xor32_f32(m2));
        const float sc = m1 + m2;          // score of the group holding this lane, slot i
        // group of (slot i, this lane) is (64 i + lane) / gs; lane g < G takes
        // the score of group g from lane (g * gs - 64 i), which is in slot i
        const int per_slot = 64 / gs;      // groups per slot
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (q >= per_slot) break;
          const float v = read_lane(sc, q * gs);
          if (lane == i * per_slot + q) gscore = v;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (ok[i]) s_key[wave][lane + 64 * i] = key[i];
      __syncthreads();
      if (live && lane < G) {
        float m1 = -INFINITY, m2 = -INFINITY;
        for (int q = 0; q < gs; ++q) merge_top2(m1, m2, s_key[wave][lane * gs + q], -INFINITY);
        gscore = gs == 1 ? m1 : m1 + m2;
      }
    }
    // rank of each group (ties to the lower group), then the kept set:
    // lane g < G counts the groups that beat it
    int rank = 0;
    const uint32_t mine = ordered_bits(gscore);
    for (int q = 0; q < G; ++q) {
      const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)mine, q);
      rank += (o > mine) || (o == mine && q < lane);
    }
    const uint64_t kept = wave_ballot(lane < G && rank < kg);
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (ok[i]) ok[i] = (kept >> ((lane + 64 * i) / gs)) & 1ull;
  }
  if (!live) return;  // whole wave; no barrier follows

  // Selection on 32-bit ordered keys (0 = taken or not allowed; every
  // finite key maps above 0). Each step takes the wave max of the keys; the
  // lowest lane holding it owns the winner unless another lane holds the
  // same key, in which case the lowest expert index among them wins.
  int my_e = -1;
  float my_score = 0.0f;
  uint32_t ok_key[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) ok_key[i] = ok[i] ? ordered_bits(key[i]) : 0u;
  for (int j = 0; j < k; ++j) {
    uint32_t best = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) best = max(best, ok_key[i]);
    const uint32_t top = wave_max_u32(best);
    // lowest slot of this lane holding the top key (VPL if none)
    int slot = VPL;
#pragma unroll
    for (int i = VPL - 1; i >= 0; --i)
      if (ok_key[i] == top) slot = i;
    const uint64_t holders = wave_ballot(slot < VPL);
    int e_win;
    if ((holders & (holders - 1)) == 0) {          // one lane holds it
      const int owner = (int)__builtin_ctzll(holders);
      e_win = owner + 64 * __builtin_amdgcn_readlane(slot, owner);
    } else {                                       // equal keys: lowest expert
      const int e_mine = slot < VPL ? lane + 64 * slot : 0x7FFFFFFF;
      e_win = (int)(0xFFFFFFFFu - wave_max_u32(0xFFFFFFFFu - (uint32_t)e_mine));
    }
    const int owner = e_win & 63, wslot = e_win >> 6;
    float sel = score[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i)
      if (i == wslot) sel = score[i];
    const float s_win = read_lane(sel, owner);
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane == owner && i == wslot) ok_key[i] = 0u;
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


// ---------------------------------------------------------------------------
// Team kernel: L = 8 or 16 lanes per token (64/L tokens per wave), lane tl
// of a team holds experts tl, tl + L, tl + 2L, ... Every reduction stays in
// a DPP row, so no value crosses rows and no scalar read is needed. Used when
// E <= 8 * L, k <= L and, with groups, the group size is a multiple of L.
// ---------------------------------------------------------------------------

// One DPP step of a team max over (candidate, score) pairs.
template <int CTRL>
__device__ __forceinline__ void team_step_best(uint64_t& c, float& sc) {
  const uint64_t oc = dpp_u64<CTRL>(c);
  const float os = dpp_f32<CTRL>(sc);
  if (oc > c) { c = oc; sc = os; }
}

template <int L>
__device__ __forceinline__ void team_best(uint64_t& c, float& sc) {
  team_step_best<0xB1>(c, sc);
  team_step_best<0x4E>(c, sc);
  team_step_best<0x141>(c, sc);
  if (L == 16) team_step_best<0x140>(c, sc);
}

template <int L>
__device__ __forceinline__ void team_top2(float& m1, float& m2) {
  dpp_top2<0xB1>(m1, m2);
  dpp_top2<0x4E>(m1, m2);
  dpp_top2<0x141>(m1, m2);
  if (L == 16) dpp_top2<0x140>(m1, m2);
}

template <int L>
__device__ __forceinline__ float team_max_f32(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  if (L == 16) v = fmaxf(v, dpp_f32<0x140>(v));
  return v;
}

template <int L>
__device__ __forceinline__ double team_sum_f64(double v) {
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  v += dpp_f64<0x141>(v);
  if (L == 16) v += dpp_f64<0x140>(v);
  return v;
}

// SPG: slots per expert group (a group is SPG*L experts), 0 = no groups.
template <int L, int VPL, int SPG>
__global__ __launch_bounds__(256) void route_team_kernel(
    int T, int E, int k, const float* __restrict__ logits,
    const float* __restrict__ bias, int sigmoid, int G, int kg,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  constexpr int kTeams = MOE_WAVE / L;
  const int lane = threadIdx.x & 63;
  const int tl = lane % L;
  const int t = (blockIdx.x * kRouteWaves + (threadIdx.x >> 6)) * kTeams + lane / L;
  const bool live = t < T;

  float key[VPL], score[VPL];
  bool ok[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = tl + L * i;
    ok[i] = live && e < E;
    const float l = ok[i] ? logits[(size_t)t * E + e] : 0.0f;
    const float sv = sigmoid ? (float)(1.0 / (1.0 + exp(-(double)l))) : l;
    score[i] = sv;
    key[i] = (bias != nullptr && ok[i]) ? sv + bias[e] : sv;
  }

  if (SPG > 0) {
    // group g is slots [g*SPG, (g+1)*SPG) of every lane of the team
    constexpr int NG = VPL / (SPG > 0 ? SPG : 1);
    float gsc[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      float m1 = -INFINITY, m2 = -INFINITY;
#pragma unroll
      for (int q = 0; q < SPG; ++q)
        if (ok[g * SPG + q]) merge_top2(m1, m2, key[g * SPG + q], -INFINITY);
      team_top2<L>(m1, m2);
      gsc[g] = m1 + m2;
    }
    uint32_t keep = 0;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      int rank = 0;
#pragma unroll
      for (int q = 0; q < NG; ++q)
        rank += q < G && ((gsc[q] > gsc[g]) || (gsc[q] == gsc[g] && q < g));
      keep |= (g < G && rank < kg) ? (1u << g) : 0u;
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) ok[i] = ok[i] && ((keep >> (i / (SPG > 0 ? SPG : 1))) & 1u);
  }

  uint64_t cand[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) cand[i] = ok[i] ? candidate(key[i], tl + L * i) : 0ull;
  int my_e = -1;
  float my_score = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
    float best_score = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (cand[i] > best) { best = cand[i]; best_score = score[i]; }
    team_best<L>(best, best_score);
    const int e_win = (int)(0xFFFFFFFFu - (uint32_t)best);
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (tl + L * i == e_win) cand[i] = 0ull;
    if (tl == j) { my_e = e_win; my_score = best_score; }
  }

  double u;
  if (sigmoid) {
    u = tl < k ? (double)my_score : 0.0;
  } else {
    const float m = team_max_f32<L>(tl < k ? my_score : -INFINITY);
    u = tl < k ? exp((double)my_score - (double)m) : 0.0;
  }
  const double total = team_sum_f64<L>(u);
  if (live && tl < k) {
    idx_out[(size_t)t * k + tl] = my_e;
    w_out[(size_t)t * k + tl] = (float)(u / total);
  }
}

template <int L, int VPL, int SPG>
void launch_team_spg(int T, int E, int k, const float* logits, const float* bias, int sigmoid,
                     int G, int kg, int32_t* idx_out, float* w_out, hipStream_t stream) {
  constexpr int per_block = kRouteWaves * (MOE_WAVE / L);
  hipLaunchKernelGGL((route_team_kernel<L, VPL, SPG>), dim3((T + per_block - 1) / per_block),
                     dim3(256), 0, stream, T, E, k, logits, bias, sigmoid, G, kg, idx_out, w_out);
}

// Returns false when no instance covers the group size.
template <int L, int VPL>
bool launch_team(int T, int E, int k, const float* logits, const float* bias, int sigmoid,
                 int G, int kg, int32_t* idx_out, float* w_out, hipStream_t stream) {
  const int spg = G > 1 ? E / G / L : 0;
  switch (spg) {
    case 0: launch_team_spg<L, VPL, 0>(T, E, k, logits, bias, sigmoid, G, kg, idx_out, w_out, stream); return true;
    case 1: launch_team_spg<L, VPL, 1>(T, E, k, logits, bias, sigmoid, G, kg, idx_out, w_out, stream); return true;
    case 2: if (VPL >= 2) { launch_team_spg<L, VPL, (VPL >= 2 ? 2 : 1)>(T, E, k, logits, bias, sigmoid, G, kg, idx_out, w_out, stream); return true; } return false;
    case 4: if (VPL >= 4) { launch_team_spg<L, VPL, (VPL >= 4 ? 4 : 1)>(T, E, k, logits, bias, sigmoid, G, kg, idx_out, w_out, stream); return true; } return false;
    case 8: if (VPL >= 8) { launch_team_spg<L, VPL, (VPL >= 8 ? 8 : 1)>(T, E, k, logits, bias, sigmoid, G, kg, idx_out, w_out, stream); return true; } return false;
    default: return false;
  }
}

}  // namespace

hipError_t launch_route(int T, int E, int k, const float* logits, const float* bias,
                        int sigmoid, int G, int kg, int32_t* idx_out, float* w_out,
                        hipStream_t stream) {
  if (T == 0) return hipSuccess;
  // Team kernels (8 lanes per token up to 64 experts, 16 up to 128) cut the
  // reduction cost per token; with more experts one wave per token is
  // faster, because the longer per-lane fp64 sigmoid chains of a team then
  // leave too few waves to hide their latency.
  const int L = E <= 64 ? 8 : 16;
  const bool team = E <= 128 && k <= L && (G == 1 || (E / G) % L == 0);
  if (team) {
    bool done;
    if (E <= 8) done = launch_team<8, 1>(T, E, k, logits, bias, sigmoid, G, kg, idx_out, w_out, stream);
    else if (E <= 16) done = launch_team<8, 2>(T, E, k, logits, bias, sigmoid, G, kg, idx_out, w_out, stream);
    else if (E <= 32) done = launch_team<8, 4>(T, E, k, logits, bias, sigmoid, G, kg, idx_out, w_out, stream);
    else if (E <= 64) done = launch_team<8, 8>(T, E, k, logits, bias, sigmoid, G, kg, idx_out, w_out, stream);
    else done = launch_team<16, 8>(T, E, k, logits, bias, sigmoid, G, kg, idx_out, w_out, stream);
    if (done) return hipGetLastError();
  }
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
