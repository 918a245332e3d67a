// Top-k and group-limited top-k routing on gfx950.
//
// One 64-lane wave per token (lane l holds experts [l*VPL, l*VPL + VPL)),
// or, for up to 128 experts, teams of 8 or 16 lanes per token.
// Sources: hyper.ai story on NVIDIA Hybrid-EP (each token activates only k
// experts); DeepEP article (ai-master.dev), section "Group-limited gating
// algorithm" (the choice is restricted to a few expert groups); glossary
// "Expert Parallelism" (polydesk.ai), "Le pattern de communication
// all-to-all", Phase 2 (outputs are weighted by the router scores).
//
// Precision: sigmoid and exp run in fp64 and each result is rounded once to
// fp32; selection keys are fp32; weight sums run in fp64. The fp64 exp and
// reciprocal are this file's own (exp_f64, sigmoid_f32 below).

#include "kernels.h"
#include "wave.h"

namespace moe {

// Taylor coefficients of exp_f64 below (1/13!, ..., 1/0!). Declared with
// external linkage on purpose: the compiler then cannot fold them into
// literals, and reads them as scalar loads.
__constant__ double route_exp_taylor[14] = {
    0x1.6124613a86d09p-33, 0x1.1eed8eff8d898p-29, 0x1.ae64567f544e4p-26,   // 1/13!, 1/12!, 1/11!
    0x1.27e4fb7789f5cp-22, 0x1.71de3a556c734p-19, 0x1.a01a01a01a01ap-16,   // 1/10!, 1/9!, 1/8!
    0x1.a01a01a01a01ap-13, 0x1.6c16c16c16c17p-10, 0x1.1111111111111p-7,    // 1/7!, 1/6!, 1/5!
    0x1.5555555555555p-5, 0x1.5555555555555p-3, 0x1p-1, 0x1p+0, 0x1p+0};  // 1/4!, ..., 1/0!

namespace {

constexpr int kRouteWaves = 4;  // tokens per 256-thread block

// e^x in fp64 for the routing scores, by Cody and Waite's range reduction
// and the Taylor series:
//   x = n*ln2 + r, n = rint(x * log2(e)), |r| <= ln2/2,
// with ln2 split into a head of 32 significant bits (so n * head is exact
// for |n| < 2^21) and a tail; e^r is the Taylor polynomial of degree 13
// (truncation below 3e-18 relative) by Horner's rule, and e^x = 2^n * e^r.
// x is clamped to [-800, 700]: there e^x is 0 or finite with room to spare,
// and the results that use it round to the same fp32 values as without the
// clamp. The coefficients 1/j! (route_exp_taylor) are read from constant
// memory with a wave-uniform index, so they load into scalar registers and
// each Horner step is one fp64 FMA (as literals they would cost two vector
// moves each).
  // 1/4! ... 1/0!
constexpr double kLog2e = 0x1.71547652b82fep+0;       // log2(e), nearest double
constexpr double kLn2Hi = 0x1.62e42ffp-1;             // ln2 to 32 significant bits
constexpr double kLn2Lo = -0x1.718432a1b0e26p-35;     // ln2 - kLn2Hi, nearest double

__device__ __forceinline__ double exp_f64(double x) {
  x = __builtin_fmin(__builtin_fmax(x, -800.0), 700.0);
  const double n = __builtin_rint(x * kLog2e);
  double r = __builtin_fma(-n, kLn2Hi, x);
  r = __builtin_fma(-n, kLn2Lo, r);
  double p = route_exp_taylor[0];
#pragma unroll
  for (int j = 1; j < 14; ++j) p = __builtin_fma(p, r, route_exp_taylor[j]);
  return ldexp(p, (int)n);
}

// fp32(1 / (1 + e^-l)). The reciprocal is the hardware estimate refined by
// two Newton steps; 1 + e^-l stays below 1e305, so every step is finite.
__device__ __forceinline__ float sigmoid_f32(float l) {
  const double d = 1.0 + exp_f64(-(double)l);
  double y = __builtin_amdgcn_rcp(d);
  y = __builtin_fma(y, __builtin_fma(-d, y, 1.0), y);
  y = __builtin_fma(y, __builtin_fma(-d, y, 1.0), y);
  return (float)y;
}

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

// Wave max of a 32-bit value as a wave-uniform (scalar) value: the max of
// each 16-lane row by DPP, then the gfx9 row broadcasts carry the row maxima
// to lane 63 (lane 15 of each row into the next row, in rows 1 and 3; then
// lane 31 into rows 2 and 3), and lane 63 is read into a scalar register.
// Rows left out of a broadcast receive 0, the identity of an unsigned max.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));
  v = max(v, dpp_u32<0x4E>(v));
  v = max(v, dpp_u32<0x141>(v));
  v = max(v, dpp_u32<0x140>(v));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Max and fp64 sum over the calling lane's 16-lane row, in every lane of the
// row. With k <= 16 every chosen slot sits in row 0 and the other lanes hold
// -inf (max) or +0.0 (sum), so the row result equals the wave result bit for
// bit: the first four steps of wave_max_f32 / wave_sum_f64 are these, and
// the remaining two only combine it with -inf or add +0.0.
__device__ __forceinline__ float row_max_f32(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  return fmaxf(v, dpp_f32<0x140>(v));
}
__device__ __forceinline__ double row_sum_f64(double v) {
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  v += dpp_f64<0x141>(v);
  return v + dpp_f64<0x140>(v);
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

// Loads the VPL consecutive values [e0, e0 + VPL) of `row` (zero past n),
// with one or two 16-byte loads when `vec` says the row allows them.
template <int VPL>
__device__ __forceinline__ void load_slots(float (&v)[VPL], const float* __restrict__ row, int e0,
                                           int n, bool vec) {
  if (VPL >= 4 && vec && e0 + VPL <= n) {
#pragma unroll
    for (int h = 0; h < VPL; h += 4) {
      const float4 q = *reinterpret_cast<const float4*>(row + e0 + h);
      v[h] = q.x;
      v[h + 1] = q.y;
      v[h + 2] = q.z;
      v[h + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < VPL; ++i) v[i] = e0 + i < n ? row[e0 + i] : 0.0f;
  }
}

// One wave per token; lane l holds the VPL consecutive experts
// [l*VPL, l*VPL + VPL), so a group of gs experts spans gs/VPL neighbouring
// lanes and, among equal keys, a lower lane always holds the lower expert.
// Batch blockIdx.y of `rb`.
template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(
    int T, int E, int k, const RouteBatches rb, int sigmoid, int G, int kg, int vec) {
  __shared__ float s_key[kRouteWaves][MOE_MAX_EXPERTS];
  const float* __restrict__ logits = rb.logits[blockIdx.y];
  const float* __restrict__ bias = rb.bias[blockIdx.y];
  int32_t* __restrict__ idx_out = rb.idx[blockIdx.y];
  float* __restrict__ w_out = rb.w[blockIdx.y];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRouteWaves + wave;
  const bool live = t < T;
  const int e0 = lane * VPL;

  float lg[VPL], bs[VPL];
  load_slots<VPL>(lg, logits + (size_t)(live ? t : 0) * E, e0, live ? E : 0, vec);
  if (bias != nullptr) load_slots<VPL>(bs, bias, e0, E, vec);
  float key[VPL], score[VPL];
  bool ok[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    ok[i] = live && e0 + i < E;
    const float s = sigmoid ? sigmoid_f32(lg[i]) : lg[i];
    score[i] = s;
    key[i] = (bias != nullptr && ok[i]) ? s + bs[i] : s;
  }

  if (G > 1) {  // G is uniform over the block: the barrier below is safe
    const int gs = E / G;
    const int lpg = gs / VPL;   // lanes per group
    if (gs % VPL == 0 && (lpg & (lpg - 1)) == 0) {
      // top-2 of the lane's slots, then of the group's lanes with DPP and
      // the row and half swaps; every lane ends with its group's score
      float m1 = -INFINITY, m2 = -INFINITY;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (ok[i]) merge_top2(m1, m2, key[i], -INFINITY);
      if (lpg >= 2) dpp_top2<0xB1>(m1, m2);
      if (lpg >= 4) dpp_top2<0x4E>(m1, m2);
      if (lpg >= 8) dpp_top2<0x141>(m1, m2);
      if (lpg >= 16) dpp_top2<0x140>(m1, m2);
      if (lpg >= 32) merge_top2(m1, m2, xor16_f32(m1), xor16_f32(m2));
      if (lpg >= 64) merge_top2(m1, m2, xor32_f32(m1), xor32_f32(m2));
      const float gscore = gs == 1 ? m1 : m1 + m2;
      // rank of the lane's group (ties to the lower group); every lane of
      // group q holds its score
      const int my_group = lane / lpg;
      const uint32_t mine = ordered_bits(gscore);
      int rank = 0;
      if (G <= lpg) {
        // lane r of each group compares its group with group r (r < G);
        // the group's rank is the count of its lanes whose group r beats it
        const int r = lane & (lpg - 1);
        const uint32_t o = (uint32_t)__shfl((int)mine, r * lpg);
        const uint64_t beats = wave_ballot(r < G && (o > mine || (o == mine && r < my_group)));
        const uint64_t seg = beats >> (my_group * lpg);
        rank = __popcll(seg & ((1ull << lpg) - 1));  // G >= 2, so lpg <= 32
      } else {
        for (int q = 0; q < G; ++q) {
          const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)mine, q * lpg);
          rank += (o > mine) || (o == mine && q < my_group);
        }
      }
#pragma unroll
      for (int i = 0; i < VPL; ++i) ok[i] = ok[i] && rank < kg;
    } else {
      // any group size: lane g < G scans its group in LDS
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (ok[i]) s_key[wave][e0 + i] = key[i];
      __syncthreads();
      float gscore = 0.0f;
      if (live && lane < G) {
        float m1 = -INFINITY, m2 = -INFINITY;
        for (int q = 0; q < gs; ++q) merge_top2(m1, m2, s_key[wave][lane * gs + q], -INFINITY);
        gscore = gs == 1 ? m1 : m1 + m2;
      }
      int rank = 0;
      const uint32_t mine = ordered_bits(gscore);
      for (int q = 0; q < G; ++q) {
        const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)mine, q);
        rank += (o > mine) || (o == mine && q < lane);
      }
      const uint64_t kept = wave_ballot(lane < G && rank < kg);
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (ok[i]) ok[i] = (kept >> ((e0 + i) / gs)) & 1ull;
    }
  }
  if (!live) return;  // whole wave; no barrier follows

  // The lane's candidates as ordered keys; 0 = no candidate (every finite
  // key maps above it).
  uint32_t sk[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) sk[i] = ok[i] ? ordered_bits(key[i]) : 0u;
  // k rounds. The wave max of the lanes' best remaining keys wins; among the
  // slots holding it, the lowest lane and in it the lowest slot, i.e. the
  // lowest expert (lane l holds experts [l*VPL, l*VPL + VPL)). That slot is
  // cleared, and lane j keeps the winner's expert.
  int my_e = -1;
  for (int j = 0; j < k; ++j) {
    uint32_t head = sk[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) head = max(head, sk[i]);
    const uint32_t top = wave_max_u32(head);
    uint64_t hit[VPL];
    uint64_t any = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      hit[i] = wave_ballot(sk[i] == top);
      any |= hit[i];
    }
    const int owner = (int)__builtin_ctzll(any);
    int slot = 0;
#pragma unroll
    for (int i = VPL - 1; i >= 0; --i)
      if ((hit[i] >> owner) & 1ull) slot = i;
    const bool in_owner = lane == owner;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (i == slot) sk[i] = in_owner ? 0u : sk[i];
    if (lane == j) my_e = owner * VPL + slot;
  }
  // score of the chosen expert, from the lane that holds it
  float my_score = 0.0f;
  {
    const int e = my_e < 0 ? 0 : my_e;
    const int src = e / VPL, slot = e - src * VPL;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const float v = __shfl(score[i], src);
      if (i == slot) my_score = v;
    }
  }

  // k is uniform: the branches below do not diverge
  double u;
  if (sigmoid) {
    u = lane < k ? (double)my_score : 0.0;
  } else {
    const float mv = lane < k ? my_score : -INFINITY;
    const float m = k <= 16 ? row_max_f32(mv) : wave_max_f32(mv);
    u = lane < k ? exp_f64((double)my_score - (double)m) : 0.0;
  }
  const double total = k <= 16 ? row_sum_f64(u) : wave_sum_f64(u);
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
    int T, int E, int k, const RouteBatches rb, int sigmoid, int G, int kg) {
  const float* __restrict__ logits = rb.logits[blockIdx.y];
  const float* __restrict__ bias = rb.bias[blockIdx.y];
  int32_t* __restrict__ idx_out = rb.idx[blockIdx.y];
  float* __restrict__ w_out = rb.w[blockIdx.y];
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
    const float sv = sigmoid ? sigmoid_f32(l) : l;
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
    u = tl < k ? exp_f64((double)my_score - (double)m) : 0.0;
  }
  const double total = team_sum_f64<L>(u);
  if (live && tl < k) {
    idx_out[(size_t)t * k + tl] = my_e;
    w_out[(size_t)t * k + tl] = (float)(u / total);
  }
}

// Arguments of one routing launch over nb batches.
struct RouteLaunch {
  int nb, T, E, k;
  const RouteBatches* rb;
  int sigmoid, G, kg;
  hipStream_t stream;
};

template <int L, int VPL, int SPG>
void launch_team_spg(const RouteLaunch& a) {
  constexpr int per_block = kRouteWaves * (MOE_WAVE / L);
  hipLaunchKernelGGL((route_team_kernel<L, VPL, SPG>), dim3((a.T + per_block - 1) / per_block, a.nb),
                     dim3(256), 0, a.stream, a.T, a.E, a.k, *a.rb, a.sigmoid, a.G, a.kg);
}

// Returns false when no instance covers the group size.
template <int L, int VPL>
bool launch_team(const RouteLaunch& a) {
  const int spg = a.G > 1 ? a.E / a.G / L : 0;
  switch (spg) {
    case 0: launch_team_spg<L, VPL, 0>(a); return true;
    case 1: launch_team_spg<L, VPL, 1>(a); return true;
    case 2: if (VPL >= 2) { launch_team_spg<L, VPL, (VPL >= 2 ? 2 : 1)>(a); return true; } return false;
    case 4: if (VPL >= 4) { launch_team_spg<L, VPL, (VPL >= 4 ? 4 : 1)>(a); return true; } return false;
    case 8: if (VPL >= 8) { launch_team_spg<L, VPL, (VPL >= 8 ? 8 : 1)>(a); return true; } return false;
    default: return false;
  }
}

}  // namespace

hipError_t launch_route_batches(int nb, const RouteBatches& rb, int T, int E, int k,
                                int sigmoid, int G, int kg, hipStream_t stream) {
  if (T == 0 || nb == 0) return hipSuccess;
  const RouteLaunch a{nb, T, E, k, &rb, sigmoid, G, kg, stream};
  // Team kernels (8 lanes per token up to 64 experts, 16 up to 128) cut the
  // reduction cost per token; with more experts one wave per token is
  // faster, because the longer per-lane fp64 sigmoid chains of a team then
  // leave too few waves to hide their latency.
  const int L = E <= 64 ? 8 : 16;
  const bool team = E <= 128 && k <= L && (G == 1 || (E / G) % L == 0);
  if (team) {
    bool done;
    if (E <= 8) done = launch_team<8, 1>(a);
    else if (E <= 16) done = launch_team<8, 2>(a);
    else if (E <= 32) done = launch_team<8, 4>(a);
    else if (E <= 64) done = launch_team<8, 8>(a);
    else done = launch_team<16, 8>(a);
    if (done) return hipGetLastError();
  }
  const dim3 grid((T + kRouteWaves - 1) / kRouteWaves, nb), block(256);
  const int vpl = E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : 8;
  // 16-byte loads of a lane's slots: rows of whole 16-byte units, aligned
  const auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  bool aligned = true;
  for (int b = 0; b < nb; ++b)
    aligned = aligned && a16(rb.logits[b]) && (rb.bias[b] == nullptr || a16(rb.bias[b]));
  const int vec = vpl >= 4 && E % vpl == 0 && aligned;
  if (vpl == 1)
    hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, stream, T, E, k, rb, sigmoid, G, kg, vec);
  else if (vpl == 2)
    hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, stream, T, E, k, rb, sigmoid, G, kg, vec);
  else if (vpl == 4)
    hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, stream, T, E, k, rb, sigmoid, G, kg, vec);
  else
    hipLaunchKernelGGL(route_kernel<8>, grid, block, 0, stream, T, E, k, rb, sigmoid, G, kg, vec);
  return hipGetLastError();
}

hipError_t launch_route(int T, int E, int k, const float* logits, const float* bias,
                        int sigmoid, int G, int kg, int32_t* idx_out, float* w_out,
                        hipStream_t stream) {
  RouteBatches rb{};
  rb.logits[0] = logits;
  rb.bias[0] = bias;
  rb.idx[0] = idx_out;
  rb.w[0] = w_out;
  return launch_route_batches(1, rb, T, E, k, sigmoid, G, kg, stream);
}

}  // namespace moe
