// Routing layout on gfx950: per-expert and per-rank counts, prefix-sum
// offsets and the stable row of every (token, slot) pair.
//
// Sources: glossary "Expert Parallelism" (polydesk.ai), "Le principe de
// base" (rank r owns whole experts [r*E/R, (r+1)*E/R)) and Phase 1 of "Le
// pattern de communication all-to-all" (each rank receives the tokens of
// its local experts); hyper.ai story on Hybrid-EP (buffers preallocated at
// their maximum size, so that no size has to be read back first); glossary
// sections "Megatron-LM (NVIDIA)" and "Défis et optimisations" (capacity
// and token dropping).
//
// Two launches, no global atomics, deterministic:
//   1. count: one block per tile of whole tokens builds the tile's expert
//      histogram (and per-rank distinct-token counts) in LDS and writes it
//      to the workspace.
//   2. place: every block sums the histogram columns of the tiles before it
//      (its per-expert base) and of all tiles (totals), scans the totals
//      into offsets, and gives each pair its stable row. Inside a wave, the
//      pairs of one expert are found with one ballot per expert-id bit and
//      ranked by their lane order; waves of a tile are chained through LDS.

#include "kernels.h"
#include "wave.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / MOE_WAVE;
constexpr int kTilePairs = 1024;                          // pairs per tile (max)
constexpr int kChunks = kTilePairs / kWaves / MOE_WAVE;   // 64-pair chunks per wave

__device__ __forceinline__ int clean_expert(int v, int E) {
  return (v >= 0 && v < E) ? v : -1;
}

__global__ __launch_bounds__(kThreads) void layout_count_kernel(
    int T, int E, int k, int R, int epr, int tt, const int32_t* __restrict__ idx,
    int32_t* __restrict__ ws_hist, int32_t* __restrict__ ws_rhist) {
  __shared__ int s_hist[MOE_MAX_EXPERTS];
  __shared__ int s_rhist[MOE_MAX_EXPERTS];
  __shared__ int s_idx[kTilePairs];

  const int tid = threadIdx.x;
  const int tile = blockIdx.x;
  const int tok0 = tile * tt;
  const int np = min(tt, T - tok0) * k;
  const int32_t* src = idx + (size_t)tok0 * k;
  const int nbits = ceil_log2(E);

  for (int e = tid; e < E; e += kThreads) { s_hist[e] = 0; s_rhist[e] = 0; }
  __syncthreads();

  for (int base = 0; base < np; base += kThreads) {
    const int p = base + tid;
    const int v = p < np ? clean_expert(src[p], E) : -1;
    if (p < np) s_idx[p] = v;
    const uint64_t peers = peer_mask((uint32_t)v, v >= 0, nbits);
    if (v >= 0 && count_below(peers) == 0) atomicAdd(&s_hist[v], __popcll(peers));
  }
  __syncthreads();

  if (ws_rhist != nullptr) {
    // a pair counts for its rank if no earlier slot of the token is on it
    for (int p = tid; p < np; p += kThreads) {
      const int v = s_idx[p];
      if (v < 0) continue;
      const int r = v / epr;
      const int j = p % k;
      bool first = true;
      for (int q = 0; q < j; ++q) {
        const int o = s_idx[p - j + q];
        first = first && !(o >= 0 && o / epr == r);
      }
      if (first) atomicAdd(&s_rhist[r], 1);
    }
    __syncthreads();
    for (int r = tid; r < R; r += kThreads) ws_rhist[(size_t)tile * R + r] = s_rhist[r];
  }
  for (int e = tid; e < E; e += kThreads) ws_hist[(size_t)tile * E + e] = s_hist[e];
}

// Exclusive scan of s[0..n) in place (n <= 4 * kThreads); returns the total
// to every thread.
__device__ int block_exclusive_scan(int* s, int n, int* s_wave) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int v[4], sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = tid * 4 + q;
    v[q] = i < n ? s[i] : 0;
    sum += v[q];
  }
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int run = incl - sum, total = 0;
  for (int w = 0; w < kWaves; ++w) {
    const int x = s_wave[w];
    if (w < wave) run += x;
    total += x;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = tid * 4 + q;
    if (i < n) s[i] = run;
    run += v[q];
  }
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(kThreads) void layout_place_kernel(
    int T, int E, int k, int R, int epr, int cap, int tt, int ntiles, int num_rows,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ ws_hist,
    const int32_t* __restrict__ ws_rhist, int32_t* __restrict__ expert_counts,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ rank_counts,
    int32_t* __restrict__ rank_offsets, int32_t* __restrict__ rank_token_counts,
    int32_t* __restrict__ dst_row, int32_t* __restrict__ src_pair,
    int32_t* __restrict__ overflow) {
  __shared__ int s_tot[MOE_MAX_EXPERTS];
  __shared__ int s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int s_pre[MOE_MAX_EXPERTS];
  __shared__ int s_cnt[kWaves][MOE_MAX_EXPERTS];
  __shared__ int s_base[kWaves][MOE_MAX_EXPERTS];
  __shared__ int s_wave[kWaves];
  __shared__ int s_overflow;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.x;

  // per-expert totals and the base of this tile (sum over earlier tiles)
  for (int e = tid; e < E; e += kThreads) {
    int pre = 0, tot = 0;
    for (int b = 0; b < ntiles; ++b) {
      const int h = ws_hist[(size_t)b * E + e];
      tot += h;
      pre += b < tile ? h : 0;
    }
    s_tot[e] = tot;
    s_pre[e] = pre;
    s_off[e] = cap > 0 ? 0 : tot;
    for (int w = 0; w < kWaves; ++w) s_cnt[w][e] = 0;
  }
  if (tid == 0) s_overflow = 0;
  __syncthreads();
  if (cap > 0) {
    for (int e = tid; e <= E; e += kThreads) s_off[e] = e * cap;
    __syncthreads();
  } else {
    const int total = block_exclusive_scan(s_off, E, s_wave);
    if (tid == 0) s_off[E] = total;
    __syncthreads();
  }

  if (tile == 0) {
    for (int e = tid; e < E; e += kThreads) {
      expert_counts[e] = s_tot[e];
      expert_offsets[e] = s_off[e];
      if (cap > 0 && s_tot[e] > cap) atomicAdd(&s_overflow, s_tot[e] - cap);
    }
    if (tid == 0) expert_offsets[E] = s_off[E];
    for (int r = tid; r < R; r += kThreads) {
      int rows = 0;
      for (int e = r * epr; e < (r + 1) * epr; ++e)
        rows += cap > 0 ? min(s_tot[e], cap) : s_tot[e];
      rank_counts[r] = rows;
      rank_offsets[r] = s_off[r * epr];
      if (rank_token_counts != nullptr) {
        int c = 0;
        for (int b = 0; b < ntiles; ++b) c += ws_rhist[(size_t)b * R + r];
        rank_token_counts[r] = c;
      }
    }
    if (tid == 0) rank_offsets[R] = s_off[E];
    __syncthreads();
    if (tid == 0) overflow[0] = s_overflow;
  }

  // stable placement of this tile's pairs
  const int tok0 = tile * tt;
  const int np = T > 0 ? min(tt, T - tok0) * k : 0;
  const size_t pair0 = (size_t)tok0 * k;
  const int nbits = ceil_log2(E);
  int v[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int p = (wave * kChunks + c) * MOE_WAVE + lane;
    v[c] = p < np ? clean_expert(idx[pair0 + p], E) : -1;
    const uint64_t peers = peer_mask((uint32_t)v[c], v[c] >= 0, nbits);
    if (v[c] >= 0 && count_below(peers) == 0) atomicAdd(&s_cnt[wave][v[c]], __popcll(peers));
  }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) {
    int run = s_pre[e];
    for (int w = 0; w < kWaves; ++w) {
      s_base[w][e] = run;
      run += s_cnt[w][e];
    }
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int p = (wave * kChunks + c) * MOE_WAVE + lane;
    const int e = v[c];
    const uint64_t peers = peer_mask((uint32_t)e, e >= 0, nbits);
    int dst = -1;
    if (e >= 0) {
      const int below = count_below(peers);
      const int pos = s_base[wave][e] + below;
      if (below == 0) atomicAdd(&s_base[wave][e], __popcll(peers));
      if (cap == 0) dst = s_off[e] + pos;
      else if (pos < cap) dst = e * cap + pos;
    }
    if (p < np) {
      dst_row[pair0 + p] = dst;
      if (dst >= 0 && dst < num_rows) src_pair[dst] = (int32_t)(pair0 + p);
    }
  }

  // rows that receive no pair are marked -1 (spread over all blocks)
  for (int row = tile * kThreads + tid; row < num_rows; row += gridDim.x * kThreads) {
    bool unused;
    if (cap == 0) {
      unused = row >= s_off[E];
    } else {
      const int e = row / cap;
      unused = (row - e * cap) >= s_tot[e];
    }
    if (unused) src_pair[row] = -1;
  }
}

}  // namespace

int layout_tile_tokens(int k) { return kTilePairs / k; }

int layout_num_tiles(int T, int k) {
  const int tt = layout_tile_tokens(k);
  return (T + tt - 1) / tt;
}

size_t layout_workspace_bytes(int T, int E, int k) {
  // per tile: E expert counts + up to E rank counts
  return (size_t)layout_num_tiles(T, k) * (size_t)(2 * E) * sizeof(int32_t);
}

hipError_t launch_layout(int T, int E, int k, int R, int cap, const int32_t* idx,
                         int32_t* expert_counts, int32_t* expert_offsets,
                         int32_t* rank_counts, int32_t* rank_offsets,
                         int32_t* rank_token_counts, int32_t* dst_row,
                         int32_t* src_pair, int32_t* overflow, void* workspace,
                         hipStream_t stream) {
  const int tt = layout_tile_tokens(k);
  const int ntiles = layout_num_tiles(T, k);
  const int epr = E / R;
  const int num_rows = cap > 0 ? E * cap : T * k;
  int32_t* ws_hist = static_cast<int32_t*>(workspace);
  int32_t* ws_rhist = rank_token_counts != nullptr ? ws_hist + (size_t)ntiles * E : nullptr;
  if (ntiles > 0) {
    hipLaunchKernelGGL(layout_count_kernel, dim3(ntiles), dim3(kThreads), 0, stream,
                       T, E, k, R, epr, tt, idx, ws_hist, ws_rhist);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(layout_place_kernel, dim3(ntiles > 0 ? ntiles : 1), dim3(kThreads), 0,
                     stream, T, E, k, R, epr, cap, tt, ntiles, num_rows, idx, ws_hist,
                     ws_rhist, expert_counts, expert_offsets, rank_counts, rank_offsets,
                     rank_token_counts, dst_row, src_pair, overflow);
  return hipGetLastError();
}

}  // namespace moe
