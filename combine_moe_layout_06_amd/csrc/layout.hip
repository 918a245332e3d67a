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
// Two launches (one when all pairs fit in one tile of 1024 pairs, three for
// hundreds of tiles), no global atomics, deterministic:
//   1. count (layout_count_kernel): one block per tile of whole tokens
//      builds the tile's expert histogram (and per-rank distinct-token
//      counts) in LDS and writes it to the workspace.
//   2. place (layout_wide_kernel): one 1024-thread block per tile, one pair
//      per thread. Every block adds the histogram rows of the tiles before it
//      (its per-expert base) and of all tiles (totals), scans the totals into
//      offsets, and gives each pair its stable row. Inside a wave, the pairs
//      of one expert are found with one ballot per expert-id bit and ranked
//      by their lane order; the waves of a tile are chained through LDS. With
//      one tile the block counts the pairs itself and no count pass runs.
// Every place block reads the whole [tiles, E] histogram, so that pass grows
// with tiles^2 * E over the grid. From 256 tiles, or past 16384 histogram
// entries, a scan pass between the two (layout_scan_kernel) rewrites the
// histogram as per-tile bases plus totals, and 256-thread place blocks
// (layout_place_kernel) read only their own row: linear in tiles * E.
//
// Also here: the (token, rank) rows of the deduplicated dispatch, placed the
// same way with the rank as the key (rank_count_kernel, rank_wide_kernel;
// rank_place_kernel after the scan pass), and the fused layout + dispatch
// launch for decode-sized inputs in capacity mode (layout_dispatch_kernel).

#include "dispatch_body.h"
#include "kernels.h"
#include "wave.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / MOE_WAVE;
constexpr int kTilePairs = 1024;                          // pairs per tile (max)
constexpr int kChunks = kTilePairs / kWaves / MOE_WAVE;   // 64-pair chunks per wave
constexpr int kStage = 8192;                              // histogram ints staged per pass
constexpr int kRankMaskWords = 256;                       // per-rank token bitmasks (one tile)
// A scan pass feeds the place pass from kScanMinTiles tiles on, or once the
// histogram outgrows two staging passes (measured crossovers: ~96 tiles for
// E = 256, ~200 for E = 8)
constexpr int kScanMinTiles = 256;
constexpr int kScanThreads = 1024;
constexpr int kScanCols = 16;                             // histogram columns per scan block
constexpr int kScanGroups = kScanThreads / kScanCols;     // row groups per scan block
constexpr int kScanBatch = 16;                            // loads in flight per thread

__device__ __forceinline__ int clean_expert(int v, int E) {
  return (v >= 0 && v < E) ? v : -1;
}

// Rank of an expert: a shift when E/R is a power of two, else a division.
__device__ __forceinline__ int rank_of(int e, int epr, int epr_shift) {
  return epr_shift >= 0 ? (e >> epr_shift) : e / epr;
}

// Batch blockIdx.y of `lb`; its workspace receives [ntiles, E] expert
// counts, then (with rank_token_counts) [ntiles, R] distinct-token counts.
__global__ __launch_bounds__(kThreads) void layout_count_kernel(
    int T, int E, int k, int R, int epr, int epr_shift, int tt, int ntiles,
    const LayoutBatches lb) {
  const LayoutBatch& bt = lb.b[blockIdx.y];
  const int32_t* __restrict__ idx = bt.idx;
  int32_t* __restrict__ ws_hist = static_cast<int32_t*>(bt.workspace);
  int32_t* __restrict__ ws_rhist =
      bt.rank_token_counts != nullptr ? ws_hist + (size_t)ntiles * E : nullptr;
  __shared__ int s_hist[MOE_MAX_EXPERTS];
  __shared__ int s_rhist[MOE_MAX_EXPERTS];
  __shared__ int s_rank[kTilePairs];     // rank of each pair, -1 if masked

  const int tid = threadIdx.x;
  const int tile = blockIdx.x;
  const int tok0 = tile * tt;
  const int ntok = min(tt, T - tok0);
  const int np = ntok * k;
  const int32_t* src = idx + (size_t)tok0 * k;

  // all loads of the tile are issued before the first use
  int v[kTilePairs / kThreads];
#pragma unroll
  for (int q = 0; q < kTilePairs / kThreads; ++q) {
    const int p = q * kThreads + tid;
    v[q] = p < np ? src[p] : -1;
  }
  for (int e = tid; e < E; e += kThreads) { s_hist[e] = 0; s_rhist[e] = 0; }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kTilePairs / kThreads; ++q) {
    const int p = q * kThreads + tid;
    const int e = clean_expert(v[q], E);
    if (p < np) s_rank[p] = e >= 0 ? rank_of(e, epr, epr_shift) : -1;
    if (e >= 0) atomicAdd(&s_hist[e], 1);
  }
  __syncthreads();

  if (ws_rhist != nullptr) {
    // one thread per token: a rank counts once, at its first slot
    for (int tl = tid; tl < ntok; tl += kThreads) {
      const int* r = s_rank + tl * k;
      if (R <= 64) {
        uint64_t seen = 0;
        for (int j = 0; j < k; ++j) {
          const int x = r[j];
          if (x >= 0 && !((seen >> x) & 1ull)) {
            seen |= 1ull << x;
            atomicAdd(&s_rhist[x], 1);
          }
        }
      } else {
        for (int j = 0; j < k; ++j) {
          const int x = r[j];
          bool first = x >= 0;
          for (int o = 0; o < j; ++o) first = first && r[o] != x;
          if (first) atomicAdd(&s_rhist[x], 1);
        }
      }
    }
    __syncthreads();
    for (int q = tid; q < R; q += kThreads) ws_rhist[(size_t)tile * R + q] = s_rhist[q];
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

// Column scan of the per-tile histograms, for many tiles. Matrix `a`
// ([ntiles, wa]) is replaced in place by its exclusive prefix over tiles (the
// base of every tile) and its column totals go to a_tot; matrix `b`
// ([ntiles, wb], nullable) only yields its column totals. Blocks [0, ga)
// take 16 columns of a each, the others 16 columns of b. The 64 row groups of
// a block (4 per wave: lane = group_in_wave * 16 + column) each own a run of
// consecutive tiles, summed in one batch of loads; the groups' sums meet in
// LDS, and a second pass rewrites the run as prefixes.
__global__ __launch_bounds__(kScanThreads) void layout_scan_kernel(
    int ntiles, int wa, int ga, int32_t* __restrict__ a, int32_t* __restrict__ a_tot, int wb,
    const int32_t* __restrict__ b, int32_t* __restrict__ b_tot) {
  __shared__ int s_sum[kScanGroups][kScanCols];
  const int tid = threadIdx.x;
  const int col = tid & (kScanCols - 1), grp = tid / kScanCols;
  const bool is_a = (int)blockIdx.x < ga;
  const int W = is_a ? wa : wb;
  const int32_t* m = is_a ? a : b;
  const int c = (is_a ? (int)blockIdx.x : (int)blockIdx.x - ga) * kScanCols + col;
  const bool live = c < W;
  const int rpg = (ntiles + kScanGroups - 1) / kScanGroups;   // tiles per row group
  const int r0 = min(grp * rpg, ntiles), r1 = min(r0 + rpg, ntiles);

  int sum = 0;
  for (int r = r0; r < r1; r += kScanBatch) {
    int x[kScanBatch];
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) x[u] = live && r + u < r1 ? m[(size_t)(r + u) * W + c] : 0;
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) sum += x[u];
  }
  s_sum[grp][col] = sum;
  __syncthreads();
  int run = 0, total = 0;
  for (int g = 0; g < kScanGroups; ++g) {
    const int s = s_sum[g][col];
    run += g < grp ? s : 0;
    total += s;
  }
  if (!live) return;
  if (grp == 0) (is_a ? a_tot : b_tot)[c] = total;
  if (!is_a) return;
  for (int r = r0; r < r1; r += kScanBatch) {
    int x[kScanBatch];
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) x[u] = r + u < r1 ? a[(size_t)(r + u) * W + c] : 0;
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      if (r + u < r1) a[(size_t)(r + u) * W + c] = run;
      run += x[u];
    }
  }
}

// The 256-thread place pass, in two modes:
//   - self_count (the layout blocks of the fused layout + dispatch launch):
//     all pairs form one tile (T*k <= kTilePairs) and no count pass ran.
//     Every block loads all pairs and builds the histogram itself (block 0
//     also the distinct-token counts), so the layout needs no launch before
//     it; the pairs are loaded chunk-major (chunk c of wave w = pairs
//     [(4c + w)*64, +64)), and block b places chunk b only, after the pairs
//     of the chunks before it, so up to four blocks share the placement.
//   - otherwise the scan pass has run (many tiles): ws_hist holds the base of
//     every tile and ws_tot / ws_rtot the totals, so the block reads its own
//     row only.
// Block `tile` of `nblocks` (the place kernel's blockIdx.x and gridDim.x, or
// the layout blocks of the fused layout + dispatch launch).
__device__ __forceinline__ void layout_place_body(
    int tile, int nblocks,
    int T, int E, int k, int R, int epr, int epr_shift, int cap, int tt, int ntiles,
    int self_count, int num_rows,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ ws_hist,
    const int32_t* __restrict__ ws_rhist, const int32_t* __restrict__ ws_tot,
    const int32_t* __restrict__ ws_rtot, int32_t* __restrict__ expert_counts,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ rank_counts,
    int32_t* __restrict__ rank_offsets, int32_t* __restrict__ rank_token_counts,
    int32_t* __restrict__ dst_row, int32_t* __restrict__ src_pair,
    int32_t* __restrict__ overflow) {
  __shared__ int s_tot[MOE_MAX_EXPERTS];
  __shared__ int s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int s_pre[MOE_MAX_EXPERTS];
  __shared__ int s_rtc[MOE_MAX_EXPERTS];
  __shared__ int s_cnt[kWaves][MOE_MAX_EXPERTS];
  __shared__ int s_base[kWaves][MOE_MAX_EXPERTS];
  __shared__ int s_wave[kWaves];
  __shared__ int s_overflow;
  __shared__ int s_rank[kTilePairs];   // rank of each pair (self_count)
  __shared__ uint32_t s_rmask[kRankMaskWords];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // blocks at or past ntiles only fill unused rows
  const int tok0 = tile * tt;
  const int np = tile < ntiles ? min(tt, T - tok0) * k : 0;
  const size_t pair0 = (size_t)tok0 * k;

  // this tile's pairs and the first histogram chunk are loaded together; in
  // self_count mode every block loads all pairs (it needs their histogram)
  const int np_load = self_count ? T * k : np;
  const size_t base = self_count ? 0 : pair0;   // pair index of local pair 0
  const auto pair_of = [&](int c) {
    return self_count ? (c * kWaves + wave) * MOE_WAVE + lane : (wave * kChunks + c) * MOE_WAVE + lane;
  };
  int v[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int p = pair_of(c);
    v[c] = p < np_load ? idx[base + p] : -1;
  }
  const bool scanned = !self_count;
  // block 0 also takes the distinct-token counts of each rank
  const bool sum_rtc = !self_count && tile == 0 && rank_token_counts != nullptr;
  // after the scan pass: this tile's bases and the totals, loaded now
  constexpr int kPerThread = MOE_MAX_EXPERTS / kThreads;
  int pre0[kPerThread], tot0[kPerThread], rtc0[kPerThread];
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int e = q * kThreads + tid;
    pre0[q] = scanned && e < E && tile < ntiles ? ws_hist[(size_t)tile * E + e] : 0;
    tot0[q] = scanned && e < E ? ws_tot[e] : 0;
    rtc0[q] = scanned && sum_rtc && e < R ? ws_rtot[e] : 0;
  }

#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int e = q * kThreads + tid;
    if (e < E) {
      s_tot[e] = tot0[q];
      s_pre[e] = pre0[q];
      s_rtc[e] = rtc0[q];
      for (int w = 0; w < kWaves; ++w) s_cnt[w][e] = 0;
    }
  }
  if (tid == 0) s_overflow = 0;
  // distinct tokens per rank as per-rank token bitmasks (one tile, small T*R)
  const int mask_words = (T + 31) / 32;
  const bool rank_masks = self_count && tile == 0 && rank_token_counts != nullptr &&
                          R * mask_words <= kRankMaskWords;
  if (rank_masks)
    for (int i = tid; i < R * mask_words; i += kThreads) s_rmask[i] = 0u;

  if (self_count) {
    // the only tile: histogram of all pairs (already in v), and of the
    // pairs before this block's chunk
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int p = pair_of(c);
      const int e = clean_expert(v[c], E);
      if (e >= 0) {
        atomicAdd(&s_tot[e], 1);
        if (c < tile) atomicAdd(&s_pre[e], 1);
        if (rank_masks) {
          const int t = p / k;
          atomicOr(&s_rmask[rank_of(e, epr, epr_shift) * mask_words + (t >> 5)], 1u << (t & 31));
        }
      }
      if (p < np_load) s_rank[p] = e >= 0 ? rank_of(e, epr, epr_shift) : -1;
      if (c != tile) v[c] = -1;   // this block places chunk `tile` only
    }
    __syncthreads();
    if (rank_masks) {
      for (int r = tid; r < R; r += kThreads) {
        int n = 0;
        for (int i = 0; i < mask_words; ++i) n += __popc(s_rmask[r * mask_words + i]);
        s_rtc[r] = n;
      }
    } else if (tile == 0 && rank_token_counts != nullptr) {
      for (int tl = tid; tl < T; tl += kThreads) {
        const int* r = s_rank + tl * k;
        if (R <= 64) {
          uint64_t seen = 0;
          for (int j = 0; j < k; ++j) {
            const int x = r[j];
            if (x >= 0 && !((seen >> x) & 1ull)) {
              seen |= 1ull << x;
              atomicAdd(&s_rtc[x], 1);
            }
          }
        } else {
          for (int j = 0; j < k; ++j) {
            const int x = r[j];
            bool first = x >= 0;
            for (int o = 0; o < j; ++o) first = first && r[o] != x;
            if (first) atomicAdd(&s_rtc[x], 1);
          }
        }
      }
    }
  }

  if (!self_count) __syncthreads();   // the LDS counters are zeroed

  // pairs of one expert inside each wave (one ballot per expert-id bit) and
  // the per-wave counts: they need no histogram, so they run while its loads
  // are in flight
  const int nbits = ceil_log2(E);
  uint64_t peers[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    v[c] = clean_expert(v[c], E);
    peers[c] = peer_mask((uint32_t)v[c], v[c] >= 0, nbits);
    if (v[c] >= 0 && count_below(peers[c]) == 0) atomicAdd(&s_cnt[wave][v[c]], __popcll(peers[c]));
  }

  __syncthreads();
  for (int e = tid; e < E; e += kThreads) s_off[e] = cap > 0 ? 0 : s_tot[e];
  __syncthreads();
  if (cap > 0) {
    for (int e = tid; e <= E; e += kThreads) s_off[e] = e * cap;
    __syncthreads();
  } else {
    const int total = block_exclusive_scan(s_off, E, s_wave);
    if (tid == 0) s_off[E] = total;
    __syncthreads();
  }

  // the global counts: block 0 holds the distinct-token counts, the last
  // block (which has no other extra work) writes the rest
  if (tile == 0 && rank_token_counts != nullptr)
    for (int r = tid; r < R; r += kThreads) rank_token_counts[r] = s_rtc[r];
  if (tile == nblocks - 1) {
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
    }
    if (tid == 0) rank_offsets[R] = s_off[E];
    __syncthreads();
    if (tid == 0) overflow[0] = s_overflow;
  }

  // stable placement of this tile's pairs: chain the waves' counts, then
  // rank inside each wave by lane order
  for (int e = tid; e < E; e += kThreads) {
    int run = s_pre[e];
    for (int w = 0; w < kWaves; ++w) {
      s_base[w][e] = run;
      run += s_cnt[w][e];
    }
  }
  __syncthreads();
  const int np_place = self_count ? (tile < kChunks ? np_load : 0) : np;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int p = pair_of(c);
    const int e = v[c];
    int dst = -1;
    if (e >= 0) {
      const int below = count_below(peers[c]);
      const int pos = s_base[wave][e] + below;
      if (below == 0) atomicAdd(&s_base[wave][e], __popcll(peers[c]));
      if (cap == 0) dst = s_off[e] + pos;
      else if (pos < cap) dst = e * cap + pos;
    }
    if (p < np_place && (!self_count || c == tile)) {
      dst_row[base + p] = dst;
      if (dst >= 0 && dst < num_rows) src_pair[dst] = (int32_t)(base + p);
    }
  }

  // rows that receive no pair are marked -1; all waves of the grid share it
  const int gwave = tile * kWaves + wave, nwaves = nblocks * kWaves;
  if (cap == 0) {
    for (int row = s_off[E] + gwave * MOE_WAVE + lane; row < num_rows; row += nwaves * MOE_WAVE)
      src_pair[row] = -1;
  } else {
    for (int e = gwave; e < E; e += nwaves) {
      const int end = (e + 1) * cap;
      for (int row = e * cap + min(s_tot[e], cap) + lane; row < end; row += MOE_WAVE)
        src_pair[row] = -1;
    }
  }
}

__global__ __launch_bounds__(kThreads) void layout_place_kernel(
    int T, int E, int k, int R, int epr, int epr_shift, int cap, int tt, int ntiles,
    int self_count, int num_rows,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ ws_hist,
    const int32_t* __restrict__ ws_rhist, const int32_t* __restrict__ ws_tot,
    const int32_t* __restrict__ ws_rtot, int32_t* __restrict__ expert_counts,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ rank_counts,
    int32_t* __restrict__ rank_offsets, int32_t* __restrict__ rank_token_counts,
    int32_t* __restrict__ dst_row, int32_t* __restrict__ src_pair,
    int32_t* __restrict__ overflow) {
  layout_place_body(blockIdx.x, gridDim.x, T, E, k, R, epr, epr_shift, cap, tt, ntiles,
                    self_count, num_rows, idx, ws_hist, ws_rhist, ws_tot, ws_rtot,
                    expert_counts, expert_offsets, rank_counts, rank_offsets, rank_token_counts,
                    dst_row, src_pair, overflow);
}

// ---------------------------------------------------------------------------
// Place pass in 1024-thread blocks, one per tile of at most 1024 pairs: wave w
// holds pairs [64w, 64w + 64) of the tile, one per lane, so the wave's pairs
// of one expert take a single ballot round per expert-id bit and each wave
// has one chunk to place (a quarter of the dependent steps of the 256-thread
// place pass).
//   - SELF (all pairs form one tile and no count pass ran; ws_hist and
//     ws_rhist are not read): every block counts the tile itself, from the per-wave
//     counts; block 0 places it. The layout is then a single launch.
//   - otherwise the count pass has written the per-tile histograms
//     ([ntiles, E] in ws_hist, [ntiles, R] distinct-token counts in
//     ws_rhist) and block b places tile b: every block adds all histogram
//     rows (its totals) and the rows before its tile (its base), one LDS
//     atomic per nonzero entry, with all loads in flight at once; block 0
//     also adds the distinct-token counts. Used while ntiles * E fits
//     kWideHistLoads loads per thread.
// Block 0 writes the counts and offsets; every wave of the grid marks the
// unused rows of about one expert (capacity mode) or the rows past the last
// pair (packed mode).
// ---------------------------------------------------------------------------
constexpr int kWideThreads = 1024;
constexpr int kWideWaves = kWideThreads / MOE_WAVE;
constexpr int kWideHistLoads = 16;   // histogram entries per thread (max)
static_assert(kWideThreads == kTilePairs, "one pair per thread");
// the wide place pass covers every histogram that needs no scan pass
static_assert(kWideHistLoads * kWideThreads >= 2 * kStage, "histogram loads per thread");

// Exclusive scan of s[0..n) in place (n <= kWideThreads) by a 1024-thread
// block; returns the total to every thread.
__device__ int block_exclusive_scan_wide(int* s, int n, int* s_wave) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int v = tid < n ? s[tid] : 0;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int run = incl - v, total = 0;
#pragma unroll
  for (int w = 0; w < kWideWaves; ++w) {
    const int x = s_wave[w];
    if (w < wave) run += x;
    total += x;
  }
  if (tid < n) s[tid] = run;
  __syncthreads();
  return total;
}

// Row of flat index i of a row-major matrix with n columns (a shift when n
// is a power of two).
__device__ __forceinline__ int row_of(int i, int n, int shift) {
  return shift >= 0 ? (i >> shift) : i / n;
}

// Batch blockIdx.y of `lb` (its workspace as layout_count_kernel wrote it).
template <bool SELF>
__global__ __launch_bounds__(kWideThreads) void layout_wide_kernel(
    int T, int E, int k, int R, int epr, int epr_shift, int cap, int tt, int ntiles,
    int num_rows, int e_shift, int r_shift, const LayoutBatches lb) {
  const LayoutBatch& bt = lb.b[blockIdx.y];
  const int32_t* __restrict__ idx = bt.idx;
  const int32_t* __restrict__ ws_hist = static_cast<const int32_t*>(bt.workspace);
  const int32_t* __restrict__ ws_rhist =
      bt.rank_token_counts != nullptr ? ws_hist + (size_t)ntiles * E : nullptr;
  int32_t* __restrict__ expert_counts = bt.expert_counts;
  int32_t* __restrict__ expert_offsets = bt.expert_offsets;
  int32_t* __restrict__ rank_counts = bt.rank_counts;
  int32_t* __restrict__ rank_offsets = bt.rank_offsets;
  int32_t* __restrict__ rank_token_counts = bt.rank_token_counts;
  int32_t* __restrict__ dst_row = bt.dst_row;
  int32_t* __restrict__ src_pair = bt.src_pair;
  int32_t* __restrict__ overflow = bt.overflow;
  __shared__ int s_cnt[kWideWaves][MOE_MAX_EXPERTS];
  __shared__ int s_tot[MOE_MAX_EXPERTS];
  __shared__ int s_pre[MOE_MAX_EXPERTS];
  __shared__ int s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int s_rtc[MOE_MAX_EXPERTS];
  __shared__ int s_rank[kTilePairs];
  __shared__ uint32_t s_rmask[kRankMaskWords];
  __shared__ int s_wave[kWideWaves];
  __shared__ int s_overflow;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.x;
  const bool lead = tile == 0;
  constexpr bool self = SELF;
  // the tile this block reads: all blocks read the only tile in self mode
  const int mine = self ? 0 : tile;
  const int np = mine < ntiles ? min(tt, T - mine * tt) * k : 0;
  const size_t pair0 = (size_t)mine * tt * k;
  const bool places = self ? lead : tile < ntiles;
  const int raw = tid < np ? idx[pair0 + tid] : -1;
  const bool rtc = lead && rank_token_counts != nullptr;
  // histogram rows (and block 0's distinct-token rows), all loads in flight
  const int hist_n = self ? 0 : ntiles * E;
  const int rhist_n = self || !rtc ? 0 : ntiles * R;
  int h[kWideHistLoads], hr[kWideHistLoads];
#pragma unroll
  for (int j = 0; j < kWideHistLoads; ++j) {
    const int i = j * kWideThreads + tid;
    h[j] = i < hist_n ? ws_hist[i] : 0;
    hr[j] = i < rhist_n ? ws_rhist[i] : 0;
  }
  if (tid < E) {
    for (int w = 0; w < kWideWaves; ++w) s_cnt[w][tid] = 0;
    s_tot[tid] = 0;
    s_pre[tid] = 0;
  }
  const int mask_words = (T + 31) / 32;
  const bool masks = self && rtc && R * mask_words <= kRankMaskWords;
  if (rtc && tid < R) s_rtc[tid] = 0;
  if (masks)
    for (int i = tid; i < R * mask_words; i += kWideThreads) s_rmask[i] = 0u;
  if (tid == 0) s_overflow = 0;
  __syncthreads();

#pragma unroll
  for (int j = 0; j < kWideHistLoads; ++j) {
    const int i = j * kWideThreads + tid;
    if (h[j] != 0) {
      const int row = row_of(i, E, e_shift), col = i - row * E;
      atomicAdd(&s_tot[col], h[j]);
      if (row < tile) atomicAdd(&s_pre[col], h[j]);
    }
    if (hr[j] != 0) atomicAdd(&s_rtc[i - row_of(i, R, r_shift) * R], hr[j]);
  }
  // the wave's pairs of one expert (one ballot per expert-id bit); the
  // lowest of them stores their number
  const int e = clean_expert(raw, E);
  const uint64_t peers = peer_mask((uint32_t)e, e >= 0, ceil_log2(E));
  const int below = count_below(peers);
  if (e >= 0 && below == 0) s_cnt[wave][e] = __popcll(peers);
  if (self && rtc) {
    const int r = e >= 0 ? rank_of(e, epr, epr_shift) : -1;
    if (tid < np) s_rank[tid] = r;
    if (masks && r >= 0) {
      const int t = tid / k;
      atomicOr(&s_rmask[r * mask_words + (t >> 5)], 1u << (t & 31));
    }
  }
  __syncthreads();

  // chain the waves: s_cnt[w][e] becomes the first position of wave w's
  // pairs of expert e (after the tiles before); totals and (capacity mode)
  // fixed offsets
  if (tid < E) {
    int c[kWideWaves];
#pragma unroll
    for (int w = 0; w < kWideWaves; ++w) c[w] = s_cnt[w][tid];
    int run = s_pre[tid];
#pragma unroll
    for (int w = 0; w < kWideWaves; ++w) {
      s_cnt[w][tid] = run;
      run += c[w];
    }
    if (self) s_tot[tid] = run;
    s_off[tid] = cap > 0 ? tid * cap : (self ? run : s_tot[tid]);
  }
  if (cap > 0 && tid == 0) s_off[E] = E * cap;
  if (masks) {
    if (tid < R) {
      int n = 0;
      for (int i = 0; i < mask_words; ++i) n += __popc(s_rmask[tid * mask_words + i]);
      s_rtc[tid] = n;
    }
  } else if (self && rtc) {
    // one thread per token: a rank counts once, at its first slot
    for (int t = tid; t < T; t += kWideThreads) {
      const int* rk = s_rank + t * k;
      for (int j = 0; j < k; ++j) {
        const int x = rk[j];
        bool first = x >= 0;
        for (int o = 0; o < j; ++o) first = first && rk[o] != x;
        if (first) atomicAdd(&s_rtc[x], 1);
      }
    }
  }
  __syncthreads();
  if (cap == 0) {
    const int total = block_exclusive_scan_wide(s_off, E, s_wave);
    if (tid == 0) s_off[E] = total;
  }
  __syncthreads();

  if (lead) {
    if (tid < E) {
      expert_counts[tid] = s_tot[tid];
      expert_offsets[tid] = s_off[tid];
      if (cap > 0 && s_tot[tid] > cap) atomicAdd(&s_overflow, s_tot[tid] - cap);
    }
    if (tid < R) {
      int rows = 0;
      for (int x = tid * epr; x < (tid + 1) * epr; ++x) rows += cap > 0 ? min(s_tot[x], cap) : s_tot[x];
      rank_counts[tid] = rows;
      rank_offsets[tid] = s_off[tid * epr];
      if (rtc) rank_token_counts[tid] = s_rtc[tid];
    }
    if (tid == 0) {
      expert_offsets[E] = s_off[E];
      rank_offsets[R] = s_off[E];
    }
  }
  if (places) {
    // stable row: the pairs of e before the tile and in the waves before,
    // then lane order
    int dst = -1;
    if (e >= 0) {
      const int pos = s_cnt[wave][e] + below;
      if (cap == 0) dst = s_off[e] + pos;
      else if (pos < cap) dst = e * cap + pos;
    }
    if (tid < np) {
      dst_row[pair0 + tid] = dst;
      if (dst >= 0 && dst < num_rows) src_pair[dst] = (int32_t)(pair0 + tid);
    }
  }

  // rows that receive no pair are marked -1; all waves of the grid share it
  const int gwave = blockIdx.x * kWideWaves + wave, nwaves = gridDim.x * kWideWaves;
  if (cap == 0) {
    for (int row = s_off[E] + gwave * MOE_WAVE + lane; row < num_rows; row += nwaves * MOE_WAVE)
      src_pair[row] = -1;
  } else {
    for (int x = gwave; x < E; x += nwaves) {
      const int end = (x + 1) * cap;
      for (int row = x * cap + min(s_tot[x], cap) + lane; row < end; row += MOE_WAVE)
        src_pair[row] = -1;
    }
  }
  if (lead) {
    __syncthreads();
    if (tid == 0) overflow[0] = s_overflow;
  }
}

// Fused layout + dispatch for one tile in capacity mode (decode-sized
// inputs): blocks [0, nl) run the single-launch layout above, blocks from nl
// on run the dispatch of DT (MOE_DTYPE_*), whose waves compute their token's
// rows from the routing (DstCapacity) instead of waiting for dst_row. The
// two halves share nothing, so they overlap completely.
template <int DT>
__global__ __launch_bounds__(kThreads) void layout_dispatch_kernel(
    int nl, int T, int E, int k, int R, int epr, int epr_shift, int cap, int tt, int num_rows,
    const int32_t* __restrict__ idx, int32_t* __restrict__ expert_counts,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ rank_counts,
    int32_t* __restrict__ rank_offsets, int32_t* __restrict__ rank_token_counts,
    int32_t* __restrict__ dst_row, int32_t* __restrict__ src_pair,
    int32_t* __restrict__ overflow, int H, int parts, int per_part,
    const u32x4* __restrict__ x, void* __restrict__ out, void* __restrict__ out_scales) {
  if ((int)blockIdx.x < nl) {
    layout_place_body(blockIdx.x, nl, T, E, k, R, epr, epr_shift, cap, tt, 1, 1, num_rows, idx,
                      nullptr, nullptr, nullptr, nullptr, expert_counts, expert_offsets,
                      rank_counts, rank_offsets, rank_token_counts, dst_row, src_pair, overflow);
    return;
  }
  const int b = blockIdx.x - nl;
  const DstCapacity dst{idx, E, cap};
  if (DT == MOE_DTYPE_BF16)
    dispatch_bf16_body(b, T, k, H / 8, parts, per_part, num_rows, x, dst,
                       static_cast<u32x4*>(out));
  else if (DT == MOE_DTYPE_FP8_E4M3)
    dispatch_fp8_body(b, T, k, H, parts, per_part, num_rows, x, dst,
                      static_cast<uint8_t*>(out), static_cast<float*>(out_scales));
  else
    dispatch_mxfp8_body(b, T, k, H, parts, per_part, num_rows, x, dst,
                        static_cast<uint8_t*>(out), static_cast<uint8_t*>(out_scales));
}

// ---------------------------------------------------------------------------
// (token, rank) rows for the deduplicated dispatch and the hierarchical
// combine (hyper.ai story on Hybrid-EP: the combine reduces inside one
// destination first, then across destinations). The pair (t, j) at the
// token's first slot on rank r stands for the (t, r) row. These pairs are
// placed the way the expert layout places its pairs, with the rank as the
// key: counted per tile, based on the tiles before, ranked by lane order
// inside each wave and chained across waves, so that the rows of a rank
// come in token order. Every other slot of the token on r shares the row.
// ---------------------------------------------------------------------------

// First slot of the token whose rank equals that of slot j (j itself when
// it is the first), or -1 for a masked slot. `r` holds the ranks of the
// token's k slots.
__device__ __forceinline__ int first_slot_of_rank(const int* r, int j) {
  const int x = r[j];
  if (x < 0) return -1;
  for (int o = 0; o < j; ++o)
    if (r[o] == x) return o;
  return j;
}

__global__ __launch_bounds__(kThreads) void rank_count_kernel(
    int T, int E, int k, int R, int epr, int epr_shift, int tt, const RankLayoutBatches rb) {
  const RankLayoutBatch& bt = rb.b[blockIdx.y];
  const int32_t* __restrict__ idx = bt.idx;
  int32_t* __restrict__ ws_rhist = static_cast<int32_t*>(bt.workspace);
  __shared__ int s_rhist[MOE_MAX_EXPERTS];
  __shared__ int s_rank[kTilePairs];

  const int tid = threadIdx.x;
  const int tile = blockIdx.x;
  const int tok0 = tile * tt;
  const int np = min(tt, T - tok0) * k;
  const int32_t* src = idx + (size_t)tok0 * k;

  int v[kTilePairs / kThreads];
#pragma unroll
  for (int q = 0; q < kTilePairs / kThreads; ++q) {
    const int p = q * kThreads + tid;
    v[q] = p < np ? src[p] : -1;
  }
  for (int r = tid; r < R; r += kThreads) s_rhist[r] = 0;
#pragma unroll
  for (int q = 0; q < kTilePairs / kThreads; ++q) {
    const int p = q * kThreads + tid;
    const int e = clean_expert(v[q], E);
    if (p < np) s_rank[p] = e >= 0 ? rank_of(e, epr, epr_shift) : -1;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kTilePairs / kThreads; ++q) {
    const int p = q * kThreads + tid;
    if (p < np) {
      const int tl = p / k, j = p - tl * k;
      if (first_slot_of_rank(s_rank + tl * k, j) == j) atomicAdd(&s_rhist[s_rank[p]], 1);
    }
  }
  __syncthreads();
  for (int r = tid; r < R; r += kThreads) ws_rhist[(size_t)tile * R + r] = s_rhist[r];
}

// The rank at the token's first slot on it for pair p of a tile (the key
// of the (token, rank) row the pair stands for), else -1; *first = that
// first slot (-1 for a masked slot). s_rank holds the ranks of the tile's
// pairs.
__device__ __forceinline__ int rank_key(const int* s_rank, int p, int k, int* first) {
  const int tl = p / k, j = p - tl * k;
  *first = first_slot_of_rank(s_rank + tl * k, j);
  return *first == j ? s_rank[p] : -1;
}

// Place pass for many tiles (after the scan pass): one 256-thread block per
// tile reads its tile's base row and the totals from the workspace. Batch
// blockIdx.y.
__global__ __launch_bounds__(kThreads) void rank_place_kernel(
    int T, int E, int k, int R, int epr, int epr_shift, int tt, int ntiles, int max_rows,
    const RankLayoutBatches rb) {
  const RankLayoutBatch& bt = rb.b[blockIdx.y];
  const int32_t* __restrict__ idx = bt.idx;
  const int32_t* __restrict__ ws_base = static_cast<const int32_t*>(bt.workspace);
  const int32_t* __restrict__ ws_tot = ws_base + (size_t)ntiles * R;
  int32_t* __restrict__ counts = bt.counts;
  int32_t* __restrict__ offsets = bt.offsets;
  int32_t* __restrict__ rank_row = bt.rank_row;
  int32_t* __restrict__ send_row = bt.send_row;
  int32_t* __restrict__ row_token = bt.row_token;
  __shared__ int s_tot[MOE_MAX_EXPERTS];
  __shared__ int s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int s_cnt[kWaves][MOE_MAX_EXPERTS];
  __shared__ int s_base[kWaves][MOE_MAX_EXPERTS];
  __shared__ int s_wave[kWaves];
  __shared__ int s_rank[kTilePairs];
  __shared__ int s_row[kTilePairs];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.x;
  const int tok0 = tile * tt;
  const int np = tile < ntiles ? min(tt, T - tok0) * k : 0;
  const size_t pair0 = (size_t)tok0 * k;

  int v[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int p = (wave * kChunks + c) * MOE_WAVE + lane;
    v[c] = p < np ? idx[pair0 + p] : -1;
  }
  for (int r = tid; r < R; r += kThreads) {
    s_tot[r] = ws_tot[r];
    s_off[r] = ws_tot[r];
    for (int w = 0; w < kWaves; ++w) s_cnt[w][r] = 0;
  }
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int p = (wave * kChunks + c) * MOE_WAVE + lane;
    const int e = clean_expert(v[c], E);
    if (p < np) s_rank[p] = e >= 0 ? rank_of(e, epr, epr_shift) : -1;
  }
  __syncthreads();

  int key[kChunks], first[kChunks];
  uint64_t peers[kChunks];
  const int nbits = ceil_log2(R);
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int p = (wave * kChunks + c) * MOE_WAVE + lane;
    key[c] = -1;
    first[c] = -1;
    if (p < np) key[c] = rank_key(s_rank, p, k, &first[c]);
    peers[c] = peer_mask((uint32_t)key[c], key[c] >= 0, nbits);
    if (key[c] >= 0 && count_below(peers[c]) == 0) atomicAdd(&s_cnt[wave][key[c]], __popcll(peers[c]));
  }
  const int total = block_exclusive_scan(s_off, R, s_wave);
  if (tid == 0) s_off[R] = total;
  __syncthreads();
  if (tile == 0) {
    for (int r = tid; r < R; r += kThreads) {
      counts[r] = s_tot[r];
      offsets[r] = s_off[r];
    }
    if (tid == 0) offsets[R] = total;
  }
  for (int r = tid; r < R; r += kThreads) {
    int run = ws_base[(size_t)tile * R + r];
    for (int w = 0; w < kWaves; ++w) {
      s_base[w][r] = run;
      run += s_cnt[w][r];
    }
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int p = (wave * kChunks + c) * MOE_WAVE + lane;
    const int r = key[c];
    int row = -1;
    if (r >= 0) {
      const int below = count_below(peers[c]);
      row = s_off[r] + s_base[wave][r] + below;
      if (below == 0) atomicAdd(&s_base[wave][r], __popcll(peers[c]));
      s_row[p] = row;
      if (row < max_rows) row_token[row] = tok0 + p / k;
    }
    if (p < np) send_row[pair0 + p] = row;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int p = (wave * kChunks + c) * MOE_WAVE + lane;
    if (p < np) rank_row[pair0 + p] = first[c] >= 0 ? s_row[(p / k) * k + first[c]] : -1;
  }

  // rows past the last (token, rank) row are marked -1
  const int gwave = tile * kWaves + wave, nwaves = gridDim.x * kWaves;
  for (int row = total + gwave * MOE_WAVE + lane; row < max_rows; row += nwaves * MOE_WAVE)
    row_token[row] = -1;
}

// Place pass in 1024-thread blocks, one pair per thread, one block per tile:
// the expert layout's wide place pass with the (token, rank) key.
//   - SELF (all pairs in one tile, no count pass ran): the block counts its
//     keys from the per-wave counts; the layout is a single launch.
//   - otherwise rank_count_kernel has written the per-tile counts [ntiles, R]
//     and every block adds all rows (its totals) and the rows before its tile
//     (its base), one LDS atomic per nonzero entry, all loads in flight at
//     once. Used while ntiles * R fits kWideHistLoads loads per thread.
// Block 0 writes the counts and offsets; the waves of the grid mark the rows
// past the last one. Batch blockIdx.y.
template <bool SELF>
__global__ __launch_bounds__(kWideThreads) void rank_wide_kernel(
    int T, int E, int k, int R, int epr, int epr_shift, int tt, int ntiles, int max_rows,
    int r_shift, const RankLayoutBatches rb) {
  const RankLayoutBatch& bt = rb.b[blockIdx.y];
  const int32_t* __restrict__ idx = bt.idx;
  const int32_t* __restrict__ ws_rhist = static_cast<const int32_t*>(bt.workspace);
  int32_t* __restrict__ row_token = bt.row_token;
  __shared__ int s_cnt[kWideWaves][MOE_MAX_EXPERTS];
  __shared__ int s_tot[MOE_MAX_EXPERTS];
  __shared__ int s_pre[MOE_MAX_EXPERTS];
  __shared__ int s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int s_rank[kTilePairs];
  __shared__ int s_row[kTilePairs];
  __shared__ int s_wave[kWideWaves];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.x;
  const int tok0 = tile * tt;
  const int np = tile < ntiles ? min(tt, T - tok0) * k : 0;
  const size_t pair0 = (size_t)tok0 * k;
  const int raw = tid < np ? idx[pair0 + tid] : -1;
  const int hist_n = SELF ? 0 : ntiles * R;
  int h[kWideHistLoads];
#pragma unroll
  for (int j = 0; j < kWideHistLoads; ++j) {
    const int i = j * kWideThreads + tid;
    h[j] = i < hist_n ? ws_rhist[i] : 0;
  }
  if (tid < R) {
    for (int w = 0; w < kWideWaves; ++w) s_cnt[w][tid] = 0;
    s_tot[tid] = 0;
    s_pre[tid] = 0;
  }
  const int e = clean_expert(raw, E);
  if (tid < np) s_rank[tid] = e >= 0 ? rank_of(e, epr, epr_shift) : -1;
  __syncthreads();

#pragma unroll
  for (int j = 0; j < kWideHistLoads; ++j) {
    const int i = j * kWideThreads + tid;
    if (h[j] != 0) {
      const int row = row_of(i, R, r_shift), col = i - row * R;
      atomicAdd(&s_tot[col], h[j]);
      if (row < tile) atomicAdd(&s_pre[col], h[j]);
    }
  }
  // the wave's keys of one rank (one ballot per rank-id bit); the lowest
  // lane of each stores their number
  int first = -1;
  const int key = tid < np ? rank_key(s_rank, tid, k, &first) : -1;
  const uint64_t peers = peer_mask((uint32_t)key, key >= 0, ceil_log2(R));
  const int below = count_below(peers);
  if (key >= 0 && below == 0) s_cnt[wave][key] = __popcll(peers);
  __syncthreads();

  // chain the waves: s_cnt[w][r] becomes the first row of wave w's keys of
  // rank r inside the rank's region (after the tiles before)
  if (tid < R) {
    int c[kWideWaves];
#pragma unroll
    for (int w = 0; w < kWideWaves; ++w) c[w] = s_cnt[w][tid];
    int run = s_pre[tid];
#pragma unroll
    for (int w = 0; w < kWideWaves; ++w) {
      s_cnt[w][tid] = run;
      run += c[w];
    }
    if (SELF) s_tot[tid] = run;
    s_off[tid] = SELF ? run : s_tot[tid];
  }
  __syncthreads();
  const int total = block_exclusive_scan_wide(s_off, R, s_wave);
  if (tid == 0) s_off[R] = total;
  __syncthreads();
  if (tile == 0) {
    if (tid < R) {
      bt.counts[tid] = s_tot[tid];
      bt.offsets[tid] = s_off[tid];
    }
    if (tid == 0) bt.offsets[R] = total;
  }

  int row = -1;
  if (key >= 0) {
    row = s_off[key] + s_cnt[wave][key] + below;
    if (row < max_rows) row_token[row] = tok0 + tid / k;
  }
  if (tid < np) {
    s_row[tid] = row;
    bt.send_row[pair0 + tid] = row;
  }
  __syncthreads();
  if (tid < np) bt.rank_row[pair0 + tid] = first >= 0 ? s_row[(tid / k) * k + first] : -1;

  // rows past the last (token, rank) row are marked -1
  const int gwave = tile * kWideWaves + wave, nwaves = gridDim.x * kWideWaves;
  for (int r = total + gwave * MOE_WAVE + lane; r < max_rows; r += nwaves * MOE_WAVE)
    row_token[r] = -1;
}

}  // namespace

int layout_tile_tokens(int k) { return kTilePairs / k; }

int layout_num_tiles(int T, int k) {
  const int tt = layout_tile_tokens(k);
  return (T + tt - 1) / tt;
}

// Many tiles: a scan pass turns the per-tile counts ([ntiles, W]) into
// per-tile bases, so that a place block reads one row instead of the whole
// histogram.
static bool layout_scans(int ntiles, int W) {
  return ntiles >= kScanMinTiles || (long long)ntiles * W > 2 * kStage;
}

size_t layout_workspace_bytes(int T, int E, int k) {
  // per tile: E expert counts + up to E rank counts; with a scan pass also
  // the E expert and up to E rank totals
  const size_t tiles = (size_t)layout_num_tiles(T, k);
  return (tiles + (layout_scans((int)tiles, E) ? 1 : 0)) * (size_t)(2 * E) * sizeof(int32_t);
}

// Many tiles: count, scan and place passes for one batch.
static hipError_t launch_layout_scanned(int T, int E, int k, int R, int cap,
                                        const LayoutBatch& bt, hipStream_t stream) {
  const int tt = layout_tile_tokens(k);
  const int ntiles = layout_num_tiles(T, k);
  const int epr = E / R;
  const int epr_shift = (epr & (epr - 1)) == 0 ? __builtin_ctz(epr) : -1;
  const int num_rows = cap > 0 ? E * cap : T * k;
  int32_t* ws_hist = static_cast<int32_t*>(bt.workspace);
  int32_t* ws_rhist = bt.rank_token_counts != nullptr ? ws_hist + (size_t)ntiles * E : nullptr;
  int32_t* ws_tot = ws_hist + (size_t)2 * ntiles * E;
  int32_t* ws_rtot = ws_rhist != nullptr ? ws_tot + E : nullptr;
  LayoutBatches one{};
  one.b[0] = bt;
  hipLaunchKernelGGL(layout_count_kernel, dim3(ntiles), dim3(kThreads), 0, stream,
                     T, E, k, R, epr, epr_shift, tt, ntiles, one);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int ga = (E + kScanCols - 1) / kScanCols;
  const int gb = ws_rhist != nullptr ? (R + kScanCols - 1) / kScanCols : 0;
  hipLaunchKernelGGL(layout_scan_kernel, dim3(ga + gb), dim3(kScanThreads), 0, stream,
                     ntiles, E, ga, ws_hist, ws_tot, R, ws_rhist, ws_rtot);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  // padded buffers: enough waves that each fills the unused rows of about
  // one expert
  const int fill_blocks = cap > 0 ? (E + kWaves - 1) / kWaves : 1;
  const int blocks = ntiles > fill_blocks ? ntiles : fill_blocks;
  hipLaunchKernelGGL(layout_place_kernel, dim3(blocks), dim3(kThreads), 0,
                     stream, T, E, k, R, epr, epr_shift, cap, tt, ntiles, 0, num_rows,
                     bt.idx, ws_hist, ws_rhist, ws_tot, ws_rtot, bt.expert_counts,
                     bt.expert_offsets, bt.rank_counts, bt.rank_offsets, bt.rank_token_counts,
                     bt.dst_row, bt.src_pair, bt.overflow);
  return hipGetLastError();
}

hipError_t launch_layout_batches(int nb, const LayoutBatches& lb, int T, int E, int k, int R,
                                 int cap, hipStream_t stream) {
  const int tt = layout_tile_tokens(k);
  const int ntiles = layout_num_tiles(T, k);
  const int epr = E / R;
  const int num_rows = cap > 0 ? E * cap : T * k;
  const int epr_shift = (epr & (epr - 1)) == 0 ? __builtin_ctz(epr) : -1;
  const bool self_count = T * k <= kTilePairs;
  if (!self_count && layout_scans(ntiles, E)) {
    for (int b = 0; b < nb; ++b) {
      const hipError_t err = launch_layout_scanned(T, E, k, R, cap, lb.b[b], stream);
      if (err != hipSuccess) return err;
    }
    return hipSuccess;
  }
  if (nb == 0) return hipSuccess;
  if (!self_count) {
    hipLaunchKernelGGL(layout_count_kernel, dim3(ntiles, nb), dim3(kThreads), 0, stream,
                       T, E, k, R, epr, epr_shift, tt, ntiles, lb);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // one block per tile; capacity mode: enough waves that each marks the
  // unused rows of about one expert
  const int fill = cap > 0 ? (E + kWideWaves - 1) / kWideWaves : 1;
  const int blocks = ntiles > fill ? ntiles : fill;
  const auto shift = [](int n) { return (n & (n - 1)) == 0 ? __builtin_ctz(n) : -1; };
  const dim3 grid(blocks, nb);
  if (self_count)
    hipLaunchKernelGGL(layout_wide_kernel<true>, grid, dim3(kWideThreads), 0, stream, T, E, k,
                       R, epr, epr_shift, cap, tt, 1, num_rows, shift(E), shift(R), lb);
  else
    hipLaunchKernelGGL(layout_wide_kernel<false>, grid, dim3(kWideThreads), 0, stream, T, E, k,
                       R, epr, epr_shift, cap, tt, ntiles, num_rows, shift(E), shift(R), lb);
  return hipGetLastError();
}

hipError_t launch_layout(int T, int E, int k, int R, int cap, const int32_t* idx,
                         int32_t* expert_counts, int32_t* expert_offsets,
                         int32_t* rank_counts, int32_t* rank_offsets,
                         int32_t* rank_token_counts, int32_t* dst_row,
                         int32_t* src_pair, int32_t* overflow, void* workspace,
                         hipStream_t stream) {
  LayoutBatches lb{};
  lb.b[0] = LayoutBatch{idx, expert_counts, expert_offsets, rank_counts, rank_offsets,
                        rank_token_counts, dst_row, src_pair, overflow, workspace};
  return launch_layout_batches(1, lb, T, E, k, R, cap, stream);
}



size_t rank_layout_workspace_bytes(int T, int k, int R) {
  // per tile: R counts; with a scan pass also the R totals
  const size_t tiles = (size_t)layout_num_tiles(T, k);
  return (tiles + (layout_scans((int)tiles, R) ? 1 : 0)) * (size_t)R * sizeof(int32_t);
}

hipError_t launch_rank_layout_batches(int nb, const RankLayoutBatches& rb, int T, int E,
                                      int k, int R, hipStream_t stream) {
  if (nb == 0) return hipSuccess;
  const int tt = layout_tile_tokens(k);
  const int ntiles = layout_num_tiles(T, k);
  const int epr = E / R;
  const int epr_shift = (epr & (epr - 1)) == 0 ? __builtin_ctz(epr) : -1;
  const int r_shift = (R & (R - 1)) == 0 ? __builtin_ctz(R) : -1;
  const int max_rows = T * (k < R ? k : R);
  if (ntiles <= 1) {
    hipLaunchKernelGGL(rank_wide_kernel<true>, dim3(1, nb), dim3(kWideThreads), 0, stream, T, E,
                       k, R, epr, epr_shift, tt, ntiles, max_rows, r_shift, rb);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(rank_count_kernel, dim3(ntiles, nb), dim3(kThreads), 0, stream,
                     T, E, k, R, epr, epr_shift, tt, rb);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (!layout_scans(ntiles, R)) {
    hipLaunchKernelGGL(rank_wide_kernel<false>, dim3(ntiles, nb), dim3(kWideThreads), 0, stream,
                       T, E, k, R, epr, epr_shift, tt, ntiles, max_rows, r_shift, rb);
    return hipGetLastError();
  }
  // hundreds of tiles: a scan pass per batch, then the 256-thread place pass
  for (int b = 0; b < nb; ++b) {
    int32_t* ws = static_cast<int32_t*>(rb.b[b].workspace);
    hipLaunchKernelGGL(layout_scan_kernel, dim3((R + kScanCols - 1) / kScanCols),
                       dim3(kScanThreads), 0, stream, ntiles, R,
                       (R + kScanCols - 1) / kScanCols, ws, ws + (size_t)ntiles * R, 0,
                       static_cast<const int32_t*>(nullptr), static_cast<int32_t*>(nullptr));
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(rank_place_kernel, dim3(ntiles, nb), dim3(kThreads), 0, stream, T, E, k, R,
                     epr, epr_shift, tt, ntiles, max_rows, rb);
  return hipGetLastError();
}

hipError_t launch_rank_layout(int T, int E, int k, int R, const int32_t* idx,
                              int32_t* counts, int32_t* offsets, int32_t* rank_row,
                              int32_t* send_row, int32_t* row_token, void* workspace,
                              hipStream_t stream) {
  RankLayoutBatches rb{};
  rb.b[0] = RankLayoutBatch{idx, counts, offsets, rank_row, send_row, row_token, workspace};
  return launch_rank_layout_batches(1, rb, T, E, k, R, stream);
}

bool layout_dispatch_fused(int T, int k, int cap) {
  return cap > 0 && T > 0 && T * k <= kTilePairs;
}

hipError_t launch_layout_dispatch(int T, int E, int k, int R, int cap, const int32_t* idx,
                                  int32_t* expert_counts, int32_t* expert_offsets,
                                  int32_t* rank_counts, int32_t* rank_offsets,
                                  int32_t* rank_token_counts, int32_t* dst_row,
                                  int32_t* src_pair, int32_t* overflow, void* workspace,
                                  int H, const void* x, int dtype, void* out, void* out_scales,
                                  hipStream_t stream) {
  const int num_rows = cap > 0 ? E * cap : T * k;
  if (!layout_dispatch_fused(T, k, cap)) {
    hipError_t err = launch_layout(T, E, k, R, cap, idx, expert_counts, expert_offsets,
                                   rank_counts, rank_offsets, rank_token_counts, dst_row,
                                   src_pair, overflow, workspace, stream);
    if (err != hipSuccess) return err;
    if (dtype == MOE_DTYPE_FP8_E4M3)
      return launch_dispatch_fp8(T, H, k, num_rows, x, dst_row, out,
                                 static_cast<float*>(out_scales), stream);
    if (dtype == MOE_DTYPE_MXFP8_E4M3)
      return launch_dispatch_mxfp8(T, H, k, num_rows, x, dst_row, out,
                                   static_cast<uint8_t*>(out_scales), stream);
    return launch_dispatch_bf16(T, H, k, num_rows, x, dst_row, out, stream);
  }
  const int tt = layout_tile_tokens(k);
  const int epr = E / R;
  const int epr_shift = (epr & (epr - 1)) == 0 ? __builtin_ctz(epr) : -1;
  // layout blocks as in the single-launch layout (capacity mode)
  const int fill_blocks = (E + kWaves - 1) / kWaves;
  const int place_blocks = (T * k + kThreads - 1) / kThreads;
  const int nl = place_blocks > fill_blocks ? place_blocks : fill_blocks;
  // dispatch blocks as in the dispatch launches
  int parts, per_part;
  if (dtype == MOE_DTYPE_FP8_E4M3)
    split_row(T, H / MOE_FP8_BLOCK, kFp8StepBlocks, 64 * kScaleSlots, &parts, &per_part);
  else if (dtype == MOE_DTYPE_MXFP8_E4M3)
    split_row(T, H / MOE_MX_BLOCK, kMxStepBlocks, 64 * kScaleSlots, &parts, &per_part);
  else
    split_row(T, H / 8, MOE_WAVE, 1 << 30, &parts, &per_part);
  const int nd = (T * parts + kWavesPerBlock - 1) / kWavesPerBlock;
  const dim3 grid(nl + nd), block(kThreads);
  const u32x4* xs = static_cast<const u32x4*>(x);
#define MOE_LD_ARGS nl, T, E, k, R, epr, epr_shift, cap, tt, num_rows, idx, expert_counts, \
    expert_offsets, rank_counts, rank_offsets, rank_token_counts, dst_row, src_pair, overflow, \
    H, parts, per_part, xs, out, out_scales
  if (dtype == MOE_DTYPE_FP8_E4M3)
    hipLaunchKernelGGL(layout_dispatch_kernel<MOE_DTYPE_FP8_E4M3>, grid, block, 0, stream,
                       MOE_LD_ARGS);
  else if (dtype == MOE_DTYPE_MXFP8_E4M3)
    hipLaunchKernelGGL(layout_dispatch_kernel<MOE_DTYPE_MXFP8_E4M3>, grid, block, 0, stream,
                       MOE_LD_ARGS);
  else
    hipLaunchKernelGGL(layout_dispatch_kernel<MOE_DTYPE_BF16>, grid, block, 0, stream,
                       MOE_LD_ARGS);
#undef MOE_LD_ARGS
  return hipGetLastError();
}

}  // namespace moe
