// Deduplicated dispatch and hierarchical combine on gfx950.
//
// Source: hyper.ai story on NVIDIA Hybrid-EP: the combine reduces
// hierarchically, first the results inside one destination, then across
// destinations. Here a destination is a rank of the glossary's placement
// ("Expert Parallelism", "Le principe de base": rank r owns whole experts
// [r*E/R, (r+1)*E/R)). One row per (token, rank) is sent (moe_dispatch with
// the send rows); the rank fans it out to the rows of its experts (expand);
// after the experts, the rank reduces each token's weighted outputs into one
// partial row (combine_local), and each token sums its partial rows
// (the unit-weight combine over the send rows).
//
//   expand:         out[q]  = rank_rows[rank_row[src_pair[q]]]      (bytes)
//   combine_local:  part[s] = bf16( sum over the token's slots j with
//                             rank_row[t, j] = s of w[t, j] * y[dst_row[t, j]] )

#include "kernels.h"
#include "wave.h"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kExpandChunks = 8;   // 16-byte chunks in flight per lane
// Workgroups per CU (occupancy caps, see lds_cap_bytes), measured on dsv3:
// expand about 2% faster at 3; the partial combine (1 KiB items) 2% faster
// at 2 than at 3, 28% faster than at 1.
constexpr int kExpandBlocksPerCu = 3;
constexpr int kCombineLocalBlocksPerCu = 2;

// One wave per destination row: the 16-byte chunks of the payload, then the
// scale bytes (as words when the row's scale bytes are a multiple of 4).
template <bool kScaleWords>
__global__ __launch_bounds__(256) void expand_kernel(
    int num_rows, int num_pairs, int num_rank_rows, int nch, int sbytes,
    const u32x4* __restrict__ src, const uint8_t* __restrict__ src_scales,
    const int32_t* __restrict__ rank_row, const int32_t* __restrict__ src_pair,
    u32x4* __restrict__ out, uint8_t* __restrict__ out_scales) {
  const int lane = threadIdx.x & 63;
  const int q = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (q >= num_rows) return;
  const int p = src_pair[q];
  if (p < 0 || p >= num_pairs) return;            // the row holds no pair
  const int s = rank_row[p];
  if (s < 0 || s >= num_rank_rows) return;
  const u32x4* a = src + (size_t)s * nch;
  u32x4* b = out + (size_t)q * nch;
  for (int base = 0; base < nch; base += MOE_WAVE * kExpandChunks) {
    u32x4 v[kExpandChunks];
#pragma unroll
    for (int u = 0; u < kExpandChunks; ++u) {
      const int c = base + u * MOE_WAVE + lane;
      v[u] = u32x4{0u, 0u, 0u, 0u};
      if (c < nch) v[u] = a[c];
    }
#pragma unroll
    for (int u = 0; u < kExpandChunks; ++u) {
      const int c = base + u * MOE_WAVE + lane;
      if (c < nch) stream_store(v[u], b + c);
    }
  }
  if (sbytes == 0) return;
  if (kScaleWords) {
    const uint32_t* sa = reinterpret_cast<const uint32_t*>(src_scales + (size_t)s * sbytes);
    uint32_t* sb = reinterpret_cast<uint32_t*>(out_scales + (size_t)q * sbytes);
    for (int i = lane; i < sbytes / 4; i += MOE_WAVE) sb[i] = sa[i];
  } else {
    const uint8_t* sa = src_scales + (size_t)s * sbytes;
    uint8_t* sb = out_scales + (size_t)q * sbytes;
    for (int i = lane; i < sbytes; i += MOE_WAVE) sb[i] = sa[i];
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

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
  for (int q = 0; q < 4; ++q) r[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
  return r;
}

// Slot order of the local reduction, computed in lanes 0..k-1: the slots
// with a (token, rank) row come first, grouped by row (groups in the order
// of their first slot), slot order inside a group. Returns the position of
// the calling lane's slot in that order; *nvalid = slots with a row.
__device__ __forceinline__ int group_order(int my_s, int k, int* nvalid) {
  const int lane = lane_id();
  int lead = lane;
  for (int o = 0; o < k; ++o) {
    const int so = read_lane(my_s, o);
    if (so == my_s && o < lead) lead = o;
  }
  const bool valid = lane < k && my_s >= 0;
  const int key = valid ? lead * MOE_MAX_TOPK + lane : MOE_MAX_TOPK * MOE_MAX_TOPK + lane;
  int pos = 0;
  for (int o = 0; o < k; ++o) pos += read_lane(key, o) < key ? 1 : 0;
  *nvalid = __popcll(wave_ballot(valid));
  return pos;
}

// Lane (slot) at position i of the order.
__device__ __forceinline__ int slot_at(int pos, int k, int i) {
  return (int)__builtin_ctzll(wave_ballot(lane_id() < k && pos == i));
}

// K > 0: compile-time top-k, all K rows of a column step loaded first.
template <int K, int U>
__global__ __launch_bounds__(256) void combine_local_kernel(
    int T, int nch, int parts, int cpp, int num_rows, int num_rank_rows,
    const u32x4* __restrict__ y, const int32_t* __restrict__ dst_row,
    const int32_t* __restrict__ rank_row, const float* __restrict__ w,
    u32x4* __restrict__ partial) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (gw >= T * parts) return;
  const int t = gw / parts;
  const int c0 = (gw - t * parts) * cpp;
  const int cnt = min(cpp, nch - c0);
  int my_d = lane < K ? dst_row[(size_t)t * K + lane] : -1;
  int my_s = lane < K ? rank_row[(size_t)t * K + lane] : -1;
  const float my_w = lane < K ? w[(size_t)t * K + lane] : 0.0f;
  if (my_d >= num_rows) my_d = -1;
  if (my_s >= num_rank_rows) my_s = -1;

  int nvalid;
  const int pos = group_order(my_s, K, &nvalid);
  int d[K], s[K];
  float wj[K];
  bool last[K];
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const int j = slot_at(pos, K, i);
    d[i] = i < nvalid ? read_lane(my_d, j) : -1;
    s[i] = i < nvalid ? read_lane(my_s, j) : -1;
    wj[i] = read_lane(my_w, j);
  }
#pragma unroll
  for (int i = 0; i < K; ++i) last[i] = i < nvalid && (i + 1 == nvalid || s[i + 1] != s[i]);

  for (int base = 0; base < cnt; base += MOE_WAVE * U) {
    u32x4 v[K][U];
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const u32x4* row = y + (size_t)(d[i] < 0 ? 0 : d[i]) * nch + c0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = base + u * MOE_WAVE + lane;
        v[i][u] = u32x4{0u, 0u, 0u, 0u};
        if (d[i] >= 0 && c < cnt) v[i][u] = stream_load(row + c);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = base + u * MOE_WAVE + lane;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < K; ++i) {
        if (d[i] >= 0) fma_row(acc, wj[i], v[i][u]);
        if (last[i]) {
          if (c < cnt) stream_store(pack_row(acc), partial + (size_t)s[i] * nch + c0 + c);
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
        }
      }
    }
  }
}

// Any k: one slot's row at a time.
__global__ __launch_bounds__(256) void combine_local_kernel_any_k(
    int T, int k, int nch, int parts, int cpp, int num_rows, int num_rank_rows,
    const u32x4* __restrict__ y, const int32_t* __restrict__ dst_row,
    const int32_t* __restrict__ rank_row, const float* __restrict__ w,
    u32x4* __restrict__ partial) {
  constexpr int U = 4;
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (gw >= T * parts) return;
  const int t = gw / parts;
  const int c0 = (gw - t * parts) * cpp;
  const int cnt = min(cpp, nch - c0);
  int my_d = lane < k ? dst_row[(size_t)t * k + lane] : -1;
  int my_s = lane < k ? rank_row[(size_t)t * k + lane] : -1;
  const float my_w = lane < k ? w[(size_t)t * k + lane] : 0.0f;
  if (my_d >= num_rows) my_d = -1;
  if (my_s >= num_rank_rows) my_s = -1;
  int nvalid;
  const int pos = group_order(my_s, k, &nvalid);

  for (int base = 0; base < cnt; base += MOE_WAVE * U) {
    float acc[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[u][q] = 0.0f;
    int j = nvalid > 0 ? slot_at(pos, k, 0) : 0;
    for (int i = 0; i < nvalid; ++i) {
      const int d = read_lane(my_d, j);
      const int s = read_lane(my_s, j);
      const float wi = read_lane(my_w, j);
      const int jn = i + 1 < nvalid ? slot_at(pos, k, i + 1) : j;
      const bool last = i + 1 == nvalid || read_lane(my_s, jn) != s;
      if (d >= 0) {
        const u32x4* row = y + (size_t)d * nch + c0;
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = base + u * MOE_WAVE + lane;
          v[u] = u32x4{0u, 0u, 0u, 0u};
          if (c < cnt) v[u] = stream_load(row + c);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) fma_row(acc[u], wi, v[u]);
      }
      if (last) {
        u32x4* dst = partial + (size_t)s * nch + c0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = base + u * MOE_WAVE + lane;
          if (c < cnt) stream_store(pack_row(acc[u]), dst + c);
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[u][q] = 0.0f;
        }
      }
      j = jn;
    }
  }
}

template <int K, int U>
void launch_local_fixed(dim3 grid, hipStream_t stream, int T, int nch, int parts, int cpp,
                        int num_rows, int num_rank_rows, const void* y, const int32_t* dst_row,
                        const int32_t* rank_row, const float* w, void* partial) {
  hipLaunchKernelGGL((combine_local_kernel<K, U>), grid, dim3(256),
                     lds_cap_bytes(kCombineLocalBlocksPerCu), stream, T, nch, parts, cpp,
                     num_rows, num_rank_rows, static_cast<const u32x4*>(y), dst_row, rank_row,
                     w, static_cast<u32x4*>(partial));
}

}  // namespace

hipError_t launch_expand(int T, int H, int k, int dtype, int num_rank_rows, const void* src,
                         const void* src_scales, const int32_t* rank_row, int num_rows,
                         const int32_t* src_pair, void* out, void* out_scales,
                         hipStream_t stream) {
  if (num_rows == 0) return hipSuccess;
  const int pbytes = dtype == MOE_DTYPE_BF16 ? 2 * H : H;
  const int sbytes = dtype == MOE_DTYPE_FP8_E4M3 ? (H / MOE_FP8_BLOCK) * 4
                     : dtype == MOE_DTYPE_MXFP8_E4M3 ? H / MOE_MX_BLOCK : 0;
  const dim3 grid((num_rows + kWavesPerBlock - 1) / kWavesPerBlock);
  const bool words = sbytes % 4 == 0;
  if (words)
    hipLaunchKernelGGL(expand_kernel<true>, grid, dim3(256), lds_cap_bytes(kExpandBlocksPerCu),
                       stream, num_rows, T * k, num_rank_rows, pbytes / 16, sbytes,
                       static_cast<const u32x4*>(src),
                       static_cast<const uint8_t*>(src_scales), rank_row, src_pair,
                       static_cast<u32x4*>(out), static_cast<uint8_t*>(out_scales));
  else
    hipLaunchKernelGGL(expand_kernel<false>, grid, dim3(256), lds_cap_bytes(kExpandBlocksPerCu),
                       stream, num_rows, T * k, num_rank_rows, pbytes / 16, sbytes,
                       static_cast<const u32x4*>(src),
                       static_cast<const uint8_t*>(src_scales), rank_row, src_pair,
                       static_cast<u32x4*>(out), static_cast<uint8_t*>(out_scales));
  return hipGetLastError();
}

hipError_t launch_combine_local(int T, int H, int k, int num_rows, int num_rank_rows,
                                const void* y, const int32_t* dst_row, const int32_t* rank_row,
                                const float* w, void* partial, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int nch = H / 8;
  // k = 8: items of 1 KiB (one 16-byte chunk per lane), as many parts as a
  // row has. On the DeepSeek-V3 shape (rows of 14 KiB, about 7 partial rows
  // per token) that took 160.1-160.6 us against 165-169 us with 2 KiB items
  // (3 KiB: 168-170, 4 KiB: 166-170; same box, 20 back-to-back launches).
  int parts = k == 8 ? nch / MOE_WAVE : (kTargetWaves + T - 1) / T;
  parts = max(1, min(parts, nch / MOE_WAVE));
  int cpp = (nch + parts - 1) / parts;
  cpp = (cpp + MOE_WAVE - 1) / MOE_WAVE * MOE_WAVE;
  parts = (nch + cpp - 1) / cpp;
  const dim3 grid((T * parts + kWavesPerBlock - 1) / kWavesPerBlock);
  switch (k) {
    case 1: launch_local_fixed<1, 4>(grid, stream, T, nch, parts, cpp, num_rows, num_rank_rows, y, dst_row, rank_row, w, partial); break;
    case 2: launch_local_fixed<2, 4>(grid, stream, T, nch, parts, cpp, num_rows, num_rank_rows, y, dst_row, rank_row, w, partial); break;
    case 4: launch_local_fixed<4, 2>(grid, stream, T, nch, parts, cpp, num_rows, num_rank_rows, y, dst_row, rank_row, w, partial); break;
    case 8: launch_local_fixed<8, 1>(grid, stream, T, nch, parts, cpp, num_rows, num_rank_rows, y, dst_row, rank_row, w, partial); break;
    default:
      hipLaunchKernelGGL(combine_local_kernel_any_k, grid, dim3(256), 0, stream, T, k, nch,
                         parts, cpp, num_rows, num_rank_rows, static_cast<const u32x4*>(y),
                         dst_row, rank_row, w, static_cast<u32x4*>(partial));
  }
  return hipGetLastError();
}

}  // namespace moe
