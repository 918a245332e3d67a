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
//   expand:         out[dst_row[t, j]] = rank_rows[s] for the slots j of
//                   t = row_token[s] with rank_row[t, j] = s         (bytes)
//   combine_local:  part[s] = bf16( sum over the slots j of t = row_token[s]
//                             with rank_row[t, j] = s of w[t, j] * y[dst_row[t, j]] )

#include "kernels.h"
#include "wave.h"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;
// Workgroups per CU (occupancy caps, see lds_cap_bytes), measured on dsv3:
// expand (7 KiB items) 64.9-65.2 us per launch at 2, 65.9-66.1 at 3,
// 67.1-67.4 at 5. The partial combine (4 KiB items) ran 139.2-139.8 us
// per launch at 5 to 8, 141-147 at 4, 221 at 2.
constexpr int kExpandBlocksPerCu = 2;
// 16-byte chunks per lane of one expand item: items of 7 KiB, one whole
// FP8 row at hidden = 7168.
constexpr int kExpandChunks = 7;
constexpr int kCombineLocalBlocksPerCu = 6;
// 16-byte chunks per lane of one partial-combine item: items of 4 KiB.
constexpr int kLocalChunks = 4;

// One wave per (row s, column part): the row's token t = row_token[s] and
// its slots j with rank_row[t, j] = s and an expert row (a ballot in lanes
// 0..k-1); the part is read once and written to each of those expert rows,
// and the part-0 wave copies the scale bytes (as words when the row's scale
// bytes are a multiple of 4). The rows are taken in their own order, so the
// received rows are read one after the other and each rank's expert rows
// are written together. On the DeepSeek-V3 shape (FP8 rows of 7 KiB) this
// took 64.9-65.4 us per launch against 68.4-68.9 us for one wave per expert
// row gathering its source row (which reads a row once per expert of its
// rank); 1 KiB items 70.8-71.2 us, 2 KiB 66.1-67.1 (same box, 20
// back-to-back launches, equal bytes).
template <bool kScaleWords>
__global__ __launch_bounds__(256) void expand_kernel(
    int T, int k, int num_rank_rows, int nch, int parts, int cpp, int sbytes, int num_rows,
    const u32x4* __restrict__ src, const uint8_t* __restrict__ src_scales,
    const int32_t* __restrict__ rank_row, const int32_t* __restrict__ row_token,
    const int32_t* __restrict__ dst_row, u32x4* __restrict__ out,
    uint8_t* __restrict__ out_scales) {
  constexpr int U = kExpandChunks;
  const int lane = threadIdx.x & 63;
  const long long gw = (long long)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (gw >= (long long)num_rank_rows * parts) return;
  const int s = (int)(gw / parts);
  const int part = (int)(gw - (long long)s * parts);
  const int c0 = part * cpp;
  const int cnt = min(cpp, nch - c0);
  const int t = row_token[s];
  if (t < 0 || t >= T) return;                     // past the last row
  const int my_q = lane < k ? dst_row[(size_t)t * k + lane] : -1;
  const int my_s = lane < k ? rank_row[(size_t)t * k + lane] : -1;
  const uint64_t slots = wave_ballot(lane < k && my_s == s && my_q >= 0 && my_q < num_rows);
  if (slots == 0) return;
  const u32x4* a = src + (size_t)s * nch + c0;
  for (int base = 0; base < cnt; base += MOE_WAVE * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = base + u * MOE_WAVE + lane;
      v[u] = u32x4{0u, 0u, 0u, 0u};
      if (c < cnt) v[u] = a[c];
    }
    for (uint64_t m = slots; m != 0; m &= m - 1) {
      u32x4* b = out + (size_t)read_lane(my_q, (int)__builtin_ctzll(m)) * nch + c0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = base + u * MOE_WAVE + lane;
        if (c < cnt) stream_store(v[u], b + c);
      }
    }
  }
  if (part != 0 || sbytes == 0) return;
  for (uint64_t m = slots; m != 0; m &= m - 1) {
    const int q = read_lane(my_q, (int)__builtin_ctzll(m));
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

// One wave per (row s, column part): the row's token t = row_token[s], its
// slots j with rank_row[t, j] = s and a kept expert row (a ballot in lanes
// 0..k-1, visited in slot order), one fp32 FMA chain per column, one bf16
// rounding. The rows are taken in their own order, so the partial rows are
// written one after the other and each rank's expert rows are read while
// that rank's rows are reduced: the order in which the receiving rank
// reduces what it holds. On the DeepSeek-V3 shape (14 KiB rows) this took
// 139.2-139.8 us per launch against 160.6-162.8 us for one wave per (token,
// 1 KiB part) reducing all of the token's ranks (same box, 20 back-to-back
// launches, equal partial bits); 1 KiB items at this order 166-167 us,
// 2 KiB 140.5-141, 7 KiB 141-142.
__global__ __launch_bounds__(256) void combine_local_kernel(
    int T, int k, int nrr, int nch, int parts, int cpp, int num_rows,
    const u32x4* __restrict__ y, const int32_t* __restrict__ dst_row,
    const int32_t* __restrict__ rank_row, const int32_t* __restrict__ row_token,
    const float* __restrict__ w, u32x4* __restrict__ partial) {
  constexpr int U = kLocalChunks;
  const int lane = threadIdx.x & 63;
  const long long gw = (long long)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (gw >= (long long)nrr * parts) return;
  const int s = (int)(gw / parts);
  const int c0 = (int)(gw - (long long)s * parts) * cpp;
  const int cnt = min(cpp, nch - c0);
  const int t = row_token[s];
  if (t < 0 || t >= T) return;                     // past the last row
  int my_d = lane < k ? dst_row[(size_t)t * k + lane] : -1;
  const int my_s = lane < k ? rank_row[(size_t)t * k + lane] : -1;
  const float my_w = lane < k ? w[(size_t)t * k + lane] : 0.0f;
  if (my_d >= num_rows) my_d = -1;
  const uint64_t slots = wave_ballot(lane < k && my_s == s && my_d >= 0);
  for (int base = 0; base < cnt; base += MOE_WAVE * U) {
    float acc[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[u][q] = 0.0f;
    for (uint64_t m = slots; m != 0; m &= m - 1) {
      const int j = (int)__builtin_ctzll(m);
      const u32x4* row = y + (size_t)read_lane(my_d, j) * nch + c0;
      const float wj = read_lane(my_w, j);
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
    u32x4* dst = partial + (size_t)s * nch + c0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = base + u * MOE_WAVE + lane;
      if (c < cnt) stream_store(pack_row(acc[u]), dst + c);
    }
  }
}

}  // namespace

hipError_t launch_expand(int T, int H, int k, int dtype, int num_rank_rows, const void* src,
                         const void* src_scales, const int32_t* rank_row,
                         const int32_t* row_token, int num_rows, const int32_t* dst_row,
                         void* out, void* out_scales, hipStream_t stream) {
  if (num_rows == 0 || num_rank_rows == 0 || T == 0) return hipSuccess;
  const int pbytes = dtype == MOE_DTYPE_BF16 ? 2 * H : H;
  const int sbytes = dtype == MOE_DTYPE_FP8_E4M3 ? (H / MOE_FP8_BLOCK) * 4
                     : dtype == MOE_DTYPE_MXFP8_E4M3 ? H / MOE_MX_BLOCK : 0;
  const int nch = pbytes / 16;
  const int cpp = MOE_WAVE * kExpandChunks;
  const int parts = (nch + cpp - 1) / cpp;
  const long long waves = (long long)num_rank_rows * parts;
  const dim3 grid((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock));
  if (sbytes % 4 == 0)
    hipLaunchKernelGGL(expand_kernel<true>, grid, dim3(256), lds_cap_bytes(kExpandBlocksPerCu),
                       stream, T, k, num_rank_rows, nch, parts, cpp, sbytes, num_rows,
                       static_cast<const u32x4*>(src), static_cast<const uint8_t*>(src_scales),
                       rank_row, row_token, dst_row, static_cast<u32x4*>(out),
                       static_cast<uint8_t*>(out_scales));
  else
    hipLaunchKernelGGL(expand_kernel<false>, grid, dim3(256), lds_cap_bytes(kExpandBlocksPerCu),
                       stream, T, k, num_rank_rows, nch, parts, cpp, sbytes, num_rows,
                       static_cast<const u32x4*>(src), static_cast<const uint8_t*>(src_scales),
                       rank_row, row_token, dst_row, static_cast<u32x4*>(out),
                       static_cast<uint8_t*>(out_scales));
  return hipGetLastError();
}

hipError_t launch_combine_local(int T, int H, int k, int num_rows, int num_rank_rows,
                                const void* y, const int32_t* dst_row, const int32_t* rank_row,
                                const int32_t* row_token, const float* w, void* partial,
                                hipStream_t stream) {
  if (T == 0 || num_rank_rows == 0) return hipSuccess;
  const int nch = H / 8;
  const int cpp = MOE_WAVE * kLocalChunks;
  const int parts = (nch + cpp - 1) / cpp;
  const long long waves = (long long)num_rank_rows * parts;
  const dim3 grid((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock));
  hipLaunchKernelGGL(combine_local_kernel, grid, dim3(256),
                     lds_cap_bytes(kCombineLocalBlocksPerCu), stream, T, k, num_rank_rows, nch,
                     parts, cpp, num_rows, static_cast<const u32x4*>(y), dst_row, rank_row,
                     row_token, w, static_cast<u32x4*>(partial));
  return hipGetLastError();
}

}  // namespace moe
