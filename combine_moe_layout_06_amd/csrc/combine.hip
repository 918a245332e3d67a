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
// With no weights (w == nullptr) every weight is 1: that is the gradient of
// dispatch with respect to x (each token sums the gradients of its rows).
//
// One 64-lane wave per (token, column part). For a compile-time k the wave
// issues the loads of all k rows (16 bytes per lane each) before the first
// FMA, so k x 1 KiB per wave are in flight; the fp32 accumulators are
// rounded once to bf16 (nearest even) and stored with one 16-byte store.

#include <atomic>

#include "kernels.h"
#include "wave.h"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;
// Workgroups per CU for the fixed-k combine (measured on dsv3, qwen3_skew
// and mixtral shapes: 3 is 1-3% faster than the 5-8 the registers allow).
constexpr int kCombineBlocksPerCu = 3;

#ifndef MOE_COMBINE_U8
#define MOE_COMBINE_U8 2   // 16-byte chunks per lane per step when k = 8
#endif

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
  const float my_w = lane < K ? (w != nullptr ? w[(size_t)t * K + lane] : 1.0f) : 0.0f;

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

// k = 8, held outputs: each wave takes IPW consecutive (token, part) items
// (a part is 128 chunks of 16 bytes, two per lane), keeps their rounded
// outputs in registers (8 per item) and stores all of them after the last
// item's rows have been read. The next item's rows and weights are loaded
// while the current rows are in flight. Launched at kHeldBlocksPerCu, so the
// grid (at most held_waves() waves) is resident at once: the chip reads the
// expert rows first and writes the outputs in one burst at the end, instead
// of mixing the output stores into the read stream. The arithmetic is the
// combine_kernel's: the same fma chain in slot order and one rounding.
constexpr int kHeldPart = 2 * MOE_WAVE;              // chunks per item
constexpr int kHeldBlocksPerCu = 2;                  // ~210 registers per lane

// Compute units of the current device, read once per device; 0 if the count
// cannot be read.
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 0;
  }
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0) {
      (void)hipGetLastError();
      return 0;
    }
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Waves the device holds at once at kHeldBlocksPerCu (2,048 on a whole
// MI355X, 256 CUs); 0 if the CU count cannot be read. A partition with fewer
// CUs gets a smaller grid, which the bounds on items per wave below then
// usually turn away.
long long held_waves() {
  return (long long)device_cus() * kHeldBlocksPerCu * kWavesPerBlock;
}
constexpr int kHeldMinItems = 8, kHeldMaxItems = 16;
// Rows of at least 7 parts (hidden > 6144): measured against the per-item
// kernel at k = 8, held outputs were 3-10% faster on rows of 7 parts (hidden
// 7040 and 7168) and 0-7% slower on rows of 4 parts (hidden 4096), equal on
// 2 parts. With short rows the wave's walk along a row costs more than the
// burst saves.
constexpr int kHeldMinParts = 7;

template <int K, int IPW>
__global__ __launch_bounds__(256) void combine_held_kernel(
    int T, int nch, int parts, int num_rows, const u32x4* __restrict__ y,
    const int32_t* __restrict__ dst_row, const float* __restrict__ w,
    u32x4* __restrict__ out) {
  constexpr int U = kHeldPart / MOE_WAVE;
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int items = T * parts;
  const int first = gw * IPW;
  if (first >= items) return;
  int tcur = first / parts;
  int nd = lane < K ? dst_row[(size_t)tcur * K + lane] : -1;
  float nwt = lane < K ? (w != nullptr ? w[(size_t)tcur * K + lane] : 1.0f) : 0.0f;

  u32x4 res[IPW][U];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int it = first + i;
#pragma unroll
    for (int u = 0; u < U; ++u) res[i][u] = u32x4{0u, 0u, 0u, 0u};
    if (it < items) {
      const int t = it / parts;
      const int c0 = (it - t * parts) * kHeldPart;
      int d[K];
      float wj[K];
#pragma unroll
      for (int j = 0; j < K; ++j) {
        d[j] = read_lane(nd, j);
        wj[j] = read_lane(nwt, j);
        if (d[j] >= num_rows) d[j] = -1;
      }
      u32x4 v[K][U];
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const u32x4* row = y + (size_t)(d[j] < 0 ? 0 : d[j]) * nch;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + u * MOE_WAVE + lane;
          v[j][u] = u32x4{0u, 0u, 0u, 0u};
          if (d[j] >= 0 && c < nch) v[j][u] = stream_load(row + c);
        }
      }
      // the next item's rows and weights, when it starts a new token
      if (i + 1 < IPW && it + 1 < items) {
        const int tn = (it + 1) / parts;
        if (tn != tcur) {
          tcur = tn;
          nd = lane < K ? dst_row[(size_t)tn * K + lane] : -1;
          nwt = lane < K ? (w != nullptr ? w[(size_t)tn * K + lane] : 1.0f) : 0.0f;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < K; ++j)
          if (d[j] >= 0) fma_row(acc, wj[j], v[j][u]);
        res[i][u] = pack_row(acc);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int it = first + i;
    if (it < items) {
      const int t = it / parts;
      const int c0 = (it - t * parts) * kHeldPart;
      u32x4* dst = out + (size_t)t * nch;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * MOE_WAVE + lane;
        if (c < nch) stream_store(res[i][u], dst + c);
      }
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
  const float my_w = lane < k ? (w != nullptr ? w[(size_t)t * k + lane] : 1.0f) : 0.0f;
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


// ---------------------------------------------------------------------------
// Backward of combine: for each live pair (t, j) with row d = dst_row[t, j]
//   dy[d, :] = bf16( w[t, j] * dout[t, :] )
//   dw[t, j] = sum_h dout[t, h] * y[d, h]        (fp32)
// Two launches, each at its own access pattern's ceiling: the dw launch only
// reads (the expert rows and dout), the dy launch only fans dout out. In one
// kernel the random-row reads and writes mixed at 5.0 TB/s (193-194 us on
// the DeepSeek-V3 shape); apart they take 77.7 us (6.8 TB/s) and 99 us.
// ---------------------------------------------------------------------------
constexpr int kBwdChunks = 4;
// dy launch: 1 KiB pieces, workgroups per CU (measured on the DeepSeek-V3
// shape, dy launch with the dw launch: 177.0-177.7 us at 5, 177.4-179.4 at 6,
// 182.6-182.8 at 4, 184.6-185.2 at 8, 183.9-185.3 uncapped; one 256-thread
// block per token with 4 KiB pieces: 183.0-184.5)
constexpr int kBwdDyBlocksPerCu = 5;

__device__ __forceinline__ float dot8(const u32x4& a, const u32x4& b, float acc) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc = __builtin_fmaf(bf16_lo(a[q]), bf16_lo(b[q]), acc);
    acc = __builtin_fmaf(bf16_hi(a[q]), bf16_hi(b[q]), acc);
  }
  return acc;
}

__device__ __forceinline__ u32x4 scale_row(const u32x4& g, float w) {
  u32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    r[q] = pack_bf16x2(w * bf16_lo(g[q]), w * bf16_hi(g[q]));
  return r;
}

// dw: one 256-thread block per token; wave v covers chunk groups v, v + 4,
// ... of the row (kBwdChunks 16-byte chunks per lane per group). Its dout
// chunks stay in registers while it walks the k rows; each pair's dot
// product is reduced in the wave and the four waves' partial sums are added
// in wave order, so the result is deterministic.
__global__ __launch_bounds__(256) void combine_backward_dw_kernel(
    int T, int k, int nch, int num_rows, const u32x4* __restrict__ dout,
    const u32x4* __restrict__ y, const int32_t* __restrict__ dst_row, float* __restrict__ dw) {
  __shared__ float s_part[kWavesPerBlock][MOE_MAX_TOPK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x;
  const int my_dst = lane < k ? dst_row[(size_t)t * k + lane] : -1;
  if (lane < k) s_part[wave][lane] = 0.0f;
  const u32x4* g_row = dout + (size_t)t * nch;
  constexpr int kGroup = MOE_WAVE * kBwdChunks;

  for (int c0 = wave * kGroup; c0 < nch; c0 += kWavesPerBlock * kGroup) {
    u32x4 g[kBwdChunks];
#pragma unroll
    for (int u = 0; u < kBwdChunks; ++u) {
      const int c = c0 + u * MOE_WAVE + lane;
      g[u] = u32x4{0u, 0u, 0u, 0u};
      if (c < nch) g[u] = stream_load(g_row + c);
    }
    for (int j = 0; j < k; ++j) {
      const int d = read_lane(my_dst, j);
      if (d < 0 || d >= num_rows) continue;
      const u32x4* y_row = y + (size_t)d * nch;
      u32x4 v[kBwdChunks];
#pragma unroll
      for (int u = 0; u < kBwdChunks; ++u) {
        const int c = c0 + u * MOE_WAVE + lane;
        v[u] = u32x4{0u, 0u, 0u, 0u};
        if (c < nch) v[u] = stream_load(y_row + c);
      }
      float part = 0.0f;
#pragma unroll
      for (int u = 0; u < kBwdChunks; ++u) part = dot8(g[u], v[u], part);
      const float sum = wave_sum_f32(part);
      if (lane == 0) s_part[wave][j] += sum;
    }
  }
  __syncthreads();
  if (wave == 0 && lane < k) {
    float acc = 0.0f;
#pragma unroll
    for (int v = 0; v < kWavesPerBlock; ++v) acc += s_part[v][lane];
    dw[(size_t)t * k + lane] = (my_dst >= 0 && my_dst < num_rows) ? acc : 0.0f;
  }
}

// dy: one wave per (token, 1 KiB piece of the row): the piece of dout in
// one 16-byte chunk per lane, scaled and written to each of the token's rows.
__global__ __launch_bounds__(256) void combine_backward_dy_kernel(
    int T, int k, int nch, int parts, int num_rows, const u32x4* __restrict__ dout,
    const int32_t* __restrict__ dst_row, const float* __restrict__ w, u32x4* __restrict__ dy) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (gw >= T * parts) return;
  const int t = gw / parts;
  const int c = (gw - t * parts) * MOE_WAVE + lane;
  const int my_dst = lane < k ? dst_row[(size_t)t * k + lane] : -1;
  const float my_w = lane < k ? w[(size_t)t * k + lane] : 0.0f;
  u32x4 g = u32x4{0u, 0u, 0u, 0u};
  if (c < nch) g = stream_load(dout + (size_t)t * nch + c);
  for (int j = 0; j < k; ++j) {
    const int d = read_lane(my_dst, j);
    if (d < 0 || d >= num_rows) continue;
    const float wj = read_lane(my_w, j);
    if (c < nch) stream_store(scale_row(g, wj), dy + (size_t)d * nch + c);
  }
}

template <int K, int U>
void launch_fixed(dim3 grid, hipStream_t stream, int T, int nch, int parts, int cpp,
                  int num_rows, const void* y, const int32_t* dst_row, const float* w,
                  void* out) {
  // The cap limits the requests in flight of a grid that runs in rounds; a
  // grid that fits the device at the cap runs without the LDS reservation
  // (decode steps of 128 tokens: 10.6 against 11.2 us per pipelined step).
  const long long at_cap = (long long)device_cus() * kCombineBlocksPerCu;
  const size_t lds = (long long)grid.x <= at_cap ? 0 : lds_cap_bytes(kCombineBlocksPerCu);
  hipLaunchKernelGGL((combine_kernel<K, U>), grid, dim3(256), lds, stream, T, nch, parts, cpp,
                     num_rows, static_cast<const u32x4*>(y), dst_row, w,
                     static_cast<u32x4*>(out));
}

template <int IPW>
void launch_held(int waves, hipStream_t stream, int T, int nch, int parts, int num_rows,
                 const void* y, const int32_t* dst_row, const float* w, void* out) {
  hipLaunchKernelGGL((combine_held_kernel<8, IPW>),
                     dim3((waves + kWavesPerBlock - 1) / kWavesPerBlock), dim3(256),
                     lds_cap_bytes(kHeldBlocksPerCu), stream, T, nch, parts, num_rows,
                     static_cast<const u32x4*>(y), dst_row, w, static_cast<u32x4*>(out));
}

// k = 8, rows of at least kHeldMinParts parts, 8..16 items per wave over
// held_waves() waves: the held-output kernel (returns false otherwise).
bool try_launch_held(int T, int nch, int k, int num_rows, const void* y,
                     const int32_t* dst_row, const float* w, void* out, hipStream_t stream) {
  if (k != 8) return false;
  const int parts = (nch + kHeldPart - 1) / kHeldPart;
  if (parts < kHeldMinParts) return false;
  const long long max_waves = held_waves();
  if (max_waves <= 0) return false;
  const long long items = (long long)T * parts;
  const long long ipw = (items + max_waves - 1) / max_waves;
  if (ipw < kHeldMinItems || ipw > kHeldMaxItems) return false;
  const int waves = (int)((items + ipw - 1) / ipw);
#define MOE_HELD(n) \
  case n: launch_held<n>(waves, stream, T, nch, parts, num_rows, y, dst_row, w, out); break;
  switch ((int)ipw) {
    MOE_HELD(8) MOE_HELD(9) MOE_HELD(10) MOE_HELD(11) MOE_HELD(12) MOE_HELD(13) MOE_HELD(14)
    MOE_HELD(15) MOE_HELD(16)
    default: return false;
  }
#undef MOE_HELD
  return true;
}

}  // namespace

hipError_t launch_combine_backward(int T, int H, int k, int num_rows, const void* dout,
                                   const void* y, const int32_t* dst_row, const float* w,
                                   void* dy, float* dw, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int nch = H / 8;
  const auto* g = static_cast<const u32x4*>(dout);
  hipLaunchKernelGGL(combine_backward_dw_kernel, dim3(T), dim3(256), 0, stream, T, k, nch,
                     num_rows, g, static_cast<const u32x4*>(y), dst_row, dw);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int parts = (nch + MOE_WAVE - 1) / MOE_WAVE;
  const long long waves = (long long)T * parts;
  hipLaunchKernelGGL(combine_backward_dy_kernel,
                     dim3((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock)), dim3(256),
                     lds_cap_bytes(kBwdDyBlocksPerCu), stream, T, k, nch, parts, num_rows, g,
                     dst_row, w, static_cast<u32x4*>(dy));
  return hipGetLastError();
}

hipError_t launch_combine(int T, int H, int k, int num_rows, const void* y,
                          const int32_t* dst_row, const float* w, void* out,
                          hipStream_t stream, bool allow_held, bool fine_items) {
  if (T == 0) return hipSuccess;
  const int nch = H / 8;
  if (allow_held && try_launch_held(T, nch, k, num_rows, y, dst_row, w, out, stream))
    return hipGetLastError();
  const bool fine = fine_items && k == 8;
  int parts = fine ? nch / MOE_WAVE : (kTargetWaves + T - 1) / T;
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
    case 8:
      // one chunk per lane when a part is one wave-wide step: no masked loads
      // (decode steps: 11.0 against 11.2 us per pipelined step, 10.35 with
      // the uncapped small grid above)
      if (fine || cpp <= MOE_WAVE)
        launch_fixed<8, 1>(grid, stream, T, nch, parts, cpp, num_rows, y, dst_row, w, out);
      else
        launch_fixed<8, MOE_COMBINE_U8>(grid, stream, T, nch, parts, cpp, num_rows, y, dst_row, w, out);
      break;
    default:
      hipLaunchKernelGGL(combine_kernel_any_k, grid, dim3(256), 0, stream, T, k, nch, parts,
                         cpp, num_rows, static_cast<const u32x4*>(y), dst_row, w,
                         static_cast<u32x4*>(out));
  }
  return hipGetLastError();
}

}  // namespace moe
