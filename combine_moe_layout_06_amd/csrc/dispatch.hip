// Dispatch kernels on gfx950: one 64-lane wave per (token, column part),
// the destination rows from moe_layout (the device code is in
// dispatch_body.h).
//
// Sources: glossary "Expert Parallelism" (polydesk.ai), "Le pattern de
// communication all-to-all", Phase 1; DeepEP article (ai-master.dev),
// "Kernels low-latency dispatch et combine", "Support FP8 et MXFP8" and
// "Configuration type"; hyper.ai story on Hybrid-EP (native FP8/BF16).

#include "dispatch_body.h"

namespace moe {
namespace {

// Workgroups per CU (occupancy caps, see lds_cap_bytes), measured on the
// dsv3, mixtral and qwen3_skew shapes: MXFP8 runs best uncapped; the row-held
// FP8 kernel at 4 or 5 (53.4, 53.2 us on dsv3), 3: 57.0, 2: 61.0, uncapped:
// 53.7. The bf16 dispatch takes 1 KiB pieces (below); with few rows per
// token each wave writes less, so it needs more waves: on qwen3_skew (k = 8,
// 8 KiB rows) 111.2-111.9 us at 5 against 120.6-121.5 with 2 KiB pieces
// uncapped (caps 4 and 6: 113-114, 2 and 3: 131-134, 8: 120-121); on
// mixtral (k = 2) 67.0-68.2 us at 8 against 68.5-69.0 with 4 KiB pieces at 4
// (1 KiB pieces at 6: 70.2-71.7, at 4: 88.0-88.7).
constexpr int kFp8RowsBlocksPerCu = 4;
constexpr int kBf16FewBlocksPerCu = 8;    // k <= 2
constexpr int kBf16ManyBlocksPerCu = 5;   // k > 2
// Steps (8 blocks of 128 columns) per row-held FP8 wave at most.
constexpr int kFp8RowMaxSteps = 8;
// Row-held kernels split a row into more parts while T * parts stays below
// this many waves (one resident round at 4 workgroups per CU on 256 CUs):
// one part per row at T = 4096, one step per part for decode-sized T.
constexpr int kRowsMinWaves = 4096;

// Parts of a row of `steps` steps: at least enough for `max_steps` steps per
// part, more for small T (up to one step per part), as even as whole steps
// allow; returns the steps per part.
inline int row_parts(int T, int steps, int max_steps, int* parts) {
  int p = (steps + max_steps - 1) / max_steps;
  const int want = T > 0 ? (kRowsMinWaves + T - 1) / T : 1;
  p = max(p, min(steps, want));
  const int per = (steps + p - 1) / p;
  *parts = (steps + per - 1) / per;
  return per;
}

// Row-held MXFP8: steps of 512 columns per wave at most, and its cap.
constexpr int kMxRowMaxSteps = 16;
#ifndef MOE_MX_CAP
#define MOE_MX_CAP 4
#endif
constexpr int kMxRowsBlocksPerCu = MOE_MX_CAP;

__global__ __launch_bounds__(256) void dispatch_bf16_kernel(
    int T, int k, int nch, int parts, int cpp, int num_rows,
    const u32x4* __restrict__ x, const int32_t* __restrict__ dst_row,
    u32x4* __restrict__ out) {
  dispatch_bf16_body(blockIdx.x, T, k, nch, parts, cpp, num_rows, x, DstRows{dst_row}, out);
}

template <int MAXST>
__global__ __launch_bounds__(256) void dispatch_fp8_rows_kernel(
    int T, int k, int H, int parts, int bpp, int num_rows,
    const u32x4* __restrict__ x, const int32_t* __restrict__ dst_row,
    uint8_t* __restrict__ out, float* __restrict__ out_scales) {
  dispatch_fp8_rows_body<MAXST>(blockIdx.x, T, k, H, parts, bpp, num_rows, x, dst_row, out,
                                out_scales);
}

template <int MAXST>
void launch_fp8_rows(int T, int H, int k, int parts, int bpp, int num_rows, const void* x,
                     const int32_t* dst_row, void* out, float* out_scales, hipStream_t stream) {
  const int waves = T * parts;
  hipLaunchKernelGGL((dispatch_fp8_rows_kernel<MAXST>),
                     dim3((waves + kWavesPerBlock - 1) / kWavesPerBlock), dim3(256),
                     lds_cap_bytes(kFp8RowsBlocksPerCu), stream, T, k, H, parts, bpp, num_rows,
                     static_cast<const u32x4*>(x), dst_row, static_cast<uint8_t*>(out),
                     out_scales);
}

template <int MAXST>
__global__ __launch_bounds__(256) void dispatch_mxfp8_rows_kernel(
    int T, int k, int H, int parts, int bpp, int num_rows,
    const u32x4* __restrict__ x, const int32_t* __restrict__ dst_row,
    uint8_t* __restrict__ out, uint8_t* __restrict__ out_scales) {
  dispatch_mxfp8_rows_body<MAXST>(blockIdx.x, T, k, H, parts, bpp, num_rows, x, dst_row, out,
                                  out_scales);
}

template <int MAXST>
void launch_mxfp8_rows(int T, int H, int k, int parts, int bpp, int num_rows, const void* x,
                       const int32_t* dst_row, void* out, uint8_t* out_scales,
                       hipStream_t stream) {
  const int waves = T * parts;
  hipLaunchKernelGGL((dispatch_mxfp8_rows_kernel<MAXST>),
                     dim3((waves + kWavesPerBlock - 1) / kWavesPerBlock), dim3(256),
                     lds_cap_bytes(kMxRowsBlocksPerCu), stream, T, k, H, parts, bpp, num_rows,
                     static_cast<const u32x4*>(x), dst_row, static_cast<uint8_t*>(out),
                     out_scales);
}

}  // namespace

hipError_t launch_dispatch_mxfp8(int T, int H, int k, int num_rows, const void* x,
                                 const int32_t* dst_row, void* out, uint8_t* out_scales,
                                 hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int nb = H / MOE_MX_BLOCK;
  const int steps = (nb + kMxStepBlocks - 1) / kMxStepBlocks;
  int parts;
  const int per = row_parts(T, steps, kMxRowMaxSteps, &parts);    // steps per part, <= 16
  const int bpp = per * kMxStepBlocks;
  // instantiated for 1, 2, 4, 7, 8, 14 and 16 steps; a part of fewer steps
  // runs in the next larger instance, its extra steps masked off
#define MOE_MX_ROWS(n) \
  launch_mxfp8_rows<n>(T, H, k, parts, bpp, num_rows, x, dst_row, out, out_scales, stream)
  if (per <= 1) MOE_MX_ROWS(1);
  else if (per <= 2) MOE_MX_ROWS(2);
  else if (per <= 4) MOE_MX_ROWS(4);
  else if (per <= 7) MOE_MX_ROWS(7);
  else if (per <= 8) MOE_MX_ROWS(8);
  else if (per <= 14) MOE_MX_ROWS(14);
  else MOE_MX_ROWS(16);
#undef MOE_MX_ROWS
  return hipGetLastError();
}

hipError_t launch_dispatch_bf16(int T, int H, int k, int num_rows, const void* x,
                                const int32_t* dst_row, void* out, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int nch = H / 8;
  int parts, cpp;
  // pieces of one 16-byte chunk per lane (1 KiB), as many parts as a row
  // has; each wave writes k short pieces
  split_row(T, nch, MOE_WAVE, MOE_WAVE, &parts, &cpp);
  const int waves = T * parts;
  hipLaunchKernelGGL(dispatch_bf16_kernel, dim3((waves + kWavesPerBlock - 1) / kWavesPerBlock),
                     dim3(256), lds_cap_bytes(k <= 2 ? kBf16FewBlocksPerCu : kBf16ManyBlocksPerCu),
                     stream, T, k, nch, parts, cpp, num_rows, static_cast<const u32x4*>(x),
                     dst_row, static_cast<u32x4*>(out));
  return hipGetLastError();
}

hipError_t launch_dispatch_fp8(int T, int H, int k, int num_rows, const void* x,
                               const int32_t* dst_row, void* out, float* out_scales,
                               hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int nb = H / MOE_FP8_BLOCK;
  const int steps = (nb + kFp8StepBlocks - 1) / kFp8StepBlocks;
  int parts;
  const int per = row_parts(T, steps, kFp8RowMaxSteps, &parts);   // steps per part, <= 8
  const int bpp = per * kFp8StepBlocks;
#define MOE_FP8_ROWS(n) \
  case n: launch_fp8_rows<n>(T, H, k, parts, bpp, num_rows, x, dst_row, out, out_scales, stream); break;
  switch (per) {
    MOE_FP8_ROWS(1) MOE_FP8_ROWS(2) MOE_FP8_ROWS(3) MOE_FP8_ROWS(4) MOE_FP8_ROWS(5)
    MOE_FP8_ROWS(6) MOE_FP8_ROWS(7) MOE_FP8_ROWS(8)
    default: return hipErrorInvalidValue;
  }
#undef MOE_FP8_ROWS
  return hipGetLastError();
}

}  // namespace moe
