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
// dsv3, mixtral and qwen3_skew shapes: FP8 runs 4-6% faster at 3 than at the
// 8 its registers allow; bf16 with k <= 2 about 3% faster at 4, while bf16
// with k = 8 and MXFP8 run best uncapped.
constexpr int kFp8BlocksPerCu = 3;
constexpr int kBf16FewBlocksPerCu = 4;

__global__ __launch_bounds__(256) void dispatch_bf16_kernel(
    int T, int k, int nch, int parts, int cpp, int num_rows,
    const u32x4* __restrict__ x, const int32_t* __restrict__ dst_row,
    u32x4* __restrict__ out) {
  dispatch_bf16_body(blockIdx.x, T, k, nch, parts, cpp, num_rows, x, DstRows{dst_row}, out);
}

__global__ __launch_bounds__(256) void dispatch_fp8_kernel(
    int T, int k, int H, int parts, int bpp, int num_rows,
    const u32x4* __restrict__ x, const int32_t* __restrict__ dst_row,
    uint8_t* __restrict__ out, float* __restrict__ out_scales) {
  dispatch_fp8_body(blockIdx.x, T, k, H, parts, bpp, num_rows, x, DstRows{dst_row}, out,
                    out_scales);
}

__global__ __launch_bounds__(256) void dispatch_mxfp8_kernel(
    int T, int k, int H, int parts, int bpp, int num_rows,
    const u32x4* __restrict__ x, const int32_t* __restrict__ dst_row,
    uint8_t* __restrict__ out, uint8_t* __restrict__ out_scales) {
  dispatch_mxfp8_body(blockIdx.x, T, k, H, parts, bpp, num_rows, x, DstRows{dst_row}, out,
                      out_scales);
}

}  // namespace

hipError_t launch_dispatch_mxfp8(int T, int H, int k, int num_rows, const void* x,
                                 const int32_t* dst_row, void* out, uint8_t* out_scales,
                                 hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int nb = H / MOE_MX_BLOCK;
  int parts, bpp;
  split_row(T, nb, kMxStepBlocks, 64 * kScaleSlots, &parts, &bpp);
  const int waves = T * parts;
  hipLaunchKernelGGL(dispatch_mxfp8_kernel, dim3((waves + kWavesPerBlock - 1) / kWavesPerBlock),
                     dim3(256), 0, stream, T, k, H, parts, bpp, num_rows,
                     static_cast<const u32x4*>(x), dst_row, static_cast<uint8_t*>(out),
                     out_scales);
  return hipGetLastError();
}

hipError_t launch_dispatch_bf16(int T, int H, int k, int num_rows, const void* x,
                                const int32_t* dst_row, void* out, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int nch = H / 8;
  int parts, cpp;
  split_row(T, nch, MOE_WAVE, 1 << 30, &parts, &cpp);
  const int waves = T * parts;
  hipLaunchKernelGGL(dispatch_bf16_kernel, dim3((waves + kWavesPerBlock - 1) / kWavesPerBlock),
                     dim3(256), lds_cap_bytes(k <= 2 ? kBf16FewBlocksPerCu : 0), stream, T, k, nch, parts, cpp, num_rows,
                     static_cast<const u32x4*>(x), dst_row, static_cast<u32x4*>(out));
  return hipGetLastError();
}

hipError_t launch_dispatch_fp8(int T, int H, int k, int num_rows, const void* x,
                               const int32_t* dst_row, void* out, float* out_scales,
                               hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int nb = H / MOE_FP8_BLOCK;
  int parts, bpp;
  split_row(T, nb, kFp8StepBlocks, 64 * kScaleSlots, &parts, &bpp);
  const int waves = T * parts;
  hipLaunchKernelGGL(dispatch_fp8_kernel, dim3((waves + kWavesPerBlock - 1) / kWavesPerBlock),
                     dim3(256), lds_cap_bytes(kFp8BlocksPerCu), stream, T, k, H, parts, bpp, num_rows,
                     static_cast<const u32x4*>(x), dst_row, static_cast<uint8_t*>(out),
                     out_scales);
  return hipGetLastError();
}

}  // namespace moe
