// Exhaustive device check of the two hardware converts the HIP path relies on
// (test code; not part of the library).
//
//   pack_bf16x2   (wave.h, the combines' output rounding): fp32 -> bf16 with
//                 v_cvt_pk_bf16_f32, against round-to-nearest-even written
//                 here on the integer bits, for all 2^32 fp32 patterns, each
//                 one in the low and in the high half of a pair. A NaN must
//                 give a NaN.
//   e4m3_pair_hw  (dispatch_body.h, the FP8 and MXFP8 dispatch codes): clamp
//                 to +-448 and v_cvt_pk_fp8_f32, against the e4m3fn rounding
//                 written here, for every non-NaN fp32 pattern.
//   e4m3_from_f32 (dispatch_body.h, the software path taken when 448 / amax
//                 overflows fp32), the same reference and domain.
//
// The e4m3fn format (OCP 8-bit floating point, the format the DeepEP article
// names in "Support FP8 et MXFP8"): 1 sign bit, 4 exponent bits with bias 7,
// 3 mantissa bits, subnormals m * 2^-9, largest finite 448; here values round
// to nearest with ties to even and larger magnitudes saturate to 448.
//
// The references are also exported for the host (convert_ref_bf16,
// convert_ref_e4m3) and checked there against the oracle's codecs.
//
// Each thread walks a strided share of the 2^32 patterns, counts mismatches
// and keeps the smallest mismatching pattern; the counts go to a caller's
// buffer of 8 uint64 with one atomic add per thread and check. Every thread
// runs a fixed number of iterations and exits.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dispatch_body.h"
#include "wave.h"

namespace {

// Nearest bf16 of an fp32 pattern, ties to even, from the dropped bits.
__host__ __device__ uint32_t ref_bf16(uint32_t u) {
  uint32_t kept = u >> 16;
  const uint32_t rem = u & 0xFFFFu;
  if (rem > 0x8000u || (rem == 0x8000u && (kept & 1u))) kept += 1u;   // may carry into the exponent
  return kept & 0xFFFFu;
}

// e4m3fn code of a non-NaN fp32 pattern (sign kept, zero included).
__host__ __device__ uint32_t ref_e4m3(uint32_t u) {
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  const int E = (int)(a >> 23);
  if (E == 255) return sign | 0x7Eu;                  // infinity saturates
  if (E == 0) return sign;                            // fp32 subnormals are below 2^-10
  const uint32_t sig = (a & 0x7FFFFFu) | 0x800000u;   // value = sig * 2^(E - 150)
  const int e = E - 127;
  uint32_t code;
  if (e >= -6) {
    // normal e4m3: keep 4 significant bits (3 stored), quantum 2^(e-3)
    uint32_t kept = sig >> 20;
    const uint32_t rem = sig & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (kept & 1u))) kept += 1u;
    int ef = e + 7;
    if (kept == 16u) { kept = 8u; ef += 1; }
    if (ef > 15 || (ef == 15 && kept - 8u > 6u)) return sign | 0x7Eu;   // above 448
    code = ((uint32_t)ef << 3) | (kept - 8u);
  } else {
    // below 2^-6: multiples of 2^-9, n = sig * 2^(E - 141)
    const int s = 141 - E;                            // >= 21
    if (s >= 26) return sign;                         // below a quarter quantum
    uint32_t kept = sig >> s;
    const uint32_t rem = sig & ((1u << s) - 1u);
    const uint32_t half = 1u << (s - 1);
    if (rem > half || (rem == half && (kept & 1u))) kept += 1u;
    code = kept;                                      // 8 is 2^-6, the smallest normal
  }
  return sign | code;
}

__device__ bool is_nan(uint32_t u) { return (u & 0x7FFFFFFFu) > 0x7F800000u; }

__global__ __launch_bounds__(256) void sweep_kernel(unsigned long long* res) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  const uint64_t first = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  unsigned long long bad_bf = 0, bad_hw = 0, bad_sw = 0, checked = 0;
  unsigned long long min_bf = ~0ull, min_hw = ~0ull, min_sw = ~0ull;
  for (uint64_t i = first; i < (1ull << 32); i += stride) {
    const uint32_t u = (uint32_t)i;
    const uint32_t v = u ^ 0x80000000u;               // pairs every pattern with its negation
    // bf16: u in the low half, v in the high half
    const uint32_t p = pack_bf16x2(__uint_as_float(u), __uint_as_float(v));
    const uint32_t lo = p & 0xFFFFu, hi = p >> 16;
    const bool ok_lo = is_nan(u) ? is_nan(lo << 16) : lo == ref_bf16(u);
    const bool ok_hi = is_nan(v) ? is_nan(hi << 16) : hi == ref_bf16(v);
    if (!ok_lo || !ok_hi) {
      ++bad_bf;
      min_bf = min(min_bf, (unsigned long long)(ok_lo ? v : u));
    }
    if (is_nan(u)) continue;
    ++checked;
    const uint32_t want = ref_e4m3(u);
    const uint32_t hw = moe::e4m3_pair_hw(__uint_as_float(u), __uint_as_float(v));
    if ((hw & 0xFFu) != want || (hw >> 8) != (want ^ 0x80u)) {
      ++bad_hw;
      min_hw = min(min_hw, (unsigned long long)u);
    }
    if (moe::e4m3_from_f32(__uint_as_float(u)) != want) {
      ++bad_sw;
      min_sw = min(min_sw, (unsigned long long)u);
    }
  }
  if (bad_bf) { atomicAdd(&res[0], bad_bf); atomicMin(&res[1], min_bf); }
  if (bad_hw) { atomicAdd(&res[2], bad_hw); atomicMin(&res[3], min_hw); }
  if (bad_sw) { atomicAdd(&res[4], bad_sw); atomicMin(&res[5], min_sw); }
  atomicAdd(&res[6], checked);
}

}  // namespace

// res: device buffer of 8 uint64, set by the caller to
// {0, ~0, 0, ~0, 0, ~0, 0, 0}. On return (after the stream synchronises):
// res[0], res[1]: bf16 mismatches and the smallest mismatching pattern;
// res[2], res[3]: the same for the clamped FP8 pack-convert;
// res[4], res[5]: the same for the software e4m3 rounding;
// res[6]: non-NaN patterns checked (2^32 - 2 * (2^23 - 1) when complete).
// Returns the launch's hipError_t.
extern "C" int convert_sweep(void* res, void* stream) {
  hipLaunchKernelGGL(sweep_kernel, dim3(4096), dim3(256), 0, (hipStream_t)stream,
                     (unsigned long long*)res);
  return (int)hipGetLastError();
}

// The two references on the host, so that CPU tests can check them against
// the oracle's codecs before they check the device.
extern "C" uint32_t convert_ref_bf16(uint32_t u) { return ref_bf16(u); }
extern "C" uint32_t convert_ref_e4m3(uint32_t u) { return ref_e4m3(u); }
