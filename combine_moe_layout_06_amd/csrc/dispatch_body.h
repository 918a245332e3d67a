// Dispatch on gfx950 (device code, shared by the dispatch kernels and the
// fused layout + dispatch launch): copy each token's hidden state to the
// rows of its k experts, as bf16, as FP8 e4m3 with one fp32 scale per 128
// columns, or as MXFP8 with one E8M0 byte per 32 columns.
//
// Sources: glossary "Expert Parallelism" (polydesk.ai), "Le pattern de
// communication all-to-all", Phase 1 (each token goes to the GPUs of its
// experts); DeepEP article (ai-master.dev), "Kernels low-latency dispatch et
// combine" (dispatch kernels that understand the MoE data and fuse steps),
// "Support FP8 et MXFP8" (FP8 halves the BF16 volume) and "Configuration
// type" (FP8 quantisation happens inside the dispatch call); hyper.ai story
// on Hybrid-EP (native FP8/BF16 dispatch).
//
// One 64-lane wave per (token, column part). The token row is read once,
// held in registers, and written to each destination row with 16-byte
// (bf16) or 8-byte (FP8) nontemporal stores: every store instruction of a
// wave covers whole 128-byte lines. FP8 quantises once per token; the
// block amax is a 16-lane DPP max inside each 64-lane wave.

#pragma once

#include "kernels.h"
#include "wave.h"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kUnroll = 4;        // 16-byte chunks per lane held at once (bf16)
constexpr int kScaleSlots = 4;    // FP8: scales of up to 256 blocks per part
constexpr int kIdxChunks = 16;    // capacity positions: up to 1024 pairs

// Where a wave finds the destination rows of its token (lane j < k: the row
// of slot j, -1 for none).
//
// DstRows: the rows moe_layout computed.
struct DstRows {
  static constexpr bool kEarly = true;    // one load: issue it first
  const int32_t* dst_row;
  __device__ __forceinline__ int operator()(int t, int k, int lane) const {
    return lane < k ? dst_row[(size_t)t * k + lane] : -1;
  }
};

// DstCapacity: the same rows computed from the routing, in capacity mode
// with at most 1024 pairs. Slot j of token t goes to row e*cap + pos, pos =
// the number of pairs of expert e before (t, j) in row-major order, or is
// dropped when pos >= cap (the layout's definition). One ballot per earlier
// 64-pair chunk and slot counts them; all loads are issued first.
struct DstCapacity {
  static constexpr bool kEarly = false;   // after the row loads are issued
  const int32_t* idx;
  int E, cap;
  __device__ __forceinline__ int operator()(int t, int k, int lane) const {
    // the token is the same in every lane: keep the counting scalar
    const int self = __builtin_amdgcn_readfirstlane(t * k);
    int my_e = lane < k ? idx[self + lane] : -1;
    my_e = (my_e >= 0 && my_e < E) ? my_e : -1;
    const int end = self + k;             // pairs up to the token's last slot
    int v[kIdxChunks];
#pragma unroll
    for (int c = 0; c < kIdxChunks; ++c) {
      const int p = c * MOE_WAVE + lane;
      v[c] = p < end ? idx[p] : -1;
    }
    int pos = 0;
    for (int j = 0; j < k; ++j) {
      const int ej = read_lane(my_e, j);
      if (ej < 0) continue;
      const int lim = self + j;           // pairs strictly before (t, j)
      int cnt = 0;
#pragma unroll
      for (int c = 0; c < kIdxChunks; ++c) {
        const int n = lim - c * MOE_WAVE;   // wave-uniform
        if (n > 0) {
          uint64_t m = wave_ballot(v[c] == ej);
          if (n < MOE_WAVE) m &= (1ull << n) - 1ull;
          cnt += __popcll(m);
        }
      }
      if (lane == j) pos = cnt;
    }
    return (my_e >= 0 && pos < cap) ? my_e * cap + pos : -1;
  }
};

template <class Dst>
__device__ __forceinline__ void dispatch_bf16_body(
    int block, int T, int k, int nch, int parts, int cpp, int num_rows,
    const u32x4* __restrict__ x, Dst dst_of, u32x4* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int gw = block * kWavesPerBlock + (threadIdx.x >> 6);
  if (gw >= T * parts) return;
  const int t = gw / parts;
  const int c0 = (gw - t * parts) * cpp;
  const int cnt = min(cpp, nch - c0);
  int my_dst = Dst::kEarly ? dst_of(t, k, lane) : -1;
  const u32x4* src = x + (size_t)t * nch + c0;

  for (int base = 0; base < cnt; base += MOE_WAVE * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = base + u * MOE_WAVE + lane;
      v[u] = u32x4{0u, 0u, 0u, 0u};
      if (c < cnt) v[u] = stream_load(src + c);
    }
    if (!Dst::kEarly && base == 0) my_dst = dst_of(t, k, lane);
    for (int j = 0; j < k; ++j) {
      const int d = read_lane(my_dst, j);
      if (d < 0 || d >= num_rows) continue;
      u32x4* dst = out + (size_t)d * nch + c0;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = base + u * MOE_WAVE + lane;
        if (c < cnt) stream_store(v[u], dst + c);
      }
    }
  }
}

// Max over the 16 lanes of each DPP row (lanes 16r .. 16r+15).
__device__ __forceinline__ uint32_t row16_max(uint32_t m) {
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x141, 0xF, 0xF, false));  // row_half_mirror
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x140, 0xF, 0xF, false));  // row_mirror
  return m;
}

// fp32 -> OCP e4m3fn code, round to nearest even, saturating at +-448.
// The sign of zero is kept. `p` is finite or +-inf here.
__device__ __forceinline__ uint32_t e4m3_from_f32(float p) {
  const uint32_t b = __float_as_uint(p);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7FFFFFFFu;
  uint32_t mag;
  if (a > 0x43E00000u) {                 // above 448: saturate
    mag = 0x7Eu;
  } else if (a >= 0x3C800000u) {         // normal e4m3 range, >= 2^-6
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);   // RNE to 3 mantissa bits
    mag = (r >> 20) - (120u << 3);                        // rebias exponent 127 -> 7
  } else {                               // subnormal range: multiples of 2^-9
    mag = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  }
  return sign | mag;
}

// Quantise one bf16 element (held in the low 16 bits of `h`) in software.
__device__ __forceinline__ uint32_t quant_one(uint32_t h, float inv) {
  const float xv = __uint_as_float(h << 16);
  if ((h & 0x7FFFu) == 0u) return (h >> 8) & 0x80u;       // +-0 keeps its sign
  return e4m3_from_f32(xv * inv);
}

__device__ __forceinline__ uint32_t quant_pair_sw(uint32_t w, float inv) {
  return quant_one(w & 0xFFFFu, inv) | (quant_one(w >> 16, inv) << 8);
}

// Two fp32 values -> two e4m3 codes (low 16 bits, `a` in the low byte) with
// the hardware pack-convert, which rounds to nearest even; the values are
// clamped to +-448 first, so larger magnitudes and infinities saturate. For
// every non-NaN fp32 value this equals e4m3_from_f32 (tests/hip/
// convert_sweep.hip compares all 2^32 patterns on the device).
__device__ __forceinline__ uint32_t e4m3_pair_hw(float a, float b) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Two bf16 -> two e4m3 codes of x * inv. Needs a finite multiplier: then
// +-0 stays +-0.
__device__ __forceinline__ uint32_t quant_pair_hw(uint32_t w, float inv) {
  return e4m3_pair_hw(__uint_as_float(w << 16) * inv, __uint_as_float(w & 0xFFFF0000u) * inv);
}

// 8 bf16 (16 bytes) -> 8 codes (8 bytes)
__device__ __forceinline__ u32x2 quant8(const u32x4& v, float inv) {
  u32x2 q;
  if (__builtin_isfinite(inv)) {
    q[0] = quant_pair_hw(v[0], inv) | (quant_pair_hw(v[1], inv) << 16);
    q[1] = quant_pair_hw(v[2], inv) | (quant_pair_hw(v[3], inv) << 16);
  } else {   // the block's amax is so small that 448/amax overflows
    q[0] = quant_pair_sw(v[0], inv) | (quant_pair_sw(v[1], inv) << 16);
    q[1] = quant_pair_sw(v[2], inv) | (quant_pair_sw(v[3], inv) << 16);
  }
  return q;
}

// Block amax of the 16 lanes of a DPP row, from the bf16 magnitudes (their
// bit patterns order like the values).
__device__ __forceinline__ float block_amax(const u32x4& v) {
  uint32_t m = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t w = v[q] & 0x7FFF7FFFu;
    m = max(m, max(w & 0xFFFFu, w >> 16));
  }
  return __uint_as_float(row16_max(m) << 16);
}

// One wave per (token, part of kFp8StepBlocks-block steps). A step covers
// 1024 columns: lane L holds chunk A = columns [8L, 8L+8) and chunk B =
// columns [512 + 8L, 512 + 8L + 8); the 16 lanes of a DPP row form one
// 128-column block of A and one of B. After quantisation the lanes of a pair
// (2i, 2i+1) swap halves, so lane 2i writes codes of A-columns [16i, 16i+16)
// and lane 2i+1 those of B-columns [16i, 16i+16): one 16-byte store per lane
// and copy.
constexpr int kFp8StepBlocks = 8;

template <class Dst>
__device__ __forceinline__ void dispatch_fp8_body(
    int block, int T, int k, int H, int parts, int bpp, int num_rows,
    const u32x4* __restrict__ x, Dst dst_of,
    uint8_t* __restrict__ out, float* __restrict__ out_scales) {
  const int lane = threadIdx.x & 63;
  const int gw = block * kWavesPerBlock + (threadIdx.x >> 6);
  if (gw >= T * parts) return;
  const int t = gw / parts;
  const int nb = H / MOE_FP8_BLOCK;
  const int nch = H / 8;
  const int b0 = (gw - t * parts) * bpp;
  const int nbp = min(bpp, nb - b0);
  int my_dst = Dst::kEarly ? dst_of(t, k, lane) : -1;
  const int group = lane >> 4;       // block of A (and of B) inside the step
  const int sub = lane & 15;         // 16-byte chunk inside the block
  const bool odd = lane & 1;
  const u32x4* src = x + (size_t)t * nch;

  float sreg[kScaleSlots];
#pragma unroll
  for (int s = 0; s < kScaleSlots; ++s) sreg[s] = 0.0f;

  for (int st = 0; st * kFp8StepBlocks < nbp; ++st) {
    const int ba = st * kFp8StepBlocks + group;          // part-local blocks
    const int bb = ba + kFp8StepBlocks / 2;
    const bool act_a = ba < nbp, act_b = bb < nbp;
    u32x4 va = {0u, 0u, 0u, 0u}, vb = {0u, 0u, 0u, 0u};
    if (act_a) va = stream_load(src + (b0 + ba) * 16 + sub);
    if (act_b) vb = stream_load(src + (b0 + bb) * 16 + sub);
    if (!Dst::kEarly && st == 0) my_dst = dst_of(t, k, lane);

    const float amax_a = block_amax(va), amax_b = block_amax(vb);
    const float scale_a = amax_a / 448.0f, scale_b = amax_b / 448.0f;
    // lanes of a block past the part's end quantise with multiplier 1 (their
    // codes are never stored), which keeps the whole wave on the fast path
    const u32x2 qa = quant8(va, act_a ? 448.0f / amax_a : 1.0f);
    const u32x2 qb = quant8(vb, act_b ? 448.0f / amax_b : 1.0f);

    // swap halves inside lane pairs: even lanes keep A, odd lanes keep B
    const u32x2 send = odd ? qa : qb;
    u32x2 recv;
    recv[0] = dpp_u32<0xB1>(send[0]);
    recv[1] = dpp_u32<0xB1>(send[1]);
    const u32x4 q = odd ? u32x4{recv[0], recv[1], qb[0], qb[1]}
                        : u32x4{qa[0], qa[1], recv[0], recv[1]};
    const int bq = odd ? bb : ba;                        // block this lane writes
    const bool act_q = odd ? act_b : act_a;
    const int col = (b0 + bq) * MOE_FP8_BLOCK + (sub & ~1) * 8;   // 16-byte aligned

    // lane (b & 63), slot (b >> 6) keeps the scale of part-local block b
#pragma unroll
    for (int g = 0; g < kFp8StepBlocks; ++g) {
      const int b = st * kFp8StepBlocks + g;
      const float sg = read_lane(g < 4 ? scale_a : scale_b, (g & 3) * 16);
      if (b < nbp && lane == (b & 63)) {
#pragma unroll
        for (int s = 0; s < kScaleSlots; ++s)
          if ((b >> 6) == s) sreg[s] = sg;
      }
    }

    for (int j = 0; j < k; ++j) {
      const int d = read_lane(my_dst, j);
      if (d < 0 || d >= num_rows) continue;
      if (act_q) stream_store(q, reinterpret_cast<u32x4*>(out + (size_t)d * H + col));
    }
  }

  for (int j = 0; j < k; ++j) {
    const int d = read_lane(my_dst, j);
    if (d < 0 || d >= num_rows) continue;
    float* srow = out_scales + (size_t)d * nb + b0;
#pragma unroll
    for (int s = 0; s < kScaleSlots; ++s) {
      const int b = s * 64 + lane;
      if (b < nbp) srow[b] = sreg[s];
    }
  }
}


// FP8 with row-held waves: one wave per (token, part of at most MAXST steps),
// the same step layout and arithmetic as dispatch_fp8_body. The wave issues
// the loads of all its steps first, keeps the codes of the whole part in
// registers (4 per step and lane) and then writes each destination row as
// one contiguous run: MAXST pieces of 1 KiB back to back, then the row's
// scales. With a part covering the whole row (7 steps at hidden 7168) every
// destination row is one 7 KiB run from one wave, which the memory writes
// faster than the same bytes as pieces from seven waves at different times
// (dsv3: 53.4 against 58.1 us).
template <int MAXST>
__device__ __forceinline__ void dispatch_fp8_rows_body(
    int block, int T, int k, int H, int parts, int bpp, int num_rows,
    const u32x4* __restrict__ x, const int32_t* __restrict__ dst_row,
    uint8_t* __restrict__ out, float* __restrict__ out_scales) {
  const int lane = threadIdx.x & 63;
  const int gw = block * kWavesPerBlock + (threadIdx.x >> 6);
  if (gw >= T * parts) return;
  const int t = gw / parts;
  const int nb = H / MOE_FP8_BLOCK;
  const int nch = H / 8;
  const int b0 = (gw - t * parts) * bpp;
  const int nbp = min(bpp, nb - b0);
  const int my_dst = lane < k ? dst_row[(size_t)t * k + lane] : -1;
  const int group = lane >> 4;       // block of A (and of B) inside a step
  const int sub = lane & 15;         // 16-byte chunk inside the block
  const bool odd = lane & 1;
  const u32x4* src = x + (size_t)t * nch;

  u32x4 va[MAXST], vb[MAXST];
#pragma unroll
  for (int st = 0; st < MAXST; ++st) {
    const int ba = st * kFp8StepBlocks + group, bb = ba + kFp8StepBlocks / 2;
    va[st] = u32x4{0u, 0u, 0u, 0u};
    vb[st] = u32x4{0u, 0u, 0u, 0u};
    if (ba < nbp) va[st] = stream_load(src + (b0 + ba) * 16 + sub);
    if (bb < nbp) vb[st] = stream_load(src + (b0 + bb) * 16 + sub);
  }

  float sreg[kScaleSlots];
#pragma unroll
  for (int s = 0; s < kScaleSlots; ++s) sreg[s] = 0.0f;
  u32x4 q[MAXST];
#pragma unroll
  for (int st = 0; st < MAXST; ++st) {
    const int ba = st * kFp8StepBlocks + group, bb = ba + kFp8StepBlocks / 2;
    const bool act_a = ba < nbp, act_b = bb < nbp;
    const float amax_a = block_amax(va[st]), amax_b = block_amax(vb[st]);
    const float scale_a = amax_a / 448.0f, scale_b = amax_b / 448.0f;
    const u32x2 qa = quant8(va[st], act_a ? 448.0f / amax_a : 1.0f);
    const u32x2 qb = quant8(vb[st], act_b ? 448.0f / amax_b : 1.0f);
    // swap halves inside lane pairs: even lanes keep A, odd lanes keep B
    const u32x2 send = odd ? qa : qb;
    u32x2 recv;
    recv[0] = dpp_u32<0xB1>(send[0]);
    recv[1] = dpp_u32<0xB1>(send[1]);
    q[st] = odd ? u32x4{recv[0], recv[1], qb[0], qb[1]} : u32x4{qa[0], qa[1], recv[0], recv[1]};
    // lane (b & 63), slot (b >> 6) keeps the scale of part-local block b
#pragma unroll
    for (int g = 0; g < kFp8StepBlocks; ++g) {
      const int b = st * kFp8StepBlocks + g;
      const float sg = read_lane(g < 4 ? scale_a : scale_b, (g & 3) * 16);
      if (b < nbp && lane == (b & 63)) {
#pragma unroll
        for (int s = 0; s < kScaleSlots; ++s)
          if ((b >> 6) == s) sreg[s] = sg;
      }
    }
  }

  for (int j = 0; j < k; ++j) {
    const int d = read_lane(my_dst, j);
    if (d < 0 || d >= num_rows) continue;
#pragma unroll
    for (int st = 0; st < MAXST; ++st) {
      const int ba = st * kFp8StepBlocks + group;
      const int bq = odd ? ba + kFp8StepBlocks / 2 : ba;   // block this lane writes
      const int col = (b0 + bq) * MOE_FP8_BLOCK + (sub & ~1) * 8;
      if (bq < nbp) stream_store(q[st], reinterpret_cast<u32x4*>(out + (size_t)d * H + col));
    }
    float* srow = out_scales + (size_t)d * nb + b0;
#pragma unroll
    for (int s = 0; s < kScaleSlots; ++s) {
      const int b = s * 64 + lane;
      if (b < nbp) srow[b] = sreg[s];
    }
  }
}

// MXFP8: one wave per (token, part); a step covers 512 columns = 16 blocks
// of 32 columns, 4 lanes per block. The shared exponent comes from the
// block amax (two DPP steps inside each quad); codes use the hardware
// pack-convert of x * 2^-e clamped to +-448 (the multiplication by a power
// of two is exact).
constexpr int kMxStepBlocks = 16;

template <class Dst>
__device__ __forceinline__ void dispatch_mxfp8_body(
    int block, int T, int k, int H, int parts, int bpp, int num_rows,
    const u32x4* __restrict__ x, Dst dst_of,
    uint8_t* __restrict__ out, uint8_t* __restrict__ out_scales) {
  const int lane = threadIdx.x & 63;
  const int gw = block * kWavesPerBlock + (threadIdx.x >> 6);
  if (gw >= T * parts) return;
  const int t = gw / parts;
  const int nb = H / MOE_MX_BLOCK;
  const int nch = H / 8;
  const int b0 = (gw - t * parts) * bpp;
  const int nbp = min(bpp, nb - b0);
  int my_dst = Dst::kEarly ? dst_of(t, k, lane) : -1;
  const int blk = lane >> 2;         // block inside the step
  const int sub = lane & 3;          // 16-byte chunk inside the block
  const u32x4* src = x + (size_t)t * nch;

  uint32_t sreg[kScaleSlots];        // E8M0 byte of part-local block (s*64 + lane)
#pragma unroll
  for (int s = 0; s < kScaleSlots; ++s) sreg[s] = 0u;

  for (int st = 0; st * kMxStepBlocks < nbp; ++st) {
    const int bl = st * kMxStepBlocks + blk;
    const bool act = bl < nbp;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (act) v = stream_load(src + (b0 + bl) * 4 + sub);
    if (!Dst::kEarly && st == 0) my_dst = dst_of(t, k, lane);

    uint32_t m = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w = v[q] & 0x7FFF7FFFu;
      m = max(m, max(w & 0xFFFFu, w >> 16));
    }
    m = max(m, dpp_u32<0xB1>(m));
    m = max(m, dpp_u32<0x4E>(m));
    const float amax = __uint_as_float(m << 16);
    int e = amax == 0.0f ? -127 : __builtin_amdgcn_frexp_expf(amax) - 1 - 8;
    e = min(max(e, -127), 127);
    const float inv = __builtin_amdgcn_ldexpf(1.0f, -e);
    u32x2 q;
    q[0] = quant_pair_hw(v[0], inv) | (quant_pair_hw(v[1], inv) << 16);
    q[1] = quant_pair_hw(v[2], inv) | (quant_pair_hw(v[3], inv) << 16);

    // lane L keeps the byte of part-local block L + 64*slot: in step st the
    // lanes of row (st % 4) receive block (st*16 + L % 16) from its first lane
    const uint32_t sb = (uint32_t)(e + 127);
    const uint32_t got = (uint32_t)__shfl((int)sb, 4 * (lane & 15));
#pragma unroll
    for (int s = 0; s < kScaleSlots; ++s)
      if (st / 4 == s && (lane >> 4) == (st & 3)) sreg[s] = got;

    if (act) {
      for (int j = 0; j < k; ++j) {
        const int d = read_lane(my_dst, j);
        if (d < 0 || d >= num_rows) continue;
        u32x2* dst = reinterpret_cast<u32x2*>(out + (size_t)d * H + (size_t)(b0 + bl) * MOE_MX_BLOCK) + sub;
        stream_store(q, dst);
      }
    }
  }

  for (int j = 0; j < k; ++j) {
    const int d = read_lane(my_dst, j);
    if (d < 0 || d >= num_rows) continue;
    uint8_t* srow = out_scales + (size_t)d * nb + b0;
#pragma unroll
    for (int s = 0; s < kScaleSlots; ++s) {
      const int b = s * 64 + lane;
      if (b < nbp) srow[b] = (uint8_t)sreg[s];
    }
  }
}

// MXFP8 with row-held waves: one wave per (token, part of at most MAXST
// steps of 512 columns), the step layout and arithmetic of
// dispatch_mxfp8_body. All loads of the part are issued first, the codes
// (2 registers per step and lane) and scale bytes are kept, and each
// destination row is then written as one contiguous run of 512-byte pieces
// followed by its scale bytes.
template <int MAXST>
__device__ __forceinline__ void dispatch_mxfp8_rows_body(
    int block, int T, int k, int H, int parts, int bpp, int num_rows,
    const u32x4* __restrict__ x, const int32_t* __restrict__ dst_row,
    uint8_t* __restrict__ out, uint8_t* __restrict__ out_scales) {
  const int lane = threadIdx.x & 63;
  const int gw = block * kWavesPerBlock + (threadIdx.x >> 6);
  if (gw >= T * parts) return;
  const int t = gw / parts;
  const int nb = H / MOE_MX_BLOCK;
  const int nch = H / 8;
  const int b0 = (gw - t * parts) * bpp;
  const int nbp = min(bpp, nb - b0);
  const int my_dst = lane < k ? dst_row[(size_t)t * k + lane] : -1;
  const int blk = lane >> 2;         // block inside a step
  const int sub = lane & 3;          // 16-byte chunk inside the block
  const u32x4* src = x + (size_t)t * nch;

  u32x4 v[MAXST];
#pragma unroll
  for (int st = 0; st < MAXST; ++st) {
    const int bl = st * kMxStepBlocks + blk;
    v[st] = u32x4{0u, 0u, 0u, 0u};
    if (bl < nbp) v[st] = stream_load(src + (b0 + bl) * 4 + sub);
  }

  uint32_t sreg[kScaleSlots];        // E8M0 byte of part-local block (s*64 + lane)
#pragma unroll
  for (int s = 0; s < kScaleSlots; ++s) sreg[s] = 0u;
  u32x2 q[MAXST];
#pragma unroll
  for (int st = 0; st < MAXST; ++st) {
    uint32_t m = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t w = v[st][c] & 0x7FFF7FFFu;
      m = max(m, max(w & 0xFFFFu, w >> 16));
    }
    m = max(m, dpp_u32<0xB1>(m));
    m = max(m, dpp_u32<0x4E>(m));
    const float amax = __uint_as_float(m << 16);
    int e = amax == 0.0f ? -127 : __builtin_amdgcn_frexp_expf(amax) - 1 - 8;
    e = min(max(e, -127), 127);
    const float inv = __builtin_amdgcn_ldexpf(1.0f, -e);
    q[st][0] = quant_pair_hw(v[st][0], inv) | (quant_pair_hw(v[st][1], inv) << 16);
    q[st][1] = quant_pair_hw(v[st][2], inv) | (quant_pair_hw(v[st][3], inv) << 16);
    // lane L keeps the byte of part-local block L + 64*slot: in step st the
    // lanes of row (st % 4) receive block (st*16 + L % 16) from its first lane
    const uint32_t sb = (uint32_t)(e + 127);
    const uint32_t got = (uint32_t)__shfl((int)sb, 4 * (lane & 15));
#pragma unroll
    for (int s = 0; s < kScaleSlots; ++s)
      if (st / 4 == s && (lane >> 4) == (st & 3)) sreg[s] = got;
  }

  for (int j = 0; j < k; ++j) {
    const int d = read_lane(my_dst, j);
    if (d < 0 || d >= num_rows) continue;
#pragma unroll
    for (int st = 0; st < MAXST; ++st) {
      const int bl = st * kMxStepBlocks + blk;
      if (bl < nbp)
        stream_store(q[st], reinterpret_cast<u32x2*>(out + (size_t)d * H +
                                                     (size_t)(b0 + bl) * MOE_MX_BLOCK) + sub);
    }
    uint8_t* srow = out_scales + (size_t)d * nb + b0;
#pragma unroll
    for (int s = 0; s < kScaleSlots; ++s) {
      const int b = s * 64 + lane;
      if (b < nbp) srow[b] = (uint8_t)sreg[s];
    }
  }
}

// Split a row of `units` into parts so that the launch has about
// kTargetWaves waves, each part a multiple of `align` units (but at least
// `min_units` and at most `max_units` units).
inline void split_row(int T, int units, int align, int max_units, int* parts, int* per_part) {
  int p = T > 0 ? (kTargetWaves + T - 1) / T : 1;
  p = max(1, min(p, units / align));
  int per = (units + p - 1) / p;
  per = (per + align - 1) / align * align;
  if (per > max_units) per = max_units;
  *per_part = per;
  *parts = (units + per - 1) / per;
}

}  // namespace
}  // namespace moe
