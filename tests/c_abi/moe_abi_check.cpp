// Stand-alone check of the C ABI (include/moe.h): a host program that uses
// libmoe_layout.so with nothing but the HIP runtime for device memory - no
// Python, no torch. It runs a small layer (softmax routing, layout, bf16
// dispatch, identity experts, combine) and the deduplicated dispatch with
// the hierarchical combine, and checks what the method fixes without an
// oracle:
//   - counts add up to T*k, offsets are their exclusive prefix sums, dst_row
//     is a bijection onto [0, T*k) with src_pair its inverse, rows of one
//     expert come in token order;
//   - with identity experts and normalised weights, combine(dispatch(x))
//     returns x bit for bit (the weights sum to 1 within k fp32 ulps, far
//     below half a bf16 ulp);
//   - the fanned-out (token, rank) rows equal the dispatched rows, and the
//     two-level sum stays within two bf16 ulps of x;
//   - the batched routing, layout and (token, rank) layout give, per batch,
//     what the single calls give;
//   - a call with bad arguments returns MOE_ERR_INVALID and names itself.
// Prints "c-abi check ok" and exits 0 on success.

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "moe.h"

#define HIP_OK(x)                                                                      \
  do {                                                                                 \
    hipError_t e_ = (x);                                                               \
    if (e_ != hipSuccess) {                                                            \
      std::fprintf(stderr, "%s:%d %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
      return 1;                                                                        \
    }                                                                                  \
  } while (0)
#define MOE_CALL(x)                                                                    \
  do {                                                                                 \
    int s_ = (x);                                                                      \
    if (s_ != MOE_OK) {                                                                \
      std::fprintf(stderr, "%s -> %s: %s\n", #x, moe_status_string(s_),               \
                   moe_last_error());                                                  \
      return 1;                                                                        \
    }                                                                                  \
  } while (0)
#define CHECK(c, msg)                                 \
  do {                                                \
    if (!(c)) {                                       \
      std::fprintf(stderr, "check failed: %s\n", msg); \
      return 1;                                       \
    }                                                 \
  } while (0)

namespace {

uint32_t next(uint64_t& s) {
  s = s * 6364136223846793005ULL + 1442695040888963407ULL;
  return (uint32_t)(s >> 33);
}

float bf16_value(uint16_t b) {
  uint32_t w = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &w, 4);
  return f;
}

template <typename T>
int to_device(const std::vector<T>& h, T** d) {
  HIP_OK(hipMalloc((void**)d, h.size() * sizeof(T) + 16));
  HIP_OK(hipMemcpy(*d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice));
  return 0;
}

template <typename T>
int alloc(size_t n, T** d) {
  HIP_OK(hipMalloc((void**)d, n * sizeof(T) + 16));
  return 0;
}

template <typename T>
int to_host(const T* d, size_t n, std::vector<T>& h) {
  h.resize(n);
  HIP_OK(hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost));
  return 0;
}

}  // namespace

int main() {
  const int T = 96, H = 256, E = 8, k = 2, R = 4;   // 192 pairs: one tile, tokens ragged
  const int pairs = T * k, rows = T * k, nrr = T * (k < R ? k : R);
  uint64_t seed = 12345;

  std::vector<float> logits((size_t)T * E);
  for (auto& v : logits) v = (float)(next(seed) % 4096) / 1024.0f - 2.0f;
  std::vector<uint16_t> x((size_t)T * H);
  for (auto& v : x) {
    const int q = (int)(next(seed) % 33) - 16;          // small integers / 8: exact in bf16
    const float f = (float)q / 8.0f;
    uint32_t w;
    std::memcpy(&w, &f, 4);
    v = (uint16_t)(w >> 16);
  }

  float *d_logits, *d_w;
  uint16_t *d_x, *d_rows, *d_out, *d_sent, *d_part;
  int32_t *d_idx, *d_ec, *d_eo, *d_rc, *d_ro, *d_rtc, *d_dst, *d_src, *d_ovf;
  int32_t *d_rtc2, *d_rto, *d_rrow, *d_srow, *d_rtok;
  if (to_device(logits, &d_logits) || to_device(x, &d_x)) return 1;
  if (alloc(pairs, &d_w) || alloc(pairs, &d_idx) || alloc(E, &d_ec) || alloc(E + 1, &d_eo) ||
      alloc(R, &d_rc) || alloc(R + 1, &d_ro) || alloc(R, &d_rtc) || alloc(pairs, &d_dst) ||
      alloc(rows, &d_src) || alloc(1, &d_ovf) || alloc((size_t)rows * H, &d_rows) ||
      alloc((size_t)T * H, &d_out) || alloc(R, &d_rtc2) || alloc(R + 1, &d_rto) ||
      alloc(pairs, &d_rrow) || alloc(pairs, &d_srow) || alloc(nrr, &d_rtok) ||
      alloc((size_t)nrr * H, &d_sent) || alloc((size_t)nrr * H, &d_part))
    return 1;
  const size_t ws_bytes = moe_layout_workspace_bytes(T, E, k);
  const size_t rws_bytes = moe_rank_layout_workspace_bytes(T, k, R);
  void *d_ws, *d_rws;
  HIP_OK(hipMalloc(&d_ws, ws_bytes + 16));
  HIP_OK(hipMalloc(&d_rws, rws_bytes + 16));
  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));

  // ---- flat pass: route, layout, dispatch, identity experts, combine
  MOE_CALL(moe_route(T, E, k, d_logits, nullptr, MOE_SCORE_SOFTMAX, 1, 1, d_idx, d_w, st));
  MOE_CALL(moe_layout(T, E, k, R, 0, d_idx, d_ec, d_eo, d_rc, d_ro, d_rtc, d_dst, d_src, d_ovf,
                      d_ws, ws_bytes, st));
  MOE_CALL(moe_dispatch(T, H, k, rows, d_x, d_dst, MOE_DTYPE_BF16, d_rows, nullptr, st));
  MOE_CALL(moe_combine(T, H, k, rows, d_rows, d_dst, d_w, d_out, st));
  HIP_OK(hipStreamSynchronize(st));

  std::vector<int32_t> idx, ec, eo, rc, ro, dst, src;
  std::vector<float> w;
  std::vector<uint16_t> out;
  if (to_host(d_idx, pairs, idx) || to_host(d_w, pairs, w) || to_host(d_ec, E, ec) ||
      to_host(d_eo, E + 1, eo) || to_host(d_rc, R, rc) || to_host(d_ro, R + 1, ro) ||
      to_host(d_dst, pairs, dst) || to_host(d_src, rows, src) ||
      to_host(d_out, (size_t)T * H, out))
    return 1;

  for (int t = 0; t < T; ++t) {
    CHECK(idx[t * k] != idx[t * k + 1], "distinct experts per token");
    const double s = (double)w[t * k] + (double)w[t * k + 1];
    CHECK(std::fabs(s - 1.0) <= 4 * 1.2e-7, "weights are normalised");
  }
  int total = 0;
  for (int e = 0; e < E; ++e) {
    CHECK(eo[e] == total, "offsets are the exclusive prefix sums");
    total += ec[e];
  }
  CHECK(total == pairs && eo[E] == pairs, "counts add up to T*k");
  for (int r = 0; r < R; ++r)
    CHECK(rc[r] == ec[2 * r] + ec[2 * r + 1] && ro[r] == eo[2 * r], "rank counts and offsets");
  std::vector<int> seen(rows, 0);
  for (int p = 0; p < pairs; ++p) {
    CHECK(dst[p] >= 0 && dst[p] < rows && !seen[dst[p]]++, "dst_row is a bijection");
    CHECK(src[dst[p]] == p, "src_pair inverts dst_row");
    const int e = idx[p];
    CHECK(dst[p] >= eo[e] && dst[p] < eo[e + 1], "row inside its expert's segment");
  }
  for (int e = 0; e < E; ++e)
    for (int r = eo[e] + 1; r < eo[e + 1]; ++r) CHECK(src[r] > src[r - 1], "stable order");
  CHECK(std::memcmp(out.data(), x.data(), x.size() * 2) == 0, "combine(dispatch(x)) == x");

  // ---- hierarchical pass on the same routing
  MOE_CALL(moe_rank_layout(T, E, k, R, d_idx, d_rtc2, d_rto, d_rrow, d_srow, d_rtok, d_rws,
                           rws_bytes, st));
  MOE_CALL(moe_dispatch(T, H, k, nrr, d_x, d_srow, MOE_DTYPE_BF16, d_sent, nullptr, st));
  HIP_OK(hipMemsetAsync(d_rows, 0xFF, (size_t)rows * H * 2, st));
  MOE_CALL(moe_expand(T, H, k, MOE_DTYPE_BF16, nrr, d_sent, nullptr, d_rrow, d_rtok, rows, d_dst, d_rows,
                      nullptr, st));
  MOE_CALL(moe_combine_local(T, H, k, rows, d_rows, d_dst, d_rrow, d_rtok, d_w, nrr, d_part, st));
  MOE_CALL(moe_combine_partials(T, H, k, nrr, d_part, d_srow, d_out, st));
  HIP_OK(hipStreamSynchronize(st));
  std::vector<int32_t> rtc, rtc2, rrow;
  std::vector<uint16_t> fanned;
  if (to_host(d_rtc, R, rtc) || to_host(d_rtc2, R, rtc2) || to_host(d_rrow, pairs, rrow) ||
      to_host(d_rows, (size_t)rows * H, fanned) || to_host(d_out, (size_t)T * H, out))
    return 1;
  for (int r = 0; r < R; ++r) CHECK(rtc[r] == rtc2[r], "distinct tokens per rank agree");
  for (int p = 0; p < pairs; ++p) {
    const int t = p / k;
    CHECK(std::memcmp(&fanned[(size_t)dst[p] * H], &x[(size_t)t * H], H * 2) == 0,
          "fanned-out rows equal the dispatched rows");
    const bool same_rank = idx[t * k] / 2 == idx[t * k + 1] / 2;
    CHECK(rrow[t * k] >= 0 && (rrow[t * k] == rrow[t * k + 1]) == same_rank,
          "slots on one rank share a row");
  }
  for (size_t i = 0; i < x.size(); ++i) {
    const float a = bf16_value(out[i]), b = bf16_value(x[i]);
    CHECK(std::fabs(a - b) <= std::ldexp(std::fabs(b), -7), "two-level sum within two ulps of x");
  }

  // ---- batched calls: batch 0 repeats the flat pass's routing and layout,
  // batch 1 routes other logits; each batch must equal its single calls
  {
    std::vector<float> logits1((size_t)T * E);
    for (auto& v : logits1) v = (float)(next(seed) % 4096) / 1024.0f - 2.0f;
    float *d_logits1, *d_wb[2];
    int32_t *d_ib[2], *d_ecb[2], *d_eob[2], *d_rcb[2], *d_rob[2], *d_rtcb[2], *d_dstb[2],
        *d_srcb[2], *d_ovfb[2];
    void* d_wsb[2];
    if (to_device(logits1, &d_logits1)) return 1;
    for (int b = 0; b < 2; ++b) {
      if (alloc(pairs, &d_wb[b]) || alloc(pairs, &d_ib[b]) || alloc(E, &d_ecb[b]) ||
          alloc(E + 1, &d_eob[b]) || alloc(R, &d_rcb[b]) || alloc(R + 1, &d_rob[b]) ||
          alloc(R, &d_rtcb[b]) || alloc(pairs, &d_dstb[b]) || alloc(rows, &d_srcb[b]) ||
          alloc(1, &d_ovfb[b]))
        return 1;
      HIP_OK(hipMalloc(&d_wsb[b], ws_bytes + 16));
    }
    const moe_route_io rio[2] = {{d_logits, nullptr, d_ib[0], d_wb[0]},
                                 {d_logits1, nullptr, d_ib[1], d_wb[1]}};
    MOE_CALL(moe_route_batched(2, rio, T, E, k, MOE_SCORE_SOFTMAX, 1, 1, st));
    moe_layout_io lio[2];
    for (int b = 0; b < 2; ++b)
      lio[b] = moe_layout_io{d_ib[b], d_ecb[b], d_eob[b], d_rcb[b], d_rob[b], d_rtcb[b],
                             d_dstb[b], d_srcb[b], d_ovfb[b], d_wsb[b], ws_bytes};
    MOE_CALL(moe_layout_batched(2, lio, T, E, k, R, 0, st));
    // single calls on batch 1's logits, into the flat pass's buffers
    MOE_CALL(moe_route(T, E, k, d_logits1, nullptr, MOE_SCORE_SOFTMAX, 1, 1, d_idx, d_w, st));
    MOE_CALL(moe_layout(T, E, k, R, 0, d_idx, d_ec, d_eo, d_rc, d_ro, d_rtc, d_dst, d_src, d_ovf,
                        d_ws, ws_bytes, st));
    HIP_OK(hipStreamSynchronize(st));
    std::vector<int32_t> i0, i1, d0, d1, s0, s1, e1, one_i, one_d, one_s, one_e;
    std::vector<float> w0, one_w;
    if (to_host(d_ib[0], pairs, i0) || to_host(d_ib[1], pairs, i1) ||
        to_host(d_dstb[0], pairs, d0) || to_host(d_dstb[1], pairs, d1) ||
        to_host(d_srcb[0], rows, s0) || to_host(d_srcb[1], rows, s1) ||
        to_host(d_ecb[1], E, e1) || to_host(d_wb[0], pairs, w0) ||
        to_host(d_idx, pairs, one_i) || to_host(d_dst, pairs, one_d) ||
        to_host(d_src, rows, one_s) || to_host(d_ec, E, one_e) || to_host(d_w, pairs, one_w))
      return 1;
    CHECK(i0 == idx && d0 == dst && s0 == src, "batch 0 equals the flat pass's route and layout");
    CHECK(std::memcmp(w0.data(), w.data(), pairs * sizeof(float)) == 0, "batch 0 weights");
    CHECK(i1 == one_i && d1 == one_d && s1 == one_s && e1 == one_e,
          "batch 1 equals its single calls");
    (void)one_w;
    // batched (token, rank) layouts of both routings; batch 0 against the flat
    // pass's rank_row, batch 1 against a single call on its routing (d_idx)
    int32_t *d_rcntb[2], *d_roffb[2], *d_rrowb[2], *d_srowb[2], *d_rtokb[2];
    void* d_rwsb[2];
    for (int b = 0; b < 2; ++b) {
      if (alloc(R, &d_rcntb[b]) || alloc(R + 1, &d_roffb[b]) || alloc(pairs, &d_rrowb[b]) ||
          alloc(pairs, &d_srowb[b]) || alloc(nrr, &d_rtokb[b]))
        return 1;
      HIP_OK(hipMalloc(&d_rwsb[b], rws_bytes + 16));
    }
    moe_rank_layout_io rlio[2];
    for (int b = 0; b < 2; ++b)
      rlio[b] = moe_rank_layout_io{d_ib[b], d_rcntb[b], d_roffb[b], d_rrowb[b], d_srowb[b],
                                   d_rtokb[b], d_rwsb[b], rws_bytes};
    MOE_CALL(moe_rank_layout_batched(2, rlio, T, E, k, R, st));
    MOE_CALL(moe_rank_layout(T, E, k, R, d_idx, d_rtc2, d_rto, d_rrow, d_srow, d_rtok, d_rws,
                             rws_bytes, st));
    HIP_OK(hipStreamSynchronize(st));
    std::vector<int32_t> rr0, rr1, sr1, rt1, ro1, one_rr, one_sr, one_rt, one_ro;
    if (to_host(d_rrowb[0], pairs, rr0) || to_host(d_rrowb[1], pairs, rr1) ||
        to_host(d_srowb[1], pairs, sr1) || to_host(d_rtokb[1], nrr, rt1) ||
        to_host(d_roffb[1], R + 1, ro1) || to_host(d_rrow, pairs, one_rr) ||
        to_host(d_srow, pairs, one_sr) || to_host(d_rtok, nrr, one_rt) ||
        to_host(d_rto, R + 1, one_ro))
      return 1;
    CHECK(rr0 == rrow, "batched rank layout 0 equals the flat pass's");
    CHECK(rr1 == one_rr && sr1 == one_sr && rt1 == one_rt && ro1 == one_ro,
          "batched rank layout 1 equals its single call");
    for (int b = 0; b < 2; ++b) {
      void* bb[] = {d_rcntb[b], d_roffb[b], d_rrowb[b], d_srowb[b], d_rtokb[b], d_rwsb[b]};
      for (void* q : bb) HIP_OK(hipFree(q));
    }
    const int bad_n = moe_route_batched(0, rio, T, E, k, MOE_SCORE_SOFTMAX, 1, 1, st);
    CHECK(bad_n == MOE_ERR_INVALID, "zero batches are rejected");
    HIP_OK(hipFree(d_logits1));
    for (int b = 0; b < 2; ++b) {
      void* bb[] = {d_wb[b], d_ib[b], d_ecb[b], d_eob[b], d_rcb[b], d_rob[b], d_rtcb[b],
                    d_dstb[b], d_srcb[b], d_ovfb[b], d_wsb[b]};
      for (void* q : bb) HIP_OK(hipFree(q));
    }
  }

  // ---- an error is reported on the host, before anything is enqueued
  const int bad = moe_dispatch(T, 100, k, rows, d_x, d_dst, MOE_DTYPE_BF16, d_rows, nullptr, st);
  CHECK(bad == MOE_ERR_INVALID, "hidden=100 is rejected");
  CHECK(std::strncmp(moe_last_error(), "moe_dispatch", 12) == 0, "the error names the call");

  HIP_OK(hipStreamDestroy(st));
  void* bufs[] = {d_logits, d_w, d_x, d_rows, d_out, d_sent, d_part, d_idx, d_ec, d_eo, d_rc,
                  d_ro, d_rtc, d_dst, d_src, d_ovf, d_rtc2, d_rto, d_rrow, d_srow, d_rtok, d_ws,
                  d_rws};
  for (void* b : bufs) HIP_OK(hipFree(b));
  std::printf("c-abi check ok: T=%d H=%d E=%d k=%d R=%d\n", T, H, E, k, R);
  return 0;
}
