// C ABI of the MoE hot path (declared in include/moe.h).
//
// Every entry point validates its scalar and pointer arguments on the host
// before it enqueues anything, so that a bad call changes no memory and can
// be tested without a GPU. Launches go to the caller's stream; the library
// never allocates, frees or synchronises.

#include <limits.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "kernels.h"

// Device scratch of moe_layout_no_alloc: the per-tile counts of the layout
// kernels. Each GPU holds its own copy. Host code never uses this name as an
// address (on the host it is only a stand-in for the symbol): the device
// address of each GPU's copy comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[MOE_LAYOUT_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[256] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return MOE_OK;
}

int from_hip(hipError_t err, const char* what) {
  if (err == hipSuccess) return ok();
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Limits shared by routing and layout.
int check_topk(const char* fn, int T, int E, int k) {
  if (T < 0) return fail(MOE_ERR_INVALID, "%s: num_tokens=%d < 0", fn, T);
  if (E < 1) return fail(MOE_ERR_INVALID, "%s: num_experts=%d < 1", fn, E);
  if (E > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_UNSUPPORTED, "%s: num_experts=%d > %d", fn, E, MOE_MAX_EXPERTS);
  if (k < 1 || k > E) return fail(MOE_ERR_INVALID, "%s: top_k=%d not in [1, %d]", fn, k, E);
  if (k > MOE_MAX_TOPK)
    return fail(MOE_ERR_UNSUPPORTED, "%s: top_k=%d > %d", fn, k, MOE_MAX_TOPK);
  if ((long long)T * k > INT_MAX) return fail(MOE_ERR_INVALID, "%s: num_tokens*top_k overflows", fn);
  return MOE_OK;
}

int check_rows(const char* fn, int T, int H, int k, int num_rows) {
  if (T < 0) return fail(MOE_ERR_INVALID, "%s: num_tokens=%d < 0", fn, T);
  if (k < 1 || k > MOE_MAX_TOPK)
    return fail(MOE_ERR_INVALID, "%s: top_k=%d not in [1, %d]", fn, k, MOE_MAX_TOPK);
  if (H < 8 || H % 8 != 0)
    return fail(MOE_ERR_INVALID, "%s: hidden=%d must be a positive multiple of 8", fn, H);
  if (num_rows < 0) return fail(MOE_ERR_INVALID, "%s: num_rows=%d < 0", fn, num_rows);
  if ((long long)T * k > INT_MAX) return fail(MOE_ERR_INVALID, "%s: num_tokens*top_k overflows", fn);
  // waves are indexed with int: T * parts <= T * H / 8
  if ((long long)T * (H / 8) > INT_MAX) return fail(MOE_ERR_INVALID, "%s: num_tokens*hidden too large", fn);
  return MOE_OK;
}

int check_route(const char* fn, int num_tokens, int num_experts, int top_k, const float* logits,
                const float* bias, int score_fn, int num_groups, int topk_groups,
                const int32_t* topk_idx, const float* topk_weights) {
  int st = check_topk(fn, num_tokens, num_experts, top_k);
  if (st != MOE_OK) return st;
  if (score_fn != MOE_SCORE_SOFTMAX && score_fn != MOE_SCORE_SIGMOID)
    return fail(MOE_ERR_INVALID, "%s: score_fn=%d", fn, score_fn);
  if (num_groups < 1 || num_groups > MOE_MAX_GROUPS || num_experts % num_groups != 0)
    return fail(MOE_ERR_INVALID, "%s: num_groups=%d must divide num_experts=%d and be <= %d", fn,
                num_groups, num_experts, MOE_MAX_GROUPS);
  if (score_fn == MOE_SCORE_SOFTMAX && num_groups != 1)
    return fail(MOE_ERR_UNSUPPORTED, "%s: softmax routing takes no groups", fn);
  if (topk_groups < 1 || topk_groups > num_groups)
    return fail(MOE_ERR_INVALID, "%s: topk_groups=%d not in [1, %d]", fn, topk_groups, num_groups);
  if ((long long)topk_groups * (num_experts / num_groups) < top_k)
    return fail(MOE_ERR_INVALID, "%s: the kept groups hold fewer than top_k experts", fn);
  if (num_tokens > 0 && (!logits || !topk_idx || !topk_weights))
    return fail(MOE_ERR_INVALID, "%s: NULL logits/topk_idx/topk_weights", fn);
  if (!aligned(logits, 4) || !aligned(bias, 4) || !aligned(topk_idx, 4) || !aligned(topk_weights, 4))
    return fail(MOE_ERR_INVALID, "%s: pointers must be 4-byte aligned", fn);
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID: return "MOE_ERR_INVALID";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error; }

int moe_route(int num_tokens, int num_experts, int top_k, const float* logits,
              const float* bias, int score_fn, int num_groups, int topk_groups,
              int32_t* topk_idx, float* topk_weights, void* stream) {
  const char* fn = "moe_route";
  const int st = check_route(fn, num_tokens, num_experts, top_k, logits, bias, score_fn,
                             num_groups, topk_groups, topk_idx, topk_weights);
  if (st != MOE_OK) return st;
  return from_hip(moe::launch_route(num_tokens, num_experts, top_k, logits, bias,
                                    score_fn == MOE_SCORE_SIGMOID, num_groups, topk_groups,
                                    topk_idx, topk_weights, static_cast<hipStream_t>(stream)),
                  fn);
}

int moe_route_batched(int num_batches, const moe_route_io* batches, int num_tokens,
                      int num_experts, int top_k, int score_fn, int num_groups,
                      int topk_groups, void* stream) {
  const char* fn = "moe_route_batched";
  if (num_batches < 1 || num_batches > MOE_MAX_BATCHES || !batches)
    return fail(MOE_ERR_INVALID, "%s: num_batches=%d not in [1, %d] (or NULL batches)", fn,
                num_batches, MOE_MAX_BATCHES);
  moe::RouteBatches rb{};
  for (int b = 0; b < num_batches; ++b) {
    const int st = check_route(fn, num_tokens, num_experts, top_k, batches[b].logits,
                               batches[b].bias, score_fn, num_groups, topk_groups,
                               batches[b].topk_idx, batches[b].topk_weights);
    if (st != MOE_OK) return st;
    rb.logits[b] = batches[b].logits;
    rb.bias[b] = batches[b].bias;
    rb.idx[b] = batches[b].topk_idx;
    rb.w[b] = batches[b].topk_weights;
  }
  return from_hip(moe::launch_route_batches(num_batches, rb, num_tokens, num_experts, top_k,
                                            score_fn == MOE_SCORE_SIGMOID, num_groups,
                                            topk_groups, static_cast<hipStream_t>(stream)),
                  fn);
}

size_t moe_layout_workspace_bytes(int num_tokens, int num_experts, int top_k) {
  if (num_tokens < 0 || num_experts < 1 || top_k < 1 || top_k > MOE_MAX_TOPK) return 0;
  return moe::layout_workspace_bytes(num_tokens, num_experts, top_k);
}

}  // extern "C"

namespace {

int check_layout(const char* fn, int num_tokens, int num_experts, int top_k, int num_ranks,
                 int capacity, const int32_t* topk_idx, int32_t* expert_counts,
                 int32_t* expert_offsets, int32_t* rank_counts, int32_t* rank_offsets,
                 int32_t* rank_token_counts, int32_t* dst_row, int32_t* src_pair,
                 int32_t* overflow, void* workspace, size_t workspace_bytes) {
  int st = check_topk(fn, num_tokens, num_experts, top_k);
  if (st != MOE_OK) return st;
  if (num_ranks < 1 || num_ranks > num_experts || num_experts % num_ranks != 0)
    return fail(MOE_ERR_INVALID, "%s: num_ranks=%d must divide num_experts=%d", fn, num_ranks,
                num_experts);
  if (capacity < 0) return fail(MOE_ERR_INVALID, "%s: capacity=%d < 0", fn, capacity);
  if ((long long)num_experts * capacity > INT_MAX)
    return fail(MOE_ERR_INVALID, "%s: num_experts*capacity overflows", fn);
  if (!expert_counts || !expert_offsets || !rank_counts || !rank_offsets || !overflow)
    return fail(MOE_ERR_INVALID, "%s: NULL count/offset/overflow output", fn);
  const long long rows = capacity > 0 ? (long long)num_experts * capacity
                                      : (long long)num_tokens * top_k;
  if (num_tokens > 0 && (!topk_idx || !dst_row))
    return fail(MOE_ERR_INVALID, "%s: NULL topk_idx/dst_row", fn);
  if (rows > 0 && !src_pair) return fail(MOE_ERR_INVALID, "%s: NULL src_pair", fn);
  const void* ptrs[] = {topk_idx, expert_counts, expert_offsets, rank_counts, rank_offsets,
                        rank_token_counts, dst_row, src_pair, overflow};
  for (const void* p : ptrs)
    if (!aligned(p, 4)) return fail(MOE_ERR_INVALID, "%s: pointers must be 4-byte aligned", fn);
  const size_t need = moe::layout_workspace_bytes(num_tokens, num_experts, top_k);
  if (workspace_bytes < need || (need > 0 && !workspace))
    return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace_bytes);
  if (!aligned(workspace, 4)) return fail(MOE_ERR_INVALID, "%s: workspace not aligned", fn);
  return MOE_OK;
}

int check_dispatch(const char* fn, int num_tokens, int hidden, int top_k, int num_rows,
                   const void* x_bf16, const int32_t* dst_row, int out_dtype, void* out,
                   void* out_scales) {
  int st = check_rows(fn, num_tokens, hidden, top_k, num_rows);
  if (st != MOE_OK) return st;
  if (out_dtype != MOE_DTYPE_BF16 && out_dtype != MOE_DTYPE_FP8_E4M3 &&
      out_dtype != MOE_DTYPE_MXFP8_E4M3)
    return fail(MOE_ERR_INVALID, "%s: out_dtype=%d", fn, out_dtype);
  const bool fp8 = out_dtype == MOE_DTYPE_FP8_E4M3;
  const bool mx = out_dtype == MOE_DTYPE_MXFP8_E4M3;
  if (fp8 && hidden % MOE_FP8_BLOCK != 0)
    return fail(MOE_ERR_INVALID, "%s: FP8 needs hidden %% %d == 0 (hidden=%d)", fn,
                MOE_FP8_BLOCK, hidden);
  if (mx && hidden % MOE_MX_BLOCK != 0)
    return fail(MOE_ERR_INVALID, "%s: MXFP8 needs hidden %% %d == 0 (hidden=%d)", fn,
                MOE_MX_BLOCK, hidden);
  if (num_tokens > 0 && (!x_bf16 || !dst_row))
    return fail(MOE_ERR_INVALID, "%s: NULL x/dst_row", fn);
  if (num_rows > 0 && !out) return fail(MOE_ERR_INVALID, "%s: NULL out", fn);
  if ((fp8 || mx) && num_rows > 0 && !out_scales)
    return fail(MOE_ERR_INVALID, "%s: NULL out_scales", fn);
  if (!fp8 && !mx && out_scales) return fail(MOE_ERR_INVALID, "%s: out_scales is for FP8 only", fn);
  if (!aligned(x_bf16, 16) || !aligned(out, 16))
    return fail(MOE_ERR_INVALID, "%s: x and out must be 16-byte aligned", fn);
  if (!aligned(dst_row, 4) || (fp8 && !aligned(out_scales, 4)))
    return fail(MOE_ERR_INVALID, "%s: dst_row/out_scales must be 4-byte aligned", fn);
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_layout(int num_tokens, int num_experts, int top_k, int num_ranks, int capacity,
               const int32_t* topk_idx, int32_t* expert_counts, int32_t* expert_offsets,
               int32_t* rank_counts, int32_t* rank_offsets, int32_t* rank_token_counts,
               int32_t* dst_row, int32_t* src_pair, int32_t* overflow, void* workspace,
               size_t workspace_bytes, void* stream) {
  const char* fn = "moe_layout";
  const int st = check_layout(fn, num_tokens, num_experts, top_k, num_ranks, capacity, topk_idx,
                              expert_counts, expert_offsets, rank_counts, rank_offsets,
                              rank_token_counts, dst_row, src_pair, overflow, workspace,
                              workspace_bytes);
  if (st != MOE_OK) return st;
  return from_hip(moe::launch_layout(num_tokens, num_experts, top_k, num_ranks, capacity,
                                     topk_idx, expert_counts, expert_offsets, rank_counts,
                                     rank_offsets, rank_token_counts, dst_row, src_pair,
                                     overflow, workspace, static_cast<hipStream_t>(stream)),
                  fn);
}

int moe_layout_batched(int num_batches, const moe_layout_io* batches, int num_tokens,
                       int num_experts, int top_k, int num_ranks, int capacity, void* stream) {
  const char* fn = "moe_layout_batched";
  if (num_batches < 1 || num_batches > MOE_MAX_BATCHES || !batches)
    return fail(MOE_ERR_INVALID, "%s: num_batches=%d not in [1, %d] (or NULL batches)", fn,
                num_batches, MOE_MAX_BATCHES);
  moe::LayoutBatches lb{};
  for (int b = 0; b < num_batches; ++b) {
    const moe_layout_io& io = batches[b];
    const int st = check_layout(fn, num_tokens, num_experts, top_k, num_ranks, capacity,
                                io.topk_idx, io.expert_counts, io.expert_offsets,
                                io.rank_counts, io.rank_offsets, io.rank_token_counts,
                                io.dst_row, io.src_pair, io.overflow, io.workspace,
                                io.workspace_bytes);
    if (st != MOE_OK) return st;
    if ((io.rank_token_counts == nullptr) != (batches[0].rank_token_counts == nullptr))
      return fail(MOE_ERR_INVALID, "%s: rank_token_counts must be given for all batches or none",
                  fn);
    lb.b[b] = moe::LayoutBatch{io.topk_idx, io.expert_counts, io.expert_offsets, io.rank_counts,
                               io.rank_offsets, io.rank_token_counts, io.dst_row, io.src_pair,
                               io.overflow, io.workspace};
  }
  return from_hip(moe::launch_layout_batches(num_batches, lb, num_tokens, num_experts, top_k,
                                             num_ranks, capacity,
                                             static_cast<hipStream_t>(stream)),
                  fn);
}

}  // extern "C"

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxScratchDevices];   // device address of each GPU's scratch

// Device address of the current device's copy of `scratch`, looked up on the
// first call with that device current and kept until the process ends.
int scratch_address(const char* fn, void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return from_hip(e, fn);
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(MOE_ERR_UNSUPPORTED, "%s: device %d beyond the %d with a scratch address", fn,
                dev, kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return fail(MOE_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                  hipGetErrorString(err));
    }
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_layout_no_alloc(int num_tokens, int num_experts, int top_k, int num_ranks,
                        int capacity, const int32_t* topk_idx, int32_t* expert_counts,
                        int32_t* expert_offsets, int32_t* rank_counts, int32_t* rank_offsets,
                        int32_t* rank_token_counts, int32_t* dst_row, int32_t* src_pair,
                        int32_t* overflow, void* stream) {
  const char* fn = "moe_layout_no_alloc";
  int st = check_topk(fn, num_tokens, num_experts, top_k);
  if (st != MOE_OK) return st;
  const size_t need = moe::layout_workspace_bytes(num_tokens, num_experts, top_k);
  if (need > MOE_LAYOUT_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE,
                "%s: these sizes need %zu bytes of scratch, more than the library's %u "
                "(call moe_layout with a workspace instead)", fn, need,
                (unsigned)MOE_LAYOUT_SCRATCH_BYTES);
  // the remaining checks of moe_layout, with a stand-in for the workspace
  // (an aligned non-null value of the scratch's size; nothing dereferences it)
  st = check_layout(fn, num_tokens, num_experts, top_k, num_ranks, capacity, topk_idx,
                    expert_counts, expert_offsets, rank_counts, rank_offsets, rank_token_counts,
                    dst_row, src_pair, overflow, reinterpret_cast<void*>(uintptr_t{256}),
                    MOE_LAYOUT_SCRATCH_BYTES);
  if (st != MOE_OK) return st;
  void* ws = nullptr;
  st = scratch_address(fn, &ws);
  if (st != MOE_OK) return st;
  return from_hip(moe::launch_layout(num_tokens, num_experts, top_k, num_ranks, capacity,
                                     topk_idx, expert_counts, expert_offsets, rank_counts,
                                     rank_offsets, rank_token_counts, dst_row, src_pair,
                                     overflow, ws, static_cast<hipStream_t>(stream)),
                  fn);
}

int moe_layout_dispatch_is_fused(int num_tokens, int top_k, int capacity) {
  if (num_tokens < 0 || top_k < 1 || top_k > MOE_MAX_TOPK || capacity < 0) return 0;
  return moe::layout_dispatch_fused(num_tokens, top_k, capacity) ? 1 : 0;
}

int moe_layout_dispatch(int num_tokens, int num_experts, int top_k, int num_ranks,
                        int capacity, const int32_t* topk_idx, int32_t* expert_counts,
                        int32_t* expert_offsets, int32_t* rank_counts, int32_t* rank_offsets,
                        int32_t* rank_token_counts, int32_t* dst_row, int32_t* src_pair,
                        int32_t* overflow, void* workspace, size_t workspace_bytes, int hidden,
                        const void* x_bf16, int out_dtype, void* out, void* out_scales,
                        void* stream) {
  const char* fn = "moe_layout_dispatch";
  int st = check_layout(fn, num_tokens, num_experts, top_k, num_ranks, capacity, topk_idx,
                        expert_counts, expert_offsets, rank_counts, rank_offsets,
                        rank_token_counts, dst_row, src_pair, overflow, workspace,
                        workspace_bytes);
  if (st != MOE_OK) return st;
  const long long rows = capacity > 0 ? (long long)num_experts * capacity
                                      : (long long)num_tokens * top_k;
  st = check_dispatch(fn, num_tokens, hidden, top_k, (int)rows, x_bf16, dst_row, out_dtype, out,
                      out_scales);
  if (st != MOE_OK) return st;
  return from_hip(moe::launch_layout_dispatch(num_tokens, num_experts, top_k, num_ranks,
                                              capacity, topk_idx, expert_counts, expert_offsets,
                                              rank_counts, rank_offsets, rank_token_counts,
                                              dst_row, src_pair, overflow, workspace, hidden,
                                              x_bf16, out_dtype, out, out_scales,
                                              static_cast<hipStream_t>(stream)),
                  fn);
}

int moe_dispatch(int num_tokens, int hidden, int top_k, int num_rows, const void* x_bf16,
                 const int32_t* dst_row, int out_dtype, void* out, void* out_scales,
                 void* stream) {
  const char* fn = "moe_dispatch";
  const int st = check_dispatch(fn, num_tokens, hidden, top_k, num_rows, x_bf16, dst_row,
                                out_dtype, out, out_scales);
  if (st != MOE_OK) return st;
  const bool fp8 = out_dtype == MOE_DTYPE_FP8_E4M3;
  const bool mx = out_dtype == MOE_DTYPE_MXFP8_E4M3;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (fp8)
    err = moe::launch_dispatch_fp8(num_tokens, hidden, top_k, num_rows, x_bf16, dst_row, out,
                                   static_cast<float*>(out_scales), s);
  else if (mx)
    err = moe::launch_dispatch_mxfp8(num_tokens, hidden, top_k, num_rows, x_bf16, dst_row, out,
                                     static_cast<uint8_t*>(out_scales), s);
  else
    err = moe::launch_dispatch_bf16(num_tokens, hidden, top_k, num_rows, x_bf16, dst_row, out, s);
  return from_hip(err, fn);
}

int moe_combine(int num_tokens, int hidden, int top_k, int num_rows, const void* expert_out_bf16,
                const int32_t* dst_row, const float* topk_weights, void* out_bf16,
                void* stream) {
  const char* fn = "moe_combine";
  int st = check_rows(fn, num_tokens, hidden, top_k, num_rows);
  if (st != MOE_OK) return st;
  if (num_tokens > 0 && (!dst_row || !topk_weights || !out_bf16))
    return fail(MOE_ERR_INVALID, "%s: NULL dst_row/topk_weights/out", fn);
  if (num_rows > 0 && !expert_out_bf16) return fail(MOE_ERR_INVALID, "%s: NULL expert_out", fn);
  if (!aligned(expert_out_bf16, 16) || !aligned(out_bf16, 16))
    return fail(MOE_ERR_INVALID, "%s: expert_out and out must be 16-byte aligned", fn);
  if (!aligned(dst_row, 4) || !aligned(topk_weights, 4))
    return fail(MOE_ERR_INVALID, "%s: dst_row/topk_weights must be 4-byte aligned", fn);
  return from_hip(moe::launch_combine(num_tokens, hidden, top_k, num_rows, expert_out_bf16,
                                      dst_row, topk_weights, out_bf16,
                                      static_cast<hipStream_t>(stream)),
                  fn);
}

int moe_dispatch_backward(int num_tokens, int hidden, int top_k, int num_rows,
                          const void* grad_rows_bf16, const int32_t* dst_row,
                          void* grad_x_bf16, void* stream) {
  const char* fn = "moe_dispatch_backward";
  int st = check_rows(fn, num_tokens, hidden, top_k, num_rows);
  if (st != MOE_OK) return st;
  if (num_tokens > 0 && (!dst_row || !grad_x_bf16))
    return fail(MOE_ERR_INVALID, "%s: NULL dst_row/grad_x", fn);
  if (num_rows > 0 && !grad_rows_bf16) return fail(MOE_ERR_INVALID, "%s: NULL grad_rows", fn);
  if (!aligned(grad_rows_bf16, 16) || !aligned(grad_x_bf16, 16))
    return fail(MOE_ERR_INVALID, "%s: grad_rows and grad_x must be 16-byte aligned", fn);
  if (!aligned(dst_row, 4)) return fail(MOE_ERR_INVALID, "%s: dst_row must be 4-byte aligned", fn);
  return from_hip(moe::launch_combine(num_tokens, hidden, top_k, num_rows, grad_rows_bf16,
                                      dst_row, nullptr, grad_x_bf16,
                                      static_cast<hipStream_t>(stream)),
                  fn);
}

int moe_combine_backward(int num_tokens, int hidden, int top_k, int num_rows,
                         const void* grad_out_bf16, const void* expert_out_bf16,
                         const int32_t* dst_row, const float* topk_weights,
                         void* grad_expert_out_bf16, float* grad_weights, void* stream) {
  const char* fn = "moe_combine_backward";
  int st = check_rows(fn, num_tokens, hidden, top_k, num_rows);
  if (st != MOE_OK) return st;
  if (num_tokens > 0 && (!grad_out_bf16 || !dst_row || !topk_weights || !grad_weights))
    return fail(MOE_ERR_INVALID, "%s: NULL grad_out/dst_row/topk_weights/grad_weights", fn);
  if (num_rows > 0 && (!expert_out_bf16 || !grad_expert_out_bf16))
    return fail(MOE_ERR_INVALID, "%s: NULL expert_out/grad_expert_out", fn);
  if (!aligned(grad_out_bf16, 16) || !aligned(expert_out_bf16, 16) ||
      !aligned(grad_expert_out_bf16, 16))
    return fail(MOE_ERR_INVALID, "%s: row buffers must be 16-byte aligned", fn);
  if (!aligned(dst_row, 4) || !aligned(topk_weights, 4) || !aligned(grad_weights, 4))
    return fail(MOE_ERR_INVALID, "%s: index/weight buffers must be 4-byte aligned", fn);
  return from_hip(moe::launch_combine_backward(num_tokens, hidden, top_k, num_rows,
                                               grad_out_bf16, expert_out_bf16, dst_row,
                                               topk_weights, grad_expert_out_bf16, grad_weights,
                                               static_cast<hipStream_t>(stream)),
                  fn);
}

size_t moe_rank_layout_workspace_bytes(int num_tokens, int top_k, int num_ranks) {
  if (num_tokens < 0 || top_k < 1 || top_k > MOE_MAX_TOPK || num_ranks < 1) return 0;
  return moe::rank_layout_workspace_bytes(num_tokens, top_k, num_ranks);
}

}  // extern "C"

namespace {

// Arguments of one (token, rank) layout.
int check_rank_layout(const char* fn, int num_tokens, int num_experts, int top_k,
                      int num_ranks, const int32_t* topk_idx, const int32_t* rank_token_counts,
                      const int32_t* rank_token_offsets, const int32_t* rank_row,
                      const int32_t* send_row, const int32_t* row_token, const void* workspace,
                      size_t workspace_bytes) {
  int st = check_topk(fn, num_tokens, num_experts, top_k);
  if (st != MOE_OK) return st;
  if (num_ranks < 1 || num_ranks > num_experts || num_experts % num_ranks != 0)
    return fail(MOE_ERR_INVALID, "%s: num_ranks=%d must divide num_experts=%d", fn, num_ranks,
                num_experts);
  if (!rank_token_counts || !rank_token_offsets)
    return fail(MOE_ERR_INVALID, "%s: NULL rank_token_counts/rank_token_offsets", fn);
  if (num_tokens > 0 && (!topk_idx || !rank_row || !send_row || !row_token))
    return fail(MOE_ERR_INVALID, "%s: NULL topk_idx/rank_row/send_row/row_token", fn);
  const void* ptrs[] = {topk_idx, rank_token_counts, rank_token_offsets, rank_row, send_row,
                        row_token};
  for (const void* p : ptrs)
    if (!aligned(p, 4)) return fail(MOE_ERR_INVALID, "%s: pointers must be 4-byte aligned", fn);
  const size_t need = moe::rank_layout_workspace_bytes(num_tokens, top_k, num_ranks);
  if (workspace_bytes < need || (need > 0 && !workspace))
    return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace_bytes);
  if (!aligned(workspace, 4)) return fail(MOE_ERR_INVALID, "%s: workspace not aligned", fn);
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_rank_layout(int num_tokens, int num_experts, int top_k, int num_ranks,
                    const int32_t* topk_idx, int32_t* rank_token_counts,
                    int32_t* rank_token_offsets, int32_t* rank_row, int32_t* send_row,
                    int32_t* row_token, void* workspace, size_t workspace_bytes,
                    void* stream) {
  const char* fn = "moe_rank_layout";
  const int st = check_rank_layout(fn, num_tokens, num_experts, top_k, num_ranks, topk_idx,
                                   rank_token_counts, rank_token_offsets, rank_row, send_row,
                                   row_token, workspace, workspace_bytes);
  if (st != MOE_OK) return st;
  return from_hip(moe::launch_rank_layout(num_tokens, num_experts, top_k, num_ranks, topk_idx,
                                          rank_token_counts, rank_token_offsets, rank_row,
                                          send_row, row_token, workspace,
                                          static_cast<hipStream_t>(stream)),
                  fn);
}

int moe_rank_layout_batched(int num_batches, const moe_rank_layout_io* batches, int num_tokens,
                            int num_experts, int top_k, int num_ranks, void* stream) {
  const char* fn = "moe_rank_layout_batched";
  if (num_batches < 1 || num_batches > MOE_MAX_BATCHES || !batches)
    return fail(MOE_ERR_INVALID, "%s: num_batches=%d not in [1, %d] (or NULL batches)", fn,
                num_batches, MOE_MAX_BATCHES);
  moe::RankLayoutBatches rb{};
  for (int b = 0; b < num_batches; ++b) {
    const moe_rank_layout_io& io = batches[b];
    const int st = check_rank_layout(fn, num_tokens, num_experts, top_k, num_ranks, io.topk_idx,
                                     io.rank_token_counts, io.rank_token_offsets, io.rank_row,
                                     io.send_row, io.row_token, io.workspace,
                                     io.workspace_bytes);
    if (st != MOE_OK) return st;
    rb.b[b] = moe::RankLayoutBatch{io.topk_idx, io.rank_token_counts, io.rank_token_offsets,
                                   io.rank_row, io.send_row, io.row_token, io.workspace};
  }
  return from_hip(moe::launch_rank_layout_batches(num_batches, rb, num_tokens, num_experts,
                                                  top_k, num_ranks,
                                                  static_cast<hipStream_t>(stream)),
                  fn);
}

int moe_expand(int num_tokens, int hidden, int top_k, int dtype, int num_rank_rows,
               const void* rank_rows, const void* rank_scales, const int32_t* rank_row,
               const int32_t* row_token, int num_rows, const int32_t* dst_row, void* out,
               void* out_scales, void* stream) {
  const char* fn = "moe_expand";
  int st = check_rows(fn, num_tokens, hidden, top_k, num_rows);
  if (st != MOE_OK) return st;
  if (num_rank_rows < 0) return fail(MOE_ERR_INVALID, "%s: num_rank_rows=%d < 0", fn, num_rank_rows);
  if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_FP8_E4M3 && dtype != MOE_DTYPE_MXFP8_E4M3)
    return fail(MOE_ERR_INVALID, "%s: dtype=%d", fn, dtype);
  const bool fp8 = dtype == MOE_DTYPE_FP8_E4M3;
  const bool mx = dtype == MOE_DTYPE_MXFP8_E4M3;
  if (fp8 && hidden % MOE_FP8_BLOCK != 0)
    return fail(MOE_ERR_INVALID, "%s: FP8 needs hidden %% %d == 0 (hidden=%d)", fn,
                MOE_FP8_BLOCK, hidden);
  if (mx && hidden % MOE_MX_BLOCK != 0)
    return fail(MOE_ERR_INVALID, "%s: MXFP8 needs hidden %% %d == 0 (hidden=%d)", fn,
                MOE_MX_BLOCK, hidden);
  if (num_rows > 0 && !out) return fail(MOE_ERR_INVALID, "%s: NULL out", fn);
  if (num_rows > 0 && num_tokens > 0 && (!rank_row || !dst_row))
    return fail(MOE_ERR_INVALID, "%s: NULL rank_row/dst_row", fn);
  if (num_rank_rows > 0 && num_rows > 0 && !row_token)
    return fail(MOE_ERR_INVALID, "%s: NULL row_token", fn);
  if (num_rank_rows > 0 && num_rows > 0 && !rank_rows)
    return fail(MOE_ERR_INVALID, "%s: NULL rank_rows", fn);
  if ((fp8 || mx) && num_rows > 0 && (!out_scales || (num_rank_rows > 0 && !rank_scales)))
    return fail(MOE_ERR_INVALID, "%s: NULL scales", fn);
  if (!fp8 && !mx && (rank_scales || out_scales))
    return fail(MOE_ERR_INVALID, "%s: scales are for FP8 and MXFP8 only", fn);
  if (!aligned(rank_rows, 16) || !aligned(out, 16))
    return fail(MOE_ERR_INVALID, "%s: rank_rows and out must be 16-byte aligned", fn);
  const bool words = fp8 || (mx && (hidden / MOE_MX_BLOCK) % 4 == 0);
  if (!aligned(rank_row, 4) || !aligned(row_token, 4) || !aligned(dst_row, 4) ||
      (words && (!aligned(rank_scales, 4) || !aligned(out_scales, 4))))
    return fail(MOE_ERR_INVALID, "%s: index and scale buffers must be 4-byte aligned", fn);
  return from_hip(moe::launch_expand(num_tokens, hidden, top_k, dtype, num_rank_rows, rank_rows,
                                     rank_scales, rank_row, row_token, num_rows, dst_row, out,
                                     out_scales, static_cast<hipStream_t>(stream)),
                  fn);
}

int moe_combine_local(int num_tokens, int hidden, int top_k, int num_rows,
                      const void* expert_out_bf16, const int32_t* dst_row,
                      const int32_t* rank_row, const int32_t* row_token,
                      const float* topk_weights, int num_rank_rows, void* partial_bf16,
                      void* stream) {
  const char* fn = "moe_combine_local";
  int st = check_rows(fn, num_tokens, hidden, top_k, num_rows);
  if (st != MOE_OK) return st;
  if (num_rank_rows < 0) return fail(MOE_ERR_INVALID, "%s: num_rank_rows=%d < 0", fn, num_rank_rows);
  if (num_tokens > 0 && (!dst_row || !rank_row || !topk_weights))
    return fail(MOE_ERR_INVALID, "%s: NULL dst_row/rank_row/topk_weights", fn);
  if (num_rank_rows > 0 && !row_token) return fail(MOE_ERR_INVALID, "%s: NULL row_token", fn);
  if (num_rows > 0 && !expert_out_bf16) return fail(MOE_ERR_INVALID, "%s: NULL expert_out", fn);
  if (num_rank_rows > 0 && !partial_bf16) return fail(MOE_ERR_INVALID, "%s: NULL partial", fn);
  if (!aligned(expert_out_bf16, 16) || !aligned(partial_bf16, 16))
    return fail(MOE_ERR_INVALID, "%s: expert_out and partial must be 16-byte aligned", fn);
  if (!aligned(dst_row, 4) || !aligned(rank_row, 4) || !aligned(row_token, 4) ||
      !aligned(topk_weights, 4))
    return fail(MOE_ERR_INVALID, "%s: index/weight buffers must be 4-byte aligned", fn);
  return from_hip(moe::launch_combine_local(num_tokens, hidden, top_k, num_rows, num_rank_rows,
                                            expert_out_bf16, dst_row, rank_row, row_token,
                                            topk_weights, partial_bf16,
                                            static_cast<hipStream_t>(stream)),
                  fn);
}

int moe_combine_partials(int num_tokens, int hidden, int top_k, int num_rank_rows,
                         const void* partial_bf16, const int32_t* send_row, void* out_bf16,
                         void* stream) {
  const char* fn = "moe_combine_partials";
  int st = check_rows(fn, num_tokens, hidden, top_k, num_rank_rows);
  if (st != MOE_OK) return st;
  if (num_tokens > 0 && (!send_row || !out_bf16))
    return fail(MOE_ERR_INVALID, "%s: NULL send_row/out", fn);
  if (num_rank_rows > 0 && !partial_bf16) return fail(MOE_ERR_INVALID, "%s: NULL partial", fn);
  if (!aligned(partial_bf16, 16) || !aligned(out_bf16, 16))
    return fail(MOE_ERR_INVALID, "%s: partial and out must be 16-byte aligned", fn);
  if (!aligned(send_row, 4)) return fail(MOE_ERR_INVALID, "%s: send_row must be 4-byte aligned", fn);
  // the per-item combine kernel: in the hierarchical pass on the DeepSeek-V3
  // shape the held-output kernel made the partial sum 1.1 us slower and the
  // pass 1% slower (same-box runs). Items of 1 KiB at k = 8: 73.2-75.2 us
  // against 74.6-77.0 with 2 KiB items (20 back-to-back launches, same box).
  return from_hip(moe::launch_combine(num_tokens, hidden, top_k, num_rank_rows, partial_bf16,
                                      send_row, nullptr, out_bf16,
                                      static_cast<hipStream_t>(stream), false, true),
                  fn);
}

}  // extern "C"
