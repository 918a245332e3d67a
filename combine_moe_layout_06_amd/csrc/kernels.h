// Internal launch functions of the HIP kernels. Each assumes its arguments
// were validated by the C-ABI layer (moe_api.hip) and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// Several independent batches of the same sizes in one launch: the grid's
// y dimension is the batch, and the per-batch pointers travel in the kernel
// arguments.
constexpr int kMaxBatches = MOE_MAX_BATCHES;

struct RouteBatches {
  const float* logits[kMaxBatches];
  const float* bias[kMaxBatches];   // entries may be null
  int32_t* idx[kMaxBatches];
  float* w[kMaxBatches];
};

hipError_t launch_route(int T, int E, int k, const float* logits, const float* bias,
                        int sigmoid, int G, int kg, int32_t* idx_out, float* w_out,
                        hipStream_t stream);
hipError_t launch_route_batches(int nb, const RouteBatches& rb, int T, int E, int k,
                                int sigmoid, int G, int kg, hipStream_t stream);

// Layout: pairs are cut into tiles of whole tokens; one block per tile.
int layout_tile_tokens(int k);
int layout_num_tiles(int T, int k);
size_t layout_workspace_bytes(int T, int E, int k);

hipError_t launch_layout(int T, int E, int k, int R, int cap, const int32_t* idx,
                         int32_t* expert_counts, int32_t* expert_offsets,
                         int32_t* rank_counts, int32_t* rank_offsets,
                         int32_t* rank_token_counts, int32_t* dst_row,
                         int32_t* src_pair, int32_t* overflow, void* workspace,
                         hipStream_t stream);

// Per-batch pointers of a batched layout (the arguments of launch_layout).
struct LayoutBatch {
  const int32_t* idx;
  int32_t* expert_counts;
  int32_t* expert_offsets;
  int32_t* rank_counts;
  int32_t* rank_offsets;
  int32_t* rank_token_counts;   // may be null
  int32_t* dst_row;
  int32_t* src_pair;
  int32_t* overflow;
  void* workspace;
};
struct LayoutBatches {
  LayoutBatch b[kMaxBatches];
};
hipError_t launch_layout_batches(int nb, const LayoutBatches& lb, int T, int E, int k, int R,
                                 int cap, hipStream_t stream);

// Layout followed by dispatch; one launch when all pairs fit one tile in
// capacity mode (layout_dispatch_fused), else the two launches above.
bool layout_dispatch_fused(int T, int k, int cap);
hipError_t launch_layout_dispatch(int T, int E, int k, int R, int cap, const int32_t* idx,
                                  int32_t* expert_counts, int32_t* expert_offsets,
                                  int32_t* rank_counts, int32_t* rank_offsets,
                                  int32_t* rank_token_counts, int32_t* dst_row,
                                  int32_t* src_pair, int32_t* overflow, void* workspace,
                                  int H, const void* x, int dtype, void* out, void* out_scales,
                                  hipStream_t stream);

// (token, rank) rows of the deduplicated dispatch.
size_t rank_layout_workspace_bytes(int T, int k, int R);
hipError_t launch_rank_layout(int T, int E, int k, int R, const int32_t* idx,
                              int32_t* counts, int32_t* offsets, int32_t* rank_row,
                              int32_t* send_row, int32_t* row_token, void* workspace,
                              hipStream_t stream);
// Several (token, rank) layouts of the same shape in one set of launches:
// batch b on grid row b.
struct RankLayoutBatch {
  const int32_t* idx;
  int32_t* counts;
  int32_t* offsets;
  int32_t* rank_row;
  int32_t* send_row;
  int32_t* row_token;
  void* workspace;
};
struct RankLayoutBatches {
  RankLayoutBatch b[kMaxBatches];
};
hipError_t launch_rank_layout_batches(int nb, const RankLayoutBatches& rb, int T, int E, int k,
                                      int R, hipStream_t stream);

hipError_t launch_dispatch_bf16(int T, int H, int k, int num_rows, const void* x,
                                const int32_t* dst_row, void* out, hipStream_t stream);

hipError_t launch_dispatch_fp8(int T, int H, int k, int num_rows, const void* x,
                               const int32_t* dst_row, void* out, float* out_scales,
                               hipStream_t stream);

hipError_t launch_dispatch_mxfp8(int T, int H, int k, int num_rows, const void* x,
                                 const int32_t* dst_row, void* out, uint8_t* out_scales,
                                 hipStream_t stream);

// w == nullptr means unit weights (the gradient of dispatch). allow_held:
// the held-output kernel may serve the shapes it is chosen for. fine_items:
// the per-item kernel at k = 8 takes items of 1 KiB (one 16-byte chunk per
// lane), as many parts as a row has.
hipError_t launch_combine(int T, int H, int k, int num_rows, const void* y,
                          const int32_t* dst_row, const float* w, void* out,
                          hipStream_t stream, bool allow_held = true,
                          bool fine_items = false);

// Fan-out of the (token, rank) rows to the expert rows, and the per-rank
// partial combine.
hipError_t launch_expand(int T, int H, int k, int dtype, int num_rank_rows, const void* src,
                         const void* src_scales, const int32_t* rank_row,
                         const int32_t* row_token, int num_rows, const int32_t* dst_row,
                         void* out, void* out_scales, hipStream_t stream);
hipError_t launch_combine_local(int T, int H, int k, int num_rows, int num_rank_rows,
                                const void* y, const int32_t* dst_row, const int32_t* rank_row,
                                const int32_t* row_token, const float* w, void* partial,
                                hipStream_t stream);

hipError_t launch_combine_backward(int T, int H, int k, int num_rows, const void* dout,
                                   const void* y, const int32_t* dst_row, const float* w,
                                   void* dy, float* dw, hipStream_t stream);

// Number of waves a row-parallel kernel aims for: several times what the
// 256 CUs hold at once (8 to 32 waves each, by kernel), so that short waves
// keep every CU busy to the end.
#ifndef MOE_TARGET_WAVES
#define MOE_TARGET_WAVES 32768
#endif
constexpr int kTargetWaves = MOE_TARGET_WAVES;

// Occupancy caps. A streaming kernel that fills each CU with as many waves as
// its registers allow can keep far more HBM requests in flight than the
// memory needs, and then runs slower: the extra queued reads and writes
// turn the bus around more often. A launch caps its workgroups per CU by
// reserving dynamic LDS that the kernel never touches (gfx950: 160 KiB of
// LDS per CU). Dynamic LDS bytes that leave room for at most `blocks`
// workgroups on a CU; 0 = no cap.
constexpr int kLdsPerCu = 160 * 1024;
inline size_t lds_cap_bytes(int blocks) {
  return blocks > 0 ? (size_t)(kLdsPerCu / (blocks + 1) + 1024) : 0;
}

}  // namespace moe
