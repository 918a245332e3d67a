/*
 * moe.h -- C ABI of the MoE expert-parallel hot path on one AMD Instinct
 * MI355X (gfx950): routing, layout, dispatch and combine.
 *
 * Sources. The operations are the ones described by four web pages on MoE
 * expert parallelism:
 *   - glossary page "Expert Parallelism (Parallélisme d'experts)"
 *     (polydesk.ai): section "Le principe de base" (each GPU owns whole
 *     experts; 8 experts over 4 GPUs gives 2 per GPU) and section "Le pattern
 *     de communication all-to-all" (Phase 1 dispatch, Phase 2 combine
 *     weighted by the router scores), sections "Megatron-LM (NVIDIA)" and
 *     "Défis et optimisations" (capacity factor, token dropping);
 *   - article "DeepEP de DeepSeek : la lib open source qui optimise la
 *     communication GPU pour les modèles MoE à l'échelle" (ai-master.dev):
 *     sections "Kernels low-latency dispatch et combine", "Support FP8 et
 *     MXFP8", "Group-limited gating algorithm", "Configuration type";
 *   - the hyper.ai story on NVIDIA Hybrid-EP: top-k routing, the dispatch and
 *     combine operators, native FP8/BF16, and buffers preallocated at a
 *     maximum size so that no size synchronisation is needed.
 * The destination GPUs ("ranks") of those pages are modelled here as
 * consecutive regions of one buffer in one GPU's HBM: rank r owns experts
 * [r*E/R, (r+1)*E/R) and its region is the rows of those experts.
 *
 * Conventions shared by every entry point:
 *   - Every array argument is a DEVICE pointer owned by the caller. The
 *     library never allocates, frees or synchronises, and keeps no state.
 *   - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued
 *     on it and the call returns without waiting.
 *   - Arguments are validated on the host BEFORE anything is enqueued: on a
 *     bad argument the call returns MOE_ERR_INVALID (or MOE_ERR_UNSUPPORTED
 *     / MOE_ERR_WORKSPACE) and touches nothing. A failed launch returns
 *     MOE_ERR_HIP. moe_last_error() describes the last failure of the
 *     calling thread.
 *   - Device-side contents are not validated. Kernels ignore an expert id
 *     outside [0, E) (treated like the mask value -1) and a row index
 *     outside [0, num_rows) (the pair is skipped), so that bad routing data
 *     can produce wrong results but never an out-of-bounds access.
 *     NaN and Inf inputs give unspecified results.
 *   - Outputs must not overlap inputs. Calls are re-entrant.
 *   - bf16 data is passed as raw 16-bit patterns; rows are contiguous with
 *     `hidden` elements each and must start 16-byte aligned.
 */
#ifndef MOE_LAYOUT_MOE_H
#define MOE_LAYOUT_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = 1,      /* bad scalar or pointer argument          */
  MOE_ERR_UNSUPPORTED = 2,  /* valid, but outside the built kernels    */
  MOE_ERR_WORKSPACE = 3,    /* workspace missing or too small          */
  MOE_ERR_HIP = 4           /* a HIP call or kernel launch failed      */
} moe_status;

enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 };
enum { MOE_DTYPE_BF16 = 0, MOE_DTYPE_FP8_E4M3 = 1, MOE_DTYPE_MXFP8_E4M3 = 2 };

#define MOE_MAX_EXPERTS 512
#define MOE_MAX_TOPK 32
#define MOE_MAX_GROUPS 64
#define MOE_MAX_BATCHES 8
#define MOE_FP8_BLOCK 128
#define MOE_MX_BLOCK 32

/* Name of a status code ("MOE_OK", ...). Never NULL. */
const char* moe_status_string(int status);

/* Text of the last failure seen by the calling thread ("" if none). */
const char* moe_last_error(void);

/*
 * moe_route -- pick k of E experts per token and their weights.
 *
 * Top-k routing: each token activates only k experts (hyper.ai story on
 * Hybrid-EP). With num_groups > 1 the choice is group-limited (DeepEP
 * article, section "Group-limited gating algorithm"): the E experts form
 * num_groups contiguous groups, each group is scored by the sum of its two
 * largest selection keys, the topk_groups best groups are kept, and the k
 * experts are chosen among the kept groups only.
 *
 *   score_fn  MOE_SCORE_SOFTMAX: s_e = l_e; weights are the softmax of the
 *             selected logits, w_j = exp(l_j) / sum_i exp(l_i).
 *             MOE_SCORE_SIGMOID: s_e = 1/(1+exp(-l_e)) (evaluated in fp64,
 *             rounded to fp32); weights w_j = s_j / sum_i s_i.
 *   key_e   = s_e + bias_e (fp32 add; bias may be NULL). The bias moves the
 *             selection only, never the weights.
 *   Order   : slot j holds the expert with the j-th largest key; equal keys
 *             go to the lower expert index. Weight sums run in fp64 and each
 *             weight is rounded once to fp32.
 *
 *   logits        [num_tokens, num_experts] fp32, row-major
 *   bias          [num_experts] fp32 or NULL
 *   topk_idx      [num_tokens, top_k] int32 output
 *   topk_weights  [num_tokens, top_k] fp32 output
 *
 * Requires 0 <= num_tokens, 1 <= top_k <= min(num_experts, MOE_MAX_TOPK),
 * num_experts <= MOE_MAX_EXPERTS; softmax needs num_groups == 1; with
 * groups: num_experts % num_groups == 0, num_groups <= MOE_MAX_GROUPS,
 * 1 <= topk_groups <= num_groups and top_k <= topk_groups * (E/num_groups).
 */
int moe_route(int num_tokens, int num_experts, int top_k,
              const float* logits, const float* bias,
              int score_fn, int num_groups, int topk_groups,
              int32_t* topk_idx, float* topk_weights, void* stream);

/*
 * moe_route_batched -- moe_route on num_batches independent batches of the
 * same sizes (each batch has its own logits, bias and outputs; the routing
 * settings are shared), in one launch instead of num_batches: the
 * batches are, for example, the micro-batches or consecutive steps whose
 * routing a caller prepares ahead of their dispatch. Each batch's results
 * equal those of moe_route on it alone (same definition: hyper.ai story on
 * Hybrid-EP for top-k routing, DeepEP article "Group-limited gating
 * algorithm" for the groups).
 *
 *   batches   HOST array of num_batches moe_route_io, read during the call
 *             only; 1 <= num_batches <= MOE_MAX_BATCHES
 * Every batch is validated as moe_route validates its arguments before
 * anything is enqueued. No output of one batch may overlap another batch's
 * inputs or outputs.
 */
typedef struct {
  const float* logits;   /* [num_tokens, num_experts] fp32 */
  const float* bias;     /* [num_experts] fp32 or NULL */
  int32_t* topk_idx;     /* [num_tokens, top_k] int32 output */
  float* topk_weights;   /* [num_tokens, top_k] fp32 output */
} moe_route_io;

int moe_route_batched(int num_batches, const moe_route_io* batches,
                      int num_tokens, int num_experts, int top_k,
                      int score_fn, int num_groups, int topk_groups,
                      void* stream);

/* Bytes of device workspace moe_layout needs for these sizes. */
size_t moe_layout_workspace_bytes(int num_tokens, int num_experts, int top_k);

/*
 * moe_layout -- counts, prefix-sum offsets and the stable destination row of
 * every (token, slot) pair (glossary "Expert Parallelism", "Le principe de
 * base" for the placement and Phase 1 for the dispatch it prepares).
 *
 * Packed mode (capacity == 0): the dispatch buffer has T*k rows, a size the
 * caller knows without reading anything back (hyper.ai story on Hybrid-EP,
 * preallocated buffers).
 *   expert_counts[e]   pairs routed to e (mask value -1 is skipped)
 *   expert_offsets[e]  sum of counts of experts < e; [E] = live pairs
 *   dst_row[t,j]       expert_offsets[e] + number of earlier pairs of e in
 *                      row-major (t, j) order (stable); -1 if masked
 * Capacity mode (capacity > 0; glossary "Megatron-LM (NVIDIA)", capacity
 * factor and token dropping): the buffer has E*capacity rows and the pair
 * with stable position p in expert e goes to row e*capacity + p when
 * p < capacity, else it is dropped (dst_row = -1).
 *   expert_counts[e]   raw demand (dropped pairs included)
 *   expert_offsets[e]  e*capacity
 *   overflow[0]        number of dropped pairs
 * Both modes:
 *   rank_counts[r]       rows written into rank r's region
 *   rank_offsets[r]      first row of rank r's region; [R] = end
 *   rank_token_counts[r] distinct tokens with >= 1 unmasked expert on rank r
 *                        (may be NULL)
 *   src_pair[row]        t*k + j of the pair stored in `row`, -1 if none
 *
 *   topk_idx   [num_tokens, top_k] int32, values in [0, E) or -1
 *   sizes: expert_counts [E], expert_offsets [E+1], rank_counts [R],
 *          rank_offsets [R+1], rank_token_counts [R], dst_row [T, k],
 *          src_pair [T*k] (packed) or [E*capacity], overflow [1]
 *   workspace  device scratch of at least moe_layout_workspace_bytes();
 *              it needs no initialisation and is overwritten (per-tile
 *              counts, for many tiles rewritten in place as per-tile bases),
 *              so calls that may overlap must not share one
 *
 * Placement uses no atomics on global memory: results are deterministic.
 * Requires num_experts % num_ranks == 0 and the limits of moe_route.
 */
int moe_layout(int num_tokens, int num_experts, int top_k, int num_ranks,
               int capacity, const int32_t* topk_idx,
               int32_t* expert_counts, int32_t* expert_offsets,
               int32_t* rank_counts, int32_t* rank_offsets,
               int32_t* rank_token_counts, int32_t* dst_row,
               int32_t* src_pair, int32_t* overflow,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_layout_batched -- moe_layout on num_batches independent batches of
 * the same sizes (each with its own routing, outputs and workspace), with
 * one launch per pass for all of them instead of one per batch and pass.
 * Each batch's results equal those of moe_layout on it alone (same
 * definitions: glossary "Expert Parallelism", "Le principe de base" and
 * "Megatron-LM (NVIDIA)"). Sizes that need the scan pass (many tiles) run
 * the batches one after the other.
 *
 *   batches   HOST array of num_batches moe_layout_io, read during the call
 *             only; 1 <= num_batches <= MOE_MAX_BATCHES; rank_token_counts
 *             must be given for every batch or for none
 * Every batch is validated as moe_layout validates its arguments before
 * anything is enqueued. Batches must not share outputs or workspaces.
 */
typedef struct {
  const int32_t* topk_idx;      /* the arrays of moe_layout, per batch */
  int32_t* expert_counts;
  int32_t* expert_offsets;
  int32_t* rank_counts;
  int32_t* rank_offsets;
  int32_t* rank_token_counts;   /* may be NULL */
  int32_t* dst_row;
  int32_t* src_pair;
  int32_t* overflow;
  void* workspace;
  size_t workspace_bytes;
} moe_layout_io;

int moe_layout_batched(int num_batches, const moe_layout_io* batches,
                       int num_tokens, int num_experts, int top_k,
                       int num_ranks, int capacity, void* stream);

/*
 * moe_layout_no_alloc -- moe_layout without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments
 * (minus workspace and workspace_bytes), same results, same kernels.
 *
 * The per-tile counts live instead in a static device array of
 * MOE_LAYOUT_SCRATCH_BYTES bytes that belongs to the library: each GPU the
 * library runs on holds its own copy from its first call on that GPU until
 * the process ends (the one exception to "keeps no state" above). The call
 * allocates and frees nothing; the first call on a device looks up that
 * device's copy once (hipGetSymbolAddress) with the device current.
 *   - Sizes whose moe_layout_workspace_bytes() exceeds
 *     MOE_LAYOUT_SCRATCH_BYTES return MOE_ERR_WORKSPACE and enqueue nothing
 *     (2 MiB covers up to 130,944 tokens at E = 256, k = 8).
 *   - The array needs no initialisation: every call writes the parts it
 *     reads. It keeps the last call's contents.
 *   - Every call on one GPU shares that GPU's array: calls that may overlap
 *     on one GPU (other streams, other threads) race and must be ordered by
 *     the caller. The stream must belong to the calling thread's current
 *     device.
 */
#define MOE_LAYOUT_SCRATCH_BYTES (2u << 20)
int moe_layout_no_alloc(int num_tokens, int num_experts, int top_k, int num_ranks,
                        int capacity, const int32_t* topk_idx,
                        int32_t* expert_counts, int32_t* expert_offsets,
                        int32_t* rank_counts, int32_t* rank_offsets,
                        int32_t* rank_token_counts, int32_t* dst_row,
                        int32_t* src_pair, int32_t* overflow, void* stream);

/*
 * moe_dispatch -- copy each token's hidden state to the rows of its
 * experts (glossary "Expert Parallelism", Phase 1; DeepEP article,
 * "Kernels low-latency dispatch et combine").
 *
 * MOE_DTYPE_BF16:     out[dst_row[t,j], :] = x[t, :]   (bit copy)
 * MOE_DTYPE_FP8_E4M3: x is quantised once per token and copied to every
 *   row of the token (DeepEP article, "Support FP8 et MXFP8": FP8 halves
 *   the BF16 bytes; "Configuration type": quantisation inside the call).
 *   For each 128-column block b of token t:
 *     a = max |x|, scale = fp32(a/448), inv = fp32(448/a),
 *     q = e4m3fn(fp32(x*inv)) rounded to nearest even, saturating at
 *     +-448; an input of +-0 gives the code of +-0.
 *   out holds the 1-byte OCP e4m3fn codes [num_rows, hidden];
 *   out_scales[row, b] = scale, fp32 [num_rows, hidden/128].
 * MOE_DTYPE_MXFP8_E4M3: microscaled FP8 (the DeepEP article's "Support FP8
 *   et MXFP8" names MXFP8; block and scale layout follow the OCP
 *   microscaling format). Per 32-column block b:
 *     e = floor(log2(max |x|)) - 8 clamped to [-127, 127] (-127 if all 0),
 *     q = e4m3fn(x / 2^e) rounded to nearest even, saturating at +-448.
 *   out holds the codes [num_rows, hidden]; out_scales holds the E8M0
 *   bytes e + 127, uint8 [num_rows, hidden/32].
 *
 *   x          [num_tokens, hidden] bf16
 *   dst_row    [num_tokens, top_k] int32 from moe_layout (-1 = no row)
 *   num_rows   rows of `out` (T*k packed, E*capacity padded)
 *   out_scales fp32 (FP8), uint8 (MXFP8) or NULL (bf16)
 * Rows that receive no pair are left untouched.
 * Requires hidden % 8 == 0 (16-byte rows); FP8 also hidden % 128 == 0,
 * MXFP8 hidden % 32 == 0.
 */
int moe_dispatch(int num_tokens, int hidden, int top_k, int num_rows,
                 const void* x_bf16, const int32_t* dst_row, int out_dtype,
                 void* out, void* out_scales, void* stream);

/*
 * moe_layout_dispatch -- moe_layout followed by moe_dispatch, with the same
 * arguments and the same results (num_rows = E*capacity, or T*k packed).
 * For decode-sized inputs in capacity mode (capacity > 0 and T*k <= 1024)
 * it is ONE launch: the layout blocks and the dispatch blocks run side by
 * side, the dispatch waves computing their token's rows from topk_idx by the
 * layout's own definition (row e*cap + number of earlier pairs of expert e,
 * dropped at cap) instead of waiting for dst_row. This is the low-latency
 * path of the DeepEP article ("Kernels low-latency dispatch et combine":
 * kernels that fuse the steps of the exchange) on buffers preallocated at
 * their maximum size (hyper.ai story on Hybrid-EP). Otherwise it runs the
 * layout launches, then the dispatch.
 *
 *   layout arguments:   as moe_layout
 *   hidden, x_bf16, out_dtype, out, out_scales:   as moe_dispatch
 * Errors: those of moe_layout and moe_dispatch, checked before anything is
 * enqueued.
 */
/* 1 when moe_layout_dispatch takes one launch for these sizes, else 0. */
int moe_layout_dispatch_is_fused(int num_tokens, int top_k, int capacity);

int moe_layout_dispatch(int num_tokens, int num_experts, int top_k, int num_ranks,
                        int capacity, const int32_t* topk_idx,
                        int32_t* expert_counts, int32_t* expert_offsets,
                        int32_t* rank_counts, int32_t* rank_offsets,
                        int32_t* rank_token_counts, int32_t* dst_row,
                        int32_t* src_pair, int32_t* overflow,
                        void* workspace, size_t workspace_bytes,
                        int hidden, const void* x_bf16, int out_dtype,
                        void* out, void* out_scales, void* stream);

/*
 * moe_combine -- bring each token's k expert outputs back and sum them
 * weighted by the router scores (glossary "Expert Parallelism", Phase 2).
 *
 *   out[t, :] = bf16( sum_j w[t,j] * y[dst_row[t,j], :] )
 *
 * The sum runs over the pairs with a row (dropped pairs add nothing, the
 * weights are not renormalised), in slot order j = 0..k-1, as a chain of
 * fp32 fused multiply-adds, rounded once to bf16 (nearest even).
 *
 *   expert_out  [num_rows, hidden] bf16
 *   dst_row     [num_tokens, top_k] int32
 *   topk_weights [num_tokens, top_k] fp32
 *   out         [num_tokens, hidden] bf16
 * Requires hidden % 8 == 0.
 */
int moe_combine(int num_tokens, int hidden, int top_k, int num_rows,
                const void* expert_out_bf16, const int32_t* dst_row,
                const float* topk_weights, void* out_bf16, void* stream);

/*
 * moe_dispatch_backward -- gradient of dispatch with respect to x. The
 * exchanges run in the backward pass too (DeepEP article, "Qu'est-ce que
 * l'Expert Parallelism": every forward and backward pass needs the
 * all-to-all). Each token collects the gradients of its rows:
 *
 *   grad_x[t, :] = bf16( sum over j with a row of grad_rows[dst_row[t,j], :] )
 *
 * summed in fp32 in slot order (moe_combine with unit weights).
 *   grad_rows  [num_rows, hidden] bf16;  grad_x [num_tokens, hidden] bf16
 * Requires hidden % 8 == 0.
 */
int moe_dispatch_backward(int num_tokens, int hidden, int top_k, int num_rows,
                          const void* grad_rows_bf16, const int32_t* dst_row,
                          void* grad_x_bf16, void* stream);

/*
 * moe_combine_backward -- gradients of moe_combine (same passage as
 * moe_dispatch_backward). For every pair (t, j) with a row d = dst_row[t,j]:
 *
 *   grad_expert_out[d, :] = bf16( topk_weights[t,j] * grad_out[t, :] )
 *   grad_weights[t, j]    = sum_h grad_out[t, h] * expert_out[d, h]   (fp32)
 *
 * Pairs without a row get grad_weights = 0 and write no row; rows of
 * grad_expert_out that no pair addresses are left untouched. The dot
 * products are summed in a fixed order (deterministic).
 *   grad_out [num_tokens, hidden] bf16; expert_out, grad_expert_out
 *   [num_rows, hidden] bf16; grad_weights [num_tokens, top_k] fp32
 * Requires hidden % 8 == 0.
 */
int moe_combine_backward(int num_tokens, int hidden, int top_k, int num_rows,
                         const void* grad_out_bf16, const void* expert_out_bf16,
                         const int32_t* dst_row, const float* topk_weights,
                         void* grad_expert_out_bf16, float* grad_weights, void* stream);

/*
 * ---------------------------------------------------------------------------
 * Deduplicated dispatch and hierarchical combine. The hyper.ai story on
 * NVIDIA Hybrid-EP describes a combine that reduces hierarchically: first
 * the results inside one destination, then across destinations. Here a
 * destination is a rank (rank r owns experts [r*E/R, (r+1)*E/R); glossary
 * "Expert Parallelism", "Le principe de base"). A token sends ONE row to
 * each rank that holds at least one of its experts, however many of its
 * experts live there; the rank fans the row out to its expert rows; after
 * the experts it reduces the token's weighted outputs into one partial row;
 * only the partial rows travel back, and each token sums its partials.
 *
 *   moe_rank_layout     (token, rank) rows: counts, offsets, maps
 *   moe_dispatch        with dst_row = send_row and num_rows = T*min(k,R):
 *                       one copy (bf16, FP8 or MXFP8) per (token, rank)
 *   moe_expand          (token, rank) rows -> expert rows (rows of moe_layout)
 *   ...experts...
 *   moe_combine_local   expert rows -> one bf16 partial row per (token, rank)
 *   moe_combine_partials  partial rows -> out[t]
 *
 * The result differs from moe_combine by the extra bf16 rounding of each
 * partial (the partial travels as a bf16 row).
 * ---------------------------------------------------------------------------
 */

/* Workspace bytes moe_rank_layout needs for these sizes (0 on bad sizes). */
size_t moe_rank_layout_workspace_bytes(int num_tokens, int top_k, int num_ranks);

/*
 * moe_rank_layout -- rows of the (token, rank) buffer, one per token and
 * rank holding at least one of the token's unmasked experts (capacity plays
 * no part: the row exists by demand). Rank r's rows are
 * [rank_token_offsets[r], rank_token_offsets[r+1]), in token order. The
 * buffer is sized for its maximum, num_rank_rows = T * min(k, R), so that no
 * count is read back before the dispatch (hyper.ai story on Hybrid-EP,
 * preallocated buffers).
 *
 *   topk_idx           [T, k] int32; ids outside [0, E) are masked slots
 *   rank_token_counts  [R]    int32 out: rows of rank r (its distinct tokens)
 *   rank_token_offsets [R+1]  int32 out: exclusive prefix sum, [R] = total
 *   rank_row           [T, k] int32 out: the (t, rank of slot j) row, for
 *                      every unmasked slot; -1 for masked slots
 *   send_row           [T, k] int32 out: rank_row at the token's first slot
 *                      (in slot order) on each rank, -1 elsewhere: the
 *                      destination map of the deduplicated moe_dispatch and
 *                      the source map of moe_combine_partials
 *   row_token          [T*min(k,R)] int32 out: token of each row, -1 past
 *                      the last row
 * Requires R to divide E. Deterministic; two launches (one when all T*k
 * pairs fit in one tile of 1024 pairs, three for many tiles). The workspace
 * needs no initialisation and is overwritten, so calls that may overlap must
 * not share one.
 */
int moe_rank_layout(int num_tokens, int num_experts, int top_k, int num_ranks,
                    const int32_t* topk_idx, int32_t* rank_token_counts,
                    int32_t* rank_token_offsets, int32_t* rank_row, int32_t* send_row,
                    int32_t* row_token, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * moe_rank_layout_batched -- moe_rank_layout on num_batches independent
 * batches of the same sizes (each with its own routing, outputs and
 * workspace), with one launch per pass for all of them. Each batch's results
 * equal those of moe_rank_layout on it alone (hyper.ai story on Hybrid-EP,
 * preallocated buffers). Sizes that need the scan pass (hundreds of tiles)
 * run one scan launch per batch.
 *
 *   batches   HOST array of num_batches moe_rank_layout_io, read during the
 *             call only; 1 <= num_batches <= MOE_MAX_BATCHES
 * Every batch is validated as moe_rank_layout validates its arguments
 * before anything is enqueued. Batches must not share outputs or
 * workspaces.
 */
typedef struct {
  const int32_t* topk_idx;      /* the arrays of moe_rank_layout, per batch */
  int32_t* rank_token_counts;
  int32_t* rank_token_offsets;
  int32_t* rank_row;
  int32_t* send_row;
  int32_t* row_token;
  void* workspace;
  size_t workspace_bytes;
} moe_rank_layout_io;

int moe_rank_layout_batched(int num_batches, const moe_rank_layout_io* batches,
                            int num_tokens, int num_experts, int top_k,
                            int num_ranks, void* stream);

/*
 * moe_expand -- on the receiving rank, copy each (token, rank) row to the
 * expert rows of that token on the rank: for every row s with
 * t = row_token[s] >= 0 and every slot j of t with rank_row[t,j] = s,
 *
 *   out[dst_row[t,j]] = rank_rows[s]          when 0 <= dst_row[t,j] < num_rows
 *
 * (payload and, for FP8 / MXFP8, the scales; a byte copy). After the
 * deduplicated dispatch this gives exactly the rows moe_dispatch writes with
 * dst_row. Expert rows that no slot reaches are left untouched. The rows are
 * visited in their own order, each read once, as the receiving rank would
 * walk what it received.
 *   dtype         MOE_DTYPE_* of the rows
 *   rank_rows     [num_rank_rows, hidden] bf16 or e4m3 codes
 *   rank_scales   FP8: fp32 [num_rank_rows, hidden/128]; MXFP8: uint8
 *                 [num_rank_rows, hidden/32]; bf16: NULL
 *   rank_row      [T, k] and row_token [num_rank_rows], both from the same
 *                 moe_rank_layout call
 *   dst_row       [T, k] from moe_layout (-1 = dropped)
 *   out, out_scales  [num_rows, ...] in the same formats
 */
int moe_expand(int num_tokens, int hidden, int top_k, int dtype, int num_rank_rows,
               const void* rank_rows, const void* rank_scales, const int32_t* rank_row,
               const int32_t* row_token, int num_rows, const int32_t* dst_row, void* out,
               void* out_scales, void* stream);

/*
 * moe_combine_local -- first level of the hierarchical combine: for each
 * (token, rank) row s,
 *
 *   partial[s, :] = bf16( sum over the token's slots j with rank_row[t,j] = s
 *                         and a kept expert row of w[t,j] * y[dst_row[t,j], :] )
 *
 * in fp32 fused multiply-adds, slot order inside the row, one rounding to
 * bf16 (nearest even), where t = row_token[s]. A row whose pairs were all
 * dropped by capacity is written as +0. Rows whose row_token is -1 (past
 * the last row) are left untouched. The rows are visited in their own
 * order, each rank's rows one after the other, as the receiving rank would
 * reduce them.
 *   expert_out [num_rows, hidden] bf16;  dst_row [T, k] from moe_layout
 *   rank_row   [T, k] and row_token [num_rank_rows], both from the same
 *              moe_rank_layout call;  topk_weights [T, k] fp32
 *   partial    [num_rank_rows, hidden] bf16
 * Requires hidden % 8 == 0.
 */
int moe_combine_local(int num_tokens, int hidden, int top_k, int num_rows,
                      const void* expert_out_bf16, const int32_t* dst_row,
                      const int32_t* rank_row, const int32_t* row_token,
                      const float* topk_weights, int num_rank_rows, void* partial_bf16,
                      void* stream);

/*
 * moe_combine_partials -- second level: each token sums its partial rows,
 *
 *   out[t, :] = bf16( sum over j with send_row[t,j] >= 0 of partial[send_row[t,j], :] )
 *
 * fp32 sum in slot order, one rounding to bf16. A token with no row gets +0.
 *   partial [num_rank_rows, hidden] bf16;  send_row [T, k] from moe_rank_layout
 *   out     [num_tokens, hidden] bf16
 * Requires hidden % 8 == 0.
 */
int moe_combine_partials(int num_tokens, int hidden, int top_k, int num_rank_rows,
                         const void* partial_bf16, const int32_t* send_row, void* out_bf16,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LAYOUT_MOE_H */
