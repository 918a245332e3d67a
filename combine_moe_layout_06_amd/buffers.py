"""Device buffers of one MoE layer pass and the calls that fill them.

Plumbing only: torch allocates the caller-owned buffers that the C ABI
writes, sized on the host from (T, H, E, k, R, capacity) so that no count
has to be read back before dispatch (packed mode: T*k rows; capacity mode:
E*capacity rows). Every computation is a call into the HIP library.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

from . import (MOE_DTYPE_BF16, MOE_DTYPE_FP8_E4M3, MOE_DTYPE_MXFP8_E4M3, MOE_FP8_BLOCK,
               MOE_MX_BLOCK, moe_combine, moe_combine_local, moe_combine_partials,
               moe_dispatch, moe_expand, moe_layout, moe_layout_dispatch,
               moe_layout_workspace_bytes,
               moe_layout_batched, moe_rank_layout, moe_rank_layout_batched,
               moe_rank_layout_workspace_bytes, moe_route, moe_route_batched)


@dataclasses.dataclass
class LayerBuffers:
    tokens: int
    hidden: int
    experts: int
    top_k: int
    ranks: int
    capacity: int
    dtype: int                    # MOE_DTYPE_* of the dispatched rows
    topk_idx: object = None
    topk_weights: object = None
    expert_counts: object = None
    expert_offsets: object = None
    rank_counts: object = None
    rank_offsets: object = None
    rank_token_counts: object = None
    dst_row: object = None
    src_pair: object = None
    overflow: object = None
    workspace: object = None
    workspace_bytes: int = 0
    dispatched: object = None     # [rows, H] bf16 (as int16) or uint8 codes
    scales: object = None         # [rows, H/128] fp32 (FP8) or [rows, H/32] uint8 (MXFP8)
    combined: object = None       # [T, H] bf16 (as int16)

    @property
    def fp8(self) -> bool:
        return self.dtype != MOE_DTYPE_BF16

    @property
    def num_rows(self) -> int:
        if self.capacity > 0:
            return self.experts * self.capacity
        return self.tokens * self.top_k

    @classmethod
    def allocate(cls, tokens, hidden, experts, top_k, ranks, capacity=0, fp8=False,
                 device="cuda", with_rank_tokens=True, dtype=None) -> "LayerBuffers":
        """`dtype` (MOE_DTYPE_*) selects the dispatched format; `fp8=True` is
        shorthand for MOE_DTYPE_FP8_E4M3."""
        import torch
        i32 = dict(dtype=torch.int32, device=device)
        if dtype is None:
            dtype = MOE_DTYPE_FP8_E4M3 if fp8 else MOE_DTYPE_BF16
        b = cls(tokens, hidden, experts, top_k, ranks, capacity, dtype)
        t, e, k, r = tokens, experts, top_k, ranks
        b.topk_idx = torch.empty((t, k), **i32)
        b.topk_weights = torch.empty((t, k), dtype=torch.float32, device=device)
        b.expert_counts = torch.empty(e, **i32)
        b.expert_offsets = torch.empty(e + 1, **i32)
        b.rank_counts = torch.empty(r, **i32)
        b.rank_offsets = torch.empty(r + 1, **i32)
        b.rank_token_counts = torch.empty(r, **i32) if with_rank_tokens else None
        b.dst_row = torch.empty((t, k), **i32)
        b.src_pair = torch.empty(max(b.num_rows, 1), **i32)
        b.overflow = torch.empty(1, **i32)
        b.workspace_bytes = moe_layout_workspace_bytes(t, e, k)
        b.workspace = torch.empty(max(b.workspace_bytes, 4), dtype=torch.uint8, device=device)
        rows = max(b.num_rows, 1)
        if dtype == MOE_DTYPE_FP8_E4M3:
            b.dispatched = torch.empty((rows, hidden), dtype=torch.uint8, device=device)
            b.scales = torch.empty((rows, hidden // MOE_FP8_BLOCK), dtype=torch.float32,
                                   device=device)
        elif dtype == MOE_DTYPE_MXFP8_E4M3:
            b.dispatched = torch.empty((rows, hidden), dtype=torch.uint8, device=device)
            b.scales = torch.empty((rows, hidden // MOE_MX_BLOCK), dtype=torch.uint8,
                                   device=device)
        else:
            b.dispatched = torch.empty((rows, hidden), dtype=torch.int16, device=device)
        b.combined = torch.empty((max(t, 1), hidden), dtype=torch.int16, device=device)
        return b

    def sharing_rows(self, with_rank_tokens=True) -> "LayerBuffers":
        """A buffer set of the same shape with its own routing and layout
        buffers (topk, counts, offsets, dst_row, src_pair, workspace) but this
        set's dispatched, scales and combined rows: for steps whose route and
        layout may run ahead while earlier steps still dispatch and combine
        on another stream, one step after the other."""
        dev = self.topk_idx.device
        b = LayerBuffers.allocate(self.tokens, 0, self.experts, self.top_k, self.ranks,
                                  self.capacity, device=dev, with_rank_tokens=with_rank_tokens,
                                  dtype=MOE_DTYPE_BF16)
        b.hidden, b.dtype = self.hidden, self.dtype
        b.dispatched, b.scales, b.combined = self.dispatched, self.scales, self.combined
        return b

    def route(self, logits, bias, score_fn, num_groups=1, topk_groups=1, stream=None):
        moe_route(self.tokens, self.experts, self.top_k, logits, bias, score_fn, num_groups,
                  topk_groups, self.topk_idx, self.topk_weights, stream)

    def layout(self, stream=None):
        moe_layout(self.tokens, self.experts, self.top_k, self.ranks, self.capacity,
                   self.topk_idx, self.expert_counts, self.expert_offsets, self.rank_counts,
                   self.rank_offsets, self.rank_token_counts, self.dst_row, self.src_pair,
                   self.overflow, self.workspace, self.workspace_bytes, stream)

    def dispatch(self, x, stream=None):
        moe_dispatch(self.tokens, self.hidden, self.top_k, self.num_rows, x, self.dst_row,
                     self.dtype, self.dispatched, self.scales, stream)

    def layout_dispatch(self, x, stream=None):
        """layout() then dispatch(x); one launch for decode-sized inputs in
        capacity mode."""
        moe_layout_dispatch(self.tokens, self.experts, self.top_k, self.ranks, self.capacity,
                            self.topk_idx, self.expert_counts, self.expert_offsets,
                            self.rank_counts, self.rank_offsets, self.rank_token_counts,
                            self.dst_row, self.src_pair, self.overflow, self.workspace,
                            self.workspace_bytes, self.hidden, x, self.dtype, self.dispatched,
                            self.scales, stream)

    def combine(self, expert_out, stream=None):
        moe_combine(self.tokens, self.hidden, self.top_k, self.num_rows, expert_out,
                    self.dst_row, self.topk_weights, self.combined, stream)


@dataclasses.dataclass
class RankBuffers:
    """Buffers of the deduplicated dispatch and the hierarchical combine:
    one row per (token, rank), sized for its maximum T * min(k, R) rows so
    that no count is read back. Used with the expert layout of a
    LayerBuffers of the same shape (its dst_row, src_pair and weights)."""
    tokens: int
    hidden: int
    experts: int
    top_k: int
    ranks: int
    dtype: int
    rank_token_counts: object = None
    rank_token_offsets: object = None
    rank_row: object = None
    send_row: object = None
    row_token: object = None
    workspace: object = None
    workspace_bytes: int = 0
    sent: object = None          # [rank rows, H] bf16 (as int16) or uint8 codes
    sent_scales: object = None   # FP8 fp32 / MXFP8 uint8 scales of the sent rows
    partial: object = None       # [rank rows, H] bf16 partial sums (as int16)

    @property
    def num_rank_rows(self) -> int:
        return self.tokens * min(self.top_k, self.ranks)

    @classmethod
    def allocate(cls, tokens, hidden, experts, top_k, ranks, dtype=MOE_DTYPE_BF16,
                 device="cuda") -> "RankBuffers":
        import torch
        i32 = dict(dtype=torch.int32, device=device)
        b = cls(tokens, hidden, experts, top_k, ranks, dtype)
        t, k, r = tokens, top_k, ranks
        n = max(b.num_rank_rows, 1)
        b.rank_token_counts = torch.empty(r, **i32)
        b.rank_token_offsets = torch.empty(r + 1, **i32)
        b.rank_row = torch.empty((t, k), **i32)
        b.send_row = torch.empty((t, k), **i32)
        b.row_token = torch.empty(n, **i32)
        b.workspace_bytes = moe_rank_layout_workspace_bytes(t, k, r)
        b.workspace = torch.empty(max(b.workspace_bytes, 4), dtype=torch.uint8, device=device)
        if dtype == MOE_DTYPE_FP8_E4M3:
            b.sent = torch.empty((n, hidden), dtype=torch.uint8, device=device)
            b.sent_scales = torch.empty((n, hidden // MOE_FP8_BLOCK), dtype=torch.float32,
                                        device=device)
        elif dtype == MOE_DTYPE_MXFP8_E4M3:
            b.sent = torch.empty((n, hidden), dtype=torch.uint8, device=device)
            b.sent_scales = torch.empty((n, hidden // MOE_MX_BLOCK), dtype=torch.uint8,
                                        device=device)
        else:
            b.sent = torch.empty((n, hidden), dtype=torch.int16, device=device)
        b.partial = torch.empty((n, hidden), dtype=torch.int16, device=device)
        return b

    def sharing_rows(self) -> "RankBuffers":
        """A set of the same shape with its own (token, rank) layout buffers
        but this set's sent rows, their scales and the partial rows (see
        LayerBuffers.sharing_rows)."""
        b = RankBuffers.allocate(self.tokens, 0, self.experts, self.top_k, self.ranks,
                                 MOE_DTYPE_BF16, device=self.rank_row.device)
        b.hidden, b.dtype = self.hidden, self.dtype
        b.sent, b.sent_scales, b.partial = self.sent, self.sent_scales, self.partial
        return b

    def rank_layout(self, topk_idx, stream=None):
        moe_rank_layout(self.tokens, self.experts, self.top_k, self.ranks, topk_idx,
                        self.rank_token_counts, self.rank_token_offsets, self.rank_row,
                        self.send_row, self.row_token, self.workspace, self.workspace_bytes,
                        stream)

    def dispatch(self, x, stream=None):
        """One copy of each token per rank it has experts on."""
        moe_dispatch(self.tokens, self.hidden, self.top_k, self.num_rank_rows, x,
                     self.send_row, self.dtype, self.sent, self.sent_scales, stream)

    def expand(self, layer: LayerBuffers, stream=None):
        """Fan the sent rows out to the expert rows of `layer`."""
        moe_expand(self.tokens, self.hidden, self.top_k, self.dtype, self.num_rank_rows,
                   self.sent, self.sent_scales, self.rank_row, self.row_token, layer.num_rows,
                   layer.dst_row, layer.dispatched, layer.scales, stream)

    def combine_local(self, layer: LayerBuffers, expert_out, stream=None):
        moe_combine_local(self.tokens, self.hidden, self.top_k, layer.num_rows, expert_out,
                          layer.dst_row, self.rank_row, self.row_token, layer.topk_weights,
                          self.num_rank_rows, self.partial, stream)

    def combine_partials(self, out, stream=None):
        moe_combine_partials(self.tokens, self.hidden, self.top_k, self.num_rank_rows,
                             self.partial, self.send_row, out, stream)


def route_batches(bufs, logits, biases, score_fn, num_groups=1, topk_groups=1, stream=None):
    """route() of every LayerBuffers in `bufs` (same sizes) on its own logits
    and bias (entries may be None), in one launch (moe_route_batched)."""
    b0 = bufs[0]
    moe_route_batched(b0.tokens, b0.experts, b0.top_k,
                      [(lg, bs, b.topk_idx, b.topk_weights)
                       for b, lg, bs in zip(bufs, logits, biases)],
                      score_fn, num_groups, topk_groups, stream)


def layout_batches(bufs, stream=None):
    """layout() of every LayerBuffers in `bufs` (same sizes), one launch per
    pass for all of them (moe_layout_batched)."""
    b0 = bufs[0]
    moe_layout_batched(b0.tokens, b0.experts, b0.top_k, b0.ranks, b0.capacity,
                       [dict(topk_idx=b.topk_idx, expert_counts=b.expert_counts,
                             expert_offsets=b.expert_offsets, rank_counts=b.rank_counts,
                             rank_offsets=b.rank_offsets, rank_token_counts=b.rank_token_counts,
                             dst_row=b.dst_row, src_pair=b.src_pair, overflow=b.overflow,
                             workspace=b.workspace, workspace_bytes=b.workspace_bytes)
                        for b in bufs], stream)


def rank_layout_batches(bufs, topk_idx, stream=None):
    """rank_layout() of every RankBuffers in `bufs` (same sizes) on the
    routing topk_idx[i] of each, one launch per pass for all of them
    (moe_rank_layout_batched)."""
    b0 = bufs[0]
    moe_rank_layout_batched(b0.tokens, b0.experts, b0.top_k, b0.ranks,
                            [dict(topk_idx=ix, rank_token_counts=b.rank_token_counts,
                                  rank_token_offsets=b.rank_token_offsets, rank_row=b.rank_row,
                                  send_row=b.send_row, row_token=b.row_token,
                                  workspace=b.workspace, workspace_bytes=b.workspace_bytes)
                             for b, ix in zip(bufs, topk_idx)], stream)


def run_layer(buf: LayerBuffers, logits, bias, x, score_fn, num_groups=1, topk_groups=1,
              stream: Optional[object] = None) -> None:
    """Route, lay out and dispatch one layer pass (combine follows the experts);
    layout and dispatch go through moe_layout_dispatch."""
    buf.route(logits, bias, score_fn, num_groups, topk_groups, stream)
    buf.layout_dispatch(x, stream)
