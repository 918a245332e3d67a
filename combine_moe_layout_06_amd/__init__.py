"""MoE expert-parallel hot path on one AMD Instinct MI355X (gfx950).

Python binding of the C ABI in include/moe.h (library libmoe_layout.so,
built by `python -m combine_moe_layout_06_amd.build`). The functions keep
the C names and argument order and only marshal arguments: every step runs
in the HIP kernels of the library. A tensor argument must be a contiguous
device tensor (its data_ptr() is passed); an int is taken as a raw device
pointer; None is NULL. `stream` defaults to torch's current stream.

There is no CPU fallback: if the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

MOE_OK = 0
MOE_ERR_INVALID = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_HIP = 4

MOE_SCORE_SOFTMAX = 0
MOE_SCORE_SIGMOID = 1
MOE_DTYPE_BF16 = 0
MOE_DTYPE_FP8_E4M3 = 1
MOE_DTYPE_MXFP8_E4M3 = 2

MOE_MAX_EXPERTS = 512
MOE_MAX_TOPK = 32
MOE_MAX_GROUPS = 64
MOE_FP8_BLOCK = 128
MOE_MX_BLOCK = 32
MOE_MAX_BATCHES = 8

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_layout.so")

EXPORTED = ("moe_status_string", "moe_last_error", "moe_route",
            "moe_layout_workspace_bytes", "moe_layout", "moe_dispatch", "moe_combine",
            "moe_dispatch_backward", "moe_combine_backward",
            "moe_rank_layout_workspace_bytes", "moe_rank_layout", "moe_expand",
            "moe_combine_local", "moe_combine_partials", "moe_layout_dispatch",
            "moe_layout_dispatch_is_fused", "moe_layout_no_alloc", "moe_route_batched",
            "moe_layout_batched", "moe_rank_layout_batched")

_lib = None


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (_status_name(status), message))
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("HIP library %s is missing; run "
                           "`python -m combine_moe_layout_06_amd.build`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    i32, vp, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    L.moe_status_string.argtypes = [i32]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_route.argtypes = [i32, i32, i32, vp, vp, i32, i32, i32, vp, vp, vp]
    L.moe_route.restype = i32
    L.moe_layout_workspace_bytes.argtypes = [i32, i32, i32]
    L.moe_layout_workspace_bytes.restype = sz
    L.moe_layout.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                             vp, sz, vp]
    L.moe_layout.restype = i32
    L.moe_dispatch.argtypes = [i32, i32, i32, i32, vp, vp, i32, vp, vp, vp]
    L.moe_dispatch.restype = i32
    L.moe_combine.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp]
    L.moe_combine.restype = i32
    L.moe_dispatch_backward.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp]
    L.moe_dispatch_backward.restype = i32
    L.moe_combine_backward.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    L.moe_combine_backward.restype = i32
    L.moe_rank_layout_workspace_bytes.argtypes = [i32, i32, i32]
    L.moe_rank_layout_workspace_bytes.restype = sz
    L.moe_rank_layout.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_rank_layout.restype = i32
    L.moe_expand.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, i32, vp, vp, vp, vp]
    L.moe_expand.restype = i32
    L.moe_combine_local.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, i32, vp, vp]
    L.moe_combine_local.restype = i32
    L.moe_combine_partials.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp]
    L.moe_combine_partials.restype = i32
    L.moe_layout_dispatch.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, vp, sz, i32, vp, i32, vp, vp, vp]
    L.moe_layout_dispatch.restype = i32
    L.moe_layout_dispatch_is_fused.argtypes = [i32, i32, i32]
    L.moe_layout_dispatch_is_fused.restype = i32
    L.moe_layout_no_alloc.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, vp]
    L.moe_layout_no_alloc.restype = i32
    L.moe_route_batched.argtypes = [i32, vp, i32, i32, i32, i32, i32, i32, vp]
    L.moe_route_batched.restype = i32
    L.moe_layout_batched.argtypes = [i32, vp, i32, i32, i32, i32, i32, vp]
    L.moe_layout_batched.restype = i32
    L.moe_rank_layout_batched.argtypes = [i32, vp, i32, i32, i32, i32, vp]
    L.moe_rank_layout_batched.restype = i32
    _lib = L
    return L


def _status_name(status: int) -> str:
    try:
        return lib().moe_status_string(status).decode()
    except Exception:  # the library itself failed to load
        return "status %d" % status


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("expected a device tensor, got one on %s" % t.device)
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


_raw_stream = None


def _current_stream() -> int:
    """Raw handle of torch's current stream on the current device. Uses the
    accessor torch's own generated code calls (well under a microsecond),
    else the public Stream object (a few microseconds, which adds up to a
    large share of a decode step's host time)."""
    global _raw_stream
    if _raw_stream is None:
        import torch
        fast = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        device = getattr(torch._C, "_cuda_getDevice", None)
        if fast is not None and device is not None:
            _raw_stream = lambda: fast(device())
        else:
            _raw_stream = lambda: torch.cuda.current_stream().cuda_stream
    return _raw_stream()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return _current_stream()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int) -> None:
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode())


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_route(num_tokens, num_experts, top_k, logits, bias, score_fn, num_groups,
              topk_groups, topk_idx, topk_weights, stream=None) -> None:
    _check(lib().moe_route(num_tokens, num_experts, top_k, _ptr(logits), _ptr(bias),
                           score_fn, num_groups, topk_groups, _ptr(topk_idx),
                           _ptr(topk_weights), _stream(stream)))


def moe_layout_workspace_bytes(num_tokens, num_experts, top_k) -> int:
    return int(lib().moe_layout_workspace_bytes(num_tokens, num_experts, top_k))


def moe_layout(num_tokens, num_experts, top_k, num_ranks, capacity, topk_idx,
               expert_counts, expert_offsets, rank_counts, rank_offsets,
               rank_token_counts, dst_row, src_pair, overflow, workspace,
               workspace_bytes, stream=None) -> None:
    _check(lib().moe_layout(num_tokens, num_experts, top_k, num_ranks, capacity,
                            _ptr(topk_idx), _ptr(expert_counts), _ptr(expert_offsets),
                            _ptr(rank_counts), _ptr(rank_offsets), _ptr(rank_token_counts),
                            _ptr(dst_row), _ptr(src_pair), _ptr(overflow), _ptr(workspace),
                            workspace_bytes, _stream(stream)))


def moe_layout_no_alloc(num_tokens, num_experts, top_k, num_ranks, capacity, topk_idx,
                        expert_counts, expert_offsets, rank_counts, rank_offsets,
                        rank_token_counts, dst_row, src_pair, overflow, stream=None) -> None:
    _check(lib().moe_layout_no_alloc(num_tokens, num_experts, top_k, num_ranks, capacity,
                                     _ptr(topk_idx), _ptr(expert_counts), _ptr(expert_offsets),
                                     _ptr(rank_counts), _ptr(rank_offsets),
                                     _ptr(rank_token_counts), _ptr(dst_row), _ptr(src_pair),
                                     _ptr(overflow), _stream(stream)))


class RouteIO(ctypes.Structure):
    """moe_route_io: one batch of moe_route_batched."""
    _fields_ = [("logits", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("topk_idx", ctypes.c_void_p), ("topk_weights", ctypes.c_void_p)]


class LayoutIO(ctypes.Structure):
    """moe_layout_io: one batch of moe_layout_batched."""
    _fields_ = [("topk_idx", ctypes.c_void_p), ("expert_counts", ctypes.c_void_p),
                ("expert_offsets", ctypes.c_void_p), ("rank_counts", ctypes.c_void_p),
                ("rank_offsets", ctypes.c_void_p), ("rank_token_counts", ctypes.c_void_p),
                ("dst_row", ctypes.c_void_p), ("src_pair", ctypes.c_void_p),
                ("overflow", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


def moe_route_batched(num_tokens, num_experts, top_k, batches, score_fn, num_groups,
                      topk_groups, stream=None) -> None:
    """batches: sequence of (logits, bias or None, topk_idx, topk_weights)
    device tensors."""
    arr = (RouteIO * max(len(batches), 1))(
        *[RouteIO(_ptr(lg), _ptr(bs), _ptr(ix), _ptr(wt)) for lg, bs, ix, wt in batches])
    _check(lib().moe_route_batched(len(batches), ctypes.cast(arr, ctypes.c_void_p), num_tokens,
                                   num_experts, top_k, score_fn, num_groups, topk_groups,
                                   _stream(stream)))


def moe_layout_batched(num_tokens, num_experts, top_k, num_ranks, capacity, batches,
                       stream=None) -> None:
    """batches: sequence of dicts with the keys of LayoutIO (device tensors;
    workspace_bytes an int)."""
    arr = (LayoutIO * max(len(batches), 1))(
        *[LayoutIO(*[_ptr(b.get(f)) for f, _ in LayoutIO._fields_[:-1]],
                   int(b["workspace_bytes"])) for b in batches])
    _check(lib().moe_layout_batched(len(batches), ctypes.cast(arr, ctypes.c_void_p), num_tokens,
                                    num_experts, top_k, num_ranks, capacity, _stream(stream)))


class RankLayoutIO(ctypes.Structure):
    """moe_rank_layout_io: one batch of moe_rank_layout_batched."""
    _fields_ = [("topk_idx", ctypes.c_void_p), ("rank_token_counts", ctypes.c_void_p),
                ("rank_token_offsets", ctypes.c_void_p), ("rank_row", ctypes.c_void_p),
                ("send_row", ctypes.c_void_p), ("row_token", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


def moe_rank_layout_batched(num_tokens, num_experts, top_k, num_ranks, batches,
                            stream=None) -> None:
    """batches: sequence of dicts with the keys of RankLayoutIO (device
    tensors; workspace_bytes an int)."""
    arr = (RankLayoutIO * max(len(batches), 1))(
        *[RankLayoutIO(*[_ptr(b.get(f)) for f, _ in RankLayoutIO._fields_[:-1]],
                       int(b["workspace_bytes"])) for b in batches])
    _check(lib().moe_rank_layout_batched(len(batches), ctypes.cast(arr, ctypes.c_void_p),
                                         num_tokens, num_experts, top_k, num_ranks,
                                         _stream(stream)))


def moe_layout_dispatch_is_fused(num_tokens, top_k, capacity) -> bool:
    return bool(lib().moe_layout_dispatch_is_fused(num_tokens, top_k, capacity))


def moe_layout_dispatch(num_tokens, num_experts, top_k, num_ranks, capacity, topk_idx,
                        expert_counts, expert_offsets, rank_counts, rank_offsets,
                        rank_token_counts, dst_row, src_pair, overflow, workspace,
                        workspace_bytes, hidden, x_bf16, out_dtype, out, out_scales,
                        stream=None) -> None:
    _check(lib().moe_layout_dispatch(num_tokens, num_experts, top_k, num_ranks, capacity,
                                     _ptr(topk_idx), _ptr(expert_counts), _ptr(expert_offsets),
                                     _ptr(rank_counts), _ptr(rank_offsets),
                                     _ptr(rank_token_counts), _ptr(dst_row), _ptr(src_pair),
                                     _ptr(overflow), _ptr(workspace), workspace_bytes, hidden,
                                     _ptr(x_bf16), out_dtype, _ptr(out), _ptr(out_scales),
                                     _stream(stream)))


def moe_dispatch(num_tokens, hidden, top_k, num_rows, x_bf16, dst_row, out_dtype, out,
                 out_scales, stream=None) -> None:
    _check(lib().moe_dispatch(num_tokens, hidden, top_k, num_rows, _ptr(x_bf16),
                              _ptr(dst_row), out_dtype, _ptr(out), _ptr(out_scales),
                              _stream(stream)))


def moe_combine(num_tokens, hidden, top_k, num_rows, expert_out_bf16, dst_row,
                topk_weights, out_bf16, stream=None) -> None:
    _check(lib().moe_combine(num_tokens, hidden, top_k, num_rows, _ptr(expert_out_bf16),
                             _ptr(dst_row), _ptr(topk_weights), _ptr(out_bf16),
                             _stream(stream)))


def moe_dispatch_backward(num_tokens, hidden, top_k, num_rows, grad_rows_bf16, dst_row,
                          grad_x_bf16, stream=None) -> None:
    _check(lib().moe_dispatch_backward(num_tokens, hidden, top_k, num_rows,
                                       _ptr(grad_rows_bf16), _ptr(dst_row), _ptr(grad_x_bf16),
                                       _stream(stream)))


def moe_combine_backward(num_tokens, hidden, top_k, num_rows, grad_out_bf16, expert_out_bf16,
                         dst_row, topk_weights, grad_expert_out_bf16, grad_weights,
                         stream=None) -> None:
    _check(lib().moe_combine_backward(num_tokens, hidden, top_k, num_rows, _ptr(grad_out_bf16),
                                      _ptr(expert_out_bf16), _ptr(dst_row), _ptr(topk_weights),
                                      _ptr(grad_expert_out_bf16), _ptr(grad_weights),
                                      _stream(stream)))


def moe_rank_layout_workspace_bytes(num_tokens, top_k, num_ranks) -> int:
    return int(lib().moe_rank_layout_workspace_bytes(num_tokens, top_k, num_ranks))


def moe_rank_layout(num_tokens, num_experts, top_k, num_ranks, topk_idx, rank_token_counts,
                    rank_token_offsets, rank_row, send_row, row_token, workspace,
                    workspace_bytes, stream=None) -> None:
    _check(lib().moe_rank_layout(num_tokens, num_experts, top_k, num_ranks, _ptr(topk_idx),
                                 _ptr(rank_token_counts), _ptr(rank_token_offsets),
                                 _ptr(rank_row), _ptr(send_row), _ptr(row_token),
                                 _ptr(workspace), workspace_bytes, _stream(stream)))


def moe_expand(num_tokens, hidden, top_k, dtype, num_rank_rows, rank_rows, rank_scales,
               rank_row, row_token, num_rows, dst_row, out, out_scales, stream=None) -> None:
    _check(lib().moe_expand(num_tokens, hidden, top_k, dtype, num_rank_rows, _ptr(rank_rows),
                            _ptr(rank_scales), _ptr(rank_row), _ptr(row_token), num_rows,
                            _ptr(dst_row), _ptr(out), _ptr(out_scales), _stream(stream)))


def moe_combine_local(num_tokens, hidden, top_k, num_rows, expert_out_bf16, dst_row, rank_row,
                      row_token, topk_weights, num_rank_rows, partial_bf16, stream=None) -> None:
    _check(lib().moe_combine_local(num_tokens, hidden, top_k, num_rows, _ptr(expert_out_bf16),
                                   _ptr(dst_row), _ptr(rank_row), _ptr(row_token),
                                   _ptr(topk_weights), num_rank_rows, _ptr(partial_bf16),
                                   _stream(stream)))


def moe_combine_partials(num_tokens, hidden, top_k, num_rank_rows, partial_bf16, send_row,
                         out_bf16, stream=None) -> None:
    _check(lib().moe_combine_partials(num_tokens, hidden, top_k, num_rank_rows,
                                      _ptr(partial_bf16), _ptr(send_row), _ptr(out_bf16),
                                      _stream(stream)))


from .buffers import (LayerBuffers, RankBuffers, layout_batches,  # noqa: E402,F401
                      rank_layout_batches, route_batches, run_layer)
