"""GPU parity of moe_layout_dispatch (layout then dispatch; one launch for
decode-sized inputs in capacity mode) against the CPU oracle.

Bars: every layout output and every dispatched row (bf16, FP8 codes and
scales, MXFP8 codes and scale bytes) bit for bit; rows that no pair reaches
keep their poison, and nothing is written past the buffers.
"""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

import combine_moe_layout_06_amd as M  # noqa: E402
from combine_moe_layout_06_amd import LayerBuffers  # noqa: E402
from gpu_helpers import dev, host, poison_like  # noqa: E402
from oracle import moe_oracle as O  # noqa: E402
from synth import workloads as W  # noqa: E402

GUARD = 8


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("the GPU tests need a visible MI355X")
    M.lib()
    yield
    torch.cuda.synchronize()


def _oracle_rows(dtype, x, dst, rows):
    if dtype == M.MOE_DTYPE_BF16:
        o, wr = O.dispatch_bf16(x, dst, rows)
        return [o], wr
    f = O.dispatch_fp8 if dtype == M.MOE_DTYPE_FP8_E4M3 else O.dispatch_mxfp8
    q, s, wr = f(x, dst, rows)
    return [q, s], wr


CASES = [
    # T, E, k, R, cap, dtype, H, distinct, mask_frac
    (128, 256, 8, 32, 128, 1, 7168, True, 0.0),    # decode shape: one launch
    (100, 16, 4, 4, 5, 0, 256, True, 0.05),        # drops at capacity
    (37, 8, 8, 2, 3, 2, 256, False, 0.1),          # repeated experts, drops, MXFP8
    (200, 64, 5, 8, 10, 1, 256, True, 0.0),        # 1000 pairs: one launch
    (205, 64, 5, 8, 10, 1, 256, True, 0.0),        # 1025 pairs: layout, then dispatch
    (300, 32, 4, 4, 0, 0, 512, True, 0.0),         # packed: layout, then dispatch
    (1, 512, 32, 16, 2, 1, 384, True, 0.0),        # one token, k = 32
    (64, 24, 6, 6, 1, 2, 96, True, 0.2),           # cap 1, MXFP8 with 3 blocks per row
    (0, 8, 2, 4, 3, 0, 256, True, 0.0),            # empty
    # packed, many tiles: count + place, then dispatch
    (4096, 256, 8, 32, 0, 1, 1024, True, 0.02),    # DeepSeek-V3 routing shape, FP8
    (3000, 64, 4, 8, 0, 0, 256, False, 0.1),       # repeated experts, masked pairs, bf16
    (1500, 8, 1, 2, 0, 2, 128, True, 0.0),         # k = 1, two tiles, MXFP8
    (8192, 128, 8, 16, 0, 0, 256, True, 0.0),      # 64 tiles x 128 experts
    (2048, 512, 8, 512, 0, 1, 128, True, 0.05),    # 16 tiles x 512 experts, 512 ranks
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T%d_E%d_k%d_R%d_cap%d_dt%d" % c[:6])
def test_layout_dispatch_parity(case):
    t, e, k, r, cap, dtype, h, distinct, mf = case
    say("layout+dispatch case", case)
    g = W.rng(sum(case[:7]) + 21)
    idx = W.random_topk_idx(g, t, e, k, distinct=distinct, mask_frac=mf)
    x = W.random_bf16_rows(g, t, h)
    b = LayerBuffers.allocate(t, h, e, k, r, cap, dtype=dtype)
    rows = b.num_rows
    b.src_pair = poison_like(max(rows, 1) + GUARD, torch.int32)
    b.dst_row = poison_like((max(t, 1), k), torch.int32)
    b.dispatched = poison_like((max(rows, 1) + GUARD, h), b.dispatched.dtype)
    if dtype:
        b.scales = poison_like((max(rows, 1) + GUARD,) + tuple(b.scales.shape[1:]), b.scales.dtype)
    if t:
        b.topk_idx.copy_(dev(idx))
    b.layout_dispatch(dev(x) if t else None)

    L = O.layout(idx, e, r, cap)
    for name in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets",
                 "rank_token_counts", "overflow"):
        got = host(getattr(b, name))
        assert np.array_equal(got.reshape(L[name].shape), L[name]), name
    assert np.array_equal(host(b.dst_row)[:t], L["dst_row"])
    src = host(b.src_pair)
    assert np.array_equal(src[:rows], L["src_pair"]) and (src[rows:] == -1).all()
    want, written = _oracle_rows(dtype, x, L["dst_row"], rows)
    got = [host(b.dispatched)] + ([host(b.scales)] if dtype else [])
    for gr, wr in zip(got, want):
        gr = gr.view(wr.dtype) if gr.dtype != wr.dtype else gr
        a, o = gr[:rows][written], wr[written]
        if a.dtype == np.float32:
            a, o = a.view(np.uint32), o.view(np.uint32)
        assert np.array_equal(a, o)
        raw = gr.view(np.uint8).reshape(gr.shape[0], -1)
        assert (raw[:rows][~written] == 0xFF).all() and (raw[rows:] == 0xFF).all()
    say("  one launch" if cap > 0 and 0 < t * k <= 1024 else "  layout, then dispatch",
        "; dropped pairs", int(L["overflow"][0]))


def test_layout_dispatch_equals_separate_calls_on_a_decode_step():
    w = W.WORKLOADS["decode"]
    inp = W.make_inputs(w, 1234)
    bufs = []
    for fused in (True, False):
        b = LayerBuffers.allocate(w.tokens, w.hidden, w.experts, w.top_k, w.ranks, w.capacity,
                                  dtype=M.MOE_DTYPE_FP8_E4M3)
        b.dispatched.zero_()
        b.scales.zero_()
        b.route(dev(inp.logits), dev(inp.bias), w.score_fn, w.groups, w.topk_groups)
        if fused:
            b.layout_dispatch(dev(inp.x))
        else:
            b.layout()
            b.dispatch(dev(inp.x))
        bufs.append(b)
    torch.cuda.synchronize()
    for name in ("topk_idx", "dst_row", "src_pair", "expert_counts", "rank_token_counts",
                 "dispatched", "scales"):
        assert torch.equal(getattr(bufs[0], name), getattr(bufs[1], name)), name



def test_layout_dispatch_reuses_its_workspace():
    """Three packed calls on the same buffers with different routing (the
    first on a workspace full of 0xFF bytes, the last without distinct-token
    counts) each match the oracle: no call depends on what an earlier one
    left in the workspace."""
    t, e, k, r, h = 2048, 64, 8, 8, 256
    b = LayerBuffers.allocate(t, h, e, k, r, 0, dtype=M.MOE_DTYPE_BF16)
    b.workspace.fill_(0xFF)
    for call in range(3):
        g = W.rng(500 + call)
        idx = W.random_topk_idx(g, t, e, k, distinct=call != 1, mask_frac=0.03 * call)
        x = W.random_bf16_rows(g, t, h)
        if call == 2:
            b.rank_token_counts = None
        b.topk_idx.copy_(dev(idx))
        b.layout_dispatch(dev(x))
        L = O.layout(idx, e, r, 0)
        names = ["expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "dst_row",
                 "src_pair", "overflow"] + (["rank_token_counts"] if call < 2 else [])
        for name in names:
            got = host(getattr(b, name))
            assert np.array_equal(got.reshape(L[name].shape), L[name]), (call, name)
        want, written = _oracle_rows(M.MOE_DTYPE_BF16, x, L["dst_row"], b.num_rows)
        got = host(b.dispatched).view(np.uint16)
        assert np.array_equal(got[written], want[0][written]), call
        say("  call", call, "matches the oracle")
