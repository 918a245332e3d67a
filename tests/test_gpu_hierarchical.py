"""GPU parity of the deduplicated dispatch and the hierarchical combine,
through the C ABI, against the CPU oracle on the same seeded inputs.

Bars: the (token, rank) layout, the sent rows (bf16, FP8 codes and scales,
MXFP8 codes and scale bytes) and the fanned-out expert rows are bit-exact;
partial rows and the final output equal the oracle's bits (both levels run
the oracle's arithmetic: fp32 fused multiply-adds in slot order, one bf16
rounding per level). Output buffers are pre-filled with 0xFF and
followed by guard rows, so unwritten rows and stray writes are caught.
"""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

import combine_moe_layout_06_amd as M  # noqa: E402
from combine_moe_layout_06_amd import LayerBuffers, RankBuffers  # noqa: E402
from gpu_helpers import assert_combine_exact, dev, host, poison_like  # noqa: E402
from oracle import moe_oracle as O  # noqa: E402
from synth import workloads as W  # noqa: E402

GUARD = 8
MARK = 0x5A5A5A5A   # guard value that no kernel writes


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


def marked(n):
    return torch.full((n,), MARK, dtype=torch.int32, device="cuda")


def gpu_rank_layout(idx, E, R):
    """moe_rank_layout into poisoned buffers with marked guards."""
    t, k = idx.shape
    nrr = t * min(k, R)
    cnt = torch.cat([poison_like(R, torch.int32), marked(GUARD)])
    off = torch.cat([poison_like(R + 1, torch.int32), marked(GUARD)])
    rr = torch.cat([poison_like(t * k, torch.int32), marked(GUARD)])
    sr = torch.cat([poison_like(t * k, torch.int32), marked(GUARD)])
    rt = torch.cat([poison_like(nrr, torch.int32), marked(GUARD)])
    wsb = M.moe_rank_layout_workspace_bytes(t, k, R)
    ws = torch.empty(max(wsb, 4), dtype=torch.uint8, device="cuda")
    M.moe_rank_layout(t, E, k, R, dev(idx) if t else None, cnt, off, rr, sr, rt, ws, wsb)
    out = dict(rank_token_counts=host(cnt), rank_token_offsets=host(off),
               rank_row=host(rr), send_row=host(sr), row_token=host(rt))
    sizes = dict(rank_token_counts=R, rank_token_offsets=R + 1, rank_row=t * k,
                 send_row=t * k, row_token=nrr)
    for name, n in sizes.items():
        assert np.all(out[name][n:] == MARK), "stray write after " + name
        out[name] = out[name][:n]
    out["rank_row"] = out["rank_row"].reshape(t, k)
    out["send_row"] = out["send_row"].reshape(t, k)
    return out, (rr, sr)


RANK_CASES = [
    # T, E, k, R, distinct, mask_frac
    (128, 8, 2, 4, True, 0.0),
    (4096, 256, 8, 32, True, 0.0),
    (8192, 128, 8, 16, True, 0.0),
    (128, 256, 8, 32, True, 0.0),        # one tile: single launch
    (129, 8, 8, 2, True, 0.0),           # ragged tile, k > R
    (1001, 12, 3, 3, False, 0.1),        # repeated experts, masked slots, R not 2^n
    (5000, 24, 8, 6, False, 0.0),
    (300, 512, 32, 512, True, 0.05),     # one expert per rank, max sizes
    (2000, 512, 32, 16, True, 0.0),
    (333, 16, 4, 1, True, 0.0),          # one rank
    (1, 512, 32, 16, True, 0.0),
    (0, 8, 2, 4, True, 0.0),             # empty
    (777, 20, 6, 5, True, 1.0),          # every slot masked
    # many tiles: from 256 tiles (or a histogram over two staging passes) a
    # scan pass feeds the place pass
    (8191, 256, 8, 32, True, 0.0),       # 64 tiles, ragged: staged
    (32773, 256, 8, 32, True, 0.0),      # 257 tiles, ragged: scanned
    (131073, 8, 2, 4, False, 0.05),      # 257 tiles of 512 tokens
    (2100, 512, 32, 512, True, 0.0),     # 66 tiles, 512 ranks: scanned
]


@pytest.mark.parametrize("case", RANK_CASES, ids=lambda c: "T%d_E%d_k%d_R%d" % c[:4])
def test_rank_layout_parity(case):
    t, e, k, r, distinct, mf = case
    say("rank layout case", case)
    g = W.rng(sum(case[:4]) + 5)
    idx = W.random_topk_idx(g, t, e, k, distinct=distinct, mask_frac=mf)
    got, _ = gpu_rank_layout(idx, e, r)
    want = O.rank_layout(idx, e, r)
    for name, val in got.items():
        assert np.array_equal(val, want[name].reshape(val.shape)), (case, name)


def test_rank_layout_ignores_out_of_range_ids():
    g = W.rng(9)
    idx = W.random_topk_idx(g, 700, 32, 4)
    idx[g.random(idx.shape) < 0.2] = 32 + 7
    idx[g.random(idx.shape) < 0.1] = -5
    got, _ = gpu_rank_layout(idx, 32, 8)
    want = O.rank_layout(idx, 32, 8)
    for name, val in got.items():
        assert np.array_equal(val, want[name].reshape(val.shape)), name


# ------------------------------------------------ dedup dispatch + fan-out

def _dispatch_oracle(dtype, x, dst, rows):
    if dtype == M.MOE_DTYPE_BF16:
        o, wr = O.dispatch_bf16(x, dst, rows)
        return [o], wr
    f = O.dispatch_fp8 if dtype == M.MOE_DTYPE_FP8_E4M3 else O.dispatch_mxfp8
    q, s, wr = f(x, dst, rows)
    return [q, s], wr


def _as_bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


@pytest.mark.parametrize("dtype", [0, 1, 2], ids=["bf16", "fp8", "mxfp8"])
@pytest.mark.parametrize("cap", [0, 5])
def test_dedup_dispatch_and_expand(dtype, cap):
    t, e, k, r, h = 600, 32, 4, 8, 512
    say("dedup dispatch + expand", dtype, cap)
    g = W.rng(40 + dtype * 2 + (cap > 0))
    idx = W.random_topk_idx(g, t, e, k, mask_frac=0.05)
    x = W.random_bf16_rows(g, t, h)
    lb = LayerBuffers.allocate(t, h, e, k, r, cap, dtype=dtype)
    rb = RankBuffers.allocate(t, h, e, k, r, dtype=dtype)
    nrr, rows = rb.num_rank_rows, lb.num_rows
    # poisoned row buffers with guard rows
    lb.dispatched = poison_like((rows + GUARD, h), lb.dispatched.dtype)
    rb.sent = poison_like((nrr + GUARD, h), rb.sent.dtype)
    if dtype:
        lb.scales = poison_like((rows + GUARD,) + tuple(lb.scales.shape[1:]), lb.scales.dtype)
        rb.sent_scales = poison_like((nrr + GUARD,) + tuple(rb.sent_scales.shape[1:]),
                                     rb.sent_scales.dtype)
    lb.topk_idx.copy_(dev(idx))
    lb.layout()
    rb.rank_layout(lb.topk_idx)
    rb.dispatch(dev(x))
    rb.expand(lb)

    L = O.layout(idx, e, r, cap)
    rl = O.rank_layout(idx, e, r)
    assert np.array_equal(host(lb.dst_row), L["dst_row"])
    assert np.array_equal(host(rb.send_row), rl["send_row"])
    want_sent, sw = _dispatch_oracle(dtype, x, rl["send_row"], nrr)
    want_rows, fw = _dispatch_oracle(dtype, x, L["dst_row"], rows)
    got_sent = [host(rb.sent)] + ([host(rb.sent_scales)] if dtype else [])
    got_rows = [host(lb.dispatched)] + ([host(lb.scales)] if dtype else [])
    for gs, ws in zip(got_sent, want_sent):
        gs = gs.view(ws.dtype) if gs.dtype != ws.dtype else gs
        assert np.array_equal(_as_bits(gs[:nrr][sw]), _as_bits(ws[sw]))
        raw = gs.view(np.uint8).reshape(gs.shape[0], -1)
        assert (raw[:nrr][~sw] == 0xFF).all() and (raw[nrr:] == 0xFF).all()
    for gr, wr in zip(got_rows, want_rows):
        gr = gr.view(wr.dtype) if gr.dtype != wr.dtype else gr
        assert np.array_equal(_as_bits(gr[:rows][fw]), _as_bits(wr[fw]))
        raw = gr.view(np.uint8).reshape(gr.shape[0], -1)
        assert (raw[:rows][~fw] == 0xFF).all() and (raw[rows:] == 0xFF).all()
    say("  sent rows %d of %d pairs" % (int(sw.sum()), int((idx >= 0).sum())))


# ------------------------------------------------------ hierarchical combine

def run_hierarchical(idx, e, r, cap, y, wts, h):
    """GPU: expert layout, rank layout, local partials, per-token sums."""
    t, k = idx.shape
    lb = LayerBuffers.allocate(t, h, e, k, r, cap)
    rb = RankBuffers.allocate(t, h, e, k, r)
    nrr = rb.num_rank_rows
    rb.partial = poison_like((nrr + GUARD, h), torch.int16)
    if t:
        lb.topk_idx.copy_(dev(idx))
        lb.topk_weights.copy_(torch.from_numpy(wts).cuda())
    lb.layout()
    rb.rank_layout(lb.topk_idx)
    out = poison_like((t + GUARD, h), torch.int16)
    y_dev = dev(y)
    rb.combine_local(lb, y_dev)
    rb.combine_partials(out)
    return lb, rb, host(out, np.uint16), host(rb.partial, np.uint16)


LOCAL_CASES = [
    # T, E, k, R, cap, H
    (300, 32, 8, 8, 0, 256),
    (257, 16, 4, 4, 3, 128),       # capacity drops, whole (token, rank) rows dropped
    (100, 12, 3, 3, 0, 64),        # any-k kernel
    (64, 8, 2, 8, 0, 512),         # one expert per rank
    (50, 512, 32, 16, 0, 64),      # k = 32
    (90, 18, 6, 3, 2, 64),         # k = 6 with drops
    (40, 8, 1, 2, 0, 72),          # k = 1, hidden not a multiple of 512
    (128, 256, 8, 32, 128, 7168),  # decode shape
    (200, 64, 8, 8, 0, 2880),      # k = 8 items of 1 KiB: 3 parts, the last one ragged
    (77, 64, 8, 16, 5, 1000),      # k = 8, one part shorter than a wave's chunk step
    (33, 16, 8, 4, 0, 8),          # k = 8, one 16-byte chunk per row
    (0, 8, 2, 4, 0, 64),           # empty
]


@pytest.mark.parametrize("case", LOCAL_CASES, ids=lambda c: "T%d_E%d_k%d_R%d_cap%d_H%d" % c)
def test_hierarchical_combine_parity(case):
    t, e, k, r, cap, h = case
    say("hierarchical combine case", case)
    g = W.rng(sum(case) + 3)
    idx = W.random_topk_idx(g, t, e, k, mask_frac=0.05)
    L = O.layout(idx, e, r, cap)
    rl = O.rank_layout(idx, e, r)
    y = W.random_bf16_rows(g, L["num_rows"], h)
    wts = W.random_weights(g, t, k)
    lb, rb, out_g, part_g = run_hierarchical(idx, e, r, cap, y, wts, h)
    nrr = rl["num_rank_rows"]
    assert np.array_equal(host(rb.rank_row), rl["rank_row"])
    part_o, written, _ = O.combine_local(y, L["dst_row"], rl["rank_row"], wts, nrr)
    # rows nobody owns and the guard stay untouched
    assert (part_g[:nrr][~written] == 0xFFFF).all() and (part_g[nrr:] == 0xFFFF).all()
    assert_combine_exact(part_g[:nrr][written], part_o[written], "partial %s" % (case,))
    out_o, _ = O.combine_partials(part_o, rl["send_row"])
    assert (out_g[t:] == 0xFFFF).all()
    assert_combine_exact(out_g[:t], out_o, "two-level %s" % (case,))
    say("  partials and outputs equal the oracle's bits")


PARTIAL_CASES = [
    # T, E, k, R, H
    (500, 64, 8, 16, 384),
    (1000, 256, 8, 32, 7168),      # k = 8 items of 1 KiB: 14 parts
    (300, 64, 8, 8, 2880),         # 3 parts, the last one ragged
    (77, 32, 8, 4, 1000),          # one part shorter than a wave's chunk step
    (33, 16, 8, 4, 8),             # one 16-byte chunk per row
    (200, 24, 6, 6, 512),          # k = 6
]


@pytest.mark.parametrize("case", PARTIAL_CASES, ids=lambda c: "T%d_E%d_k%d_R%d_H%d" % c)
def test_combine_partials_parity(case):
    """Second level alone on synthetic partial rows."""
    t, e, k, r, h = case
    g = W.rng(77 + sum(case))
    idx = W.random_topk_idx(g, t, e, k, mask_frac=0.1)
    rl = O.rank_layout(idx, e, r)
    nrr = rl["num_rank_rows"]
    part = W.random_bf16_rows(g, nrr, h)
    out = poison_like((t + GUARD, h), torch.int16)
    M.moe_combine_partials(t, h, k, nrr, dev(part), dev(rl["send_row"]), out)
    got = host(out, np.uint16)
    want, _ = O.combine_partials(part, rl["send_row"])
    assert (got[t:] == 0xFFFF).all()
    assert_combine_exact(got[:t], want, "partials")


def test_one_rank_equals_flat_combine_bit_for_bit():
    """R = 1: one partial per token, the same fp32 chain in slot order as
    moe_combine, and adding it to zero is exact: identical bits."""
    g = W.rng(78)
    t, e, k, h = 400, 16, 8, 512
    idx = W.random_topk_idx(g, t, e, k, mask_frac=0.05)
    L = O.layout(idx, e, 1)
    y = W.random_bf16_rows(g, L["num_rows"], h)
    wts = W.random_weights(g, t, k)
    lb, rb, out_g, _ = run_hierarchical(idx, e, 1, 0, y, wts, h)
    flat = poison_like((t, h), torch.int16)
    M.moe_combine(t, h, k, lb.num_rows, dev(y), lb.dst_row, lb.topk_weights, flat)
    assert np.array_equal(out_g[:t], host(flat, np.uint16))
    want, _ = O.combine(y, L["dst_row"], wts)
    assert_combine_exact(out_g[:t], want, "one rank")


# -------------------------------------------------------- whole layer pass

@pytest.mark.parametrize("name,seed", [("dsv3", 0), ("qwen3_skew", 1), ("decode", 1000),
                                       ("tiny", 2)])
def test_hierarchical_layer_end_to_end(name, seed):
    """route -> layout -> rank layout -> deduplicated dispatch -> fan-out ->
    (stand-in expert) -> partials -> output, at the workload's full size."""
    w = W.WORKLOADS[name]
    say("hierarchical layer", name, "seed", seed)
    inp = W.make_inputs(w, seed)
    t, h, k = w.tokens, w.hidden, w.top_k
    dt = w.dispatch_dtype
    lb = LayerBuffers.allocate(t, h, w.experts, k, w.ranks, w.capacity, dtype=dt)
    rb = RankBuffers.allocate(t, h, w.experts, k, w.ranks, dtype=dt)
    bias = dev(inp.bias) if inp.bias is not None else None
    lb.route(dev(inp.logits), bias, w.score_fn, w.groups, w.topk_groups)
    lb.layout()
    rb.rank_layout(lb.topk_idx)
    rb.dispatch(dev(inp.x))
    rb.expand(lb)
    idx_g = host(lb.topk_idx)
    wts = host(lb.topk_weights)
    L = O.layout(idx_g, w.experts, w.ranks, w.capacity)
    rl = O.rank_layout(idx_g, w.experts, w.ranks)
    for nm in ("rank_token_counts", "rank_token_offsets", "rank_row", "send_row", "row_token"):
        assert np.array_equal(host(getattr(rb, nm))[:rl[nm].size].reshape(rl[nm].shape),
                              rl[nm]), nm
    assert np.array_equal(host(rb.rank_token_counts), host(lb.rank_token_counts))
    rows = L["num_rows"]
    want, fw = _dispatch_oracle(dt, inp.x, L["dst_row"], rows)
    got = [host(lb.dispatched)] + ([host(lb.scales)] if dt else [])
    for gr, wr in zip(got, want):
        gr = gr.view(wr.dtype) if gr.dtype != wr.dtype else gr
        assert np.array_equal(_as_bits(gr[:rows][fw]), _as_bits(wr[fw]))
    n_sent = int(rl["rank_token_offsets"][-1])
    say("  fan-out ok: %d rows sent for %d pairs" % (n_sent, int((idx_g >= 0).sum())))

    # stand-in expert on the oracle side: the dequantised (or copied) rows
    if dt == M.MOE_DTYPE_FP8_E4M3:
        y = O.expert_dequant(want[0], want[1])
    elif dt == M.MOE_DTYPE_MXFP8_E4M3:
        y = O.expert_dequant_mx(want[0], want[1])
    else:
        y = want[0]
    rb.combine_local(lb, dev(np.ascontiguousarray(y)))
    out = poison_like((t, h), torch.int16)
    rb.combine_partials(out)
    part_o, written, _ = O.combine_local(y, L["dst_row"], rl["rank_row"], wts,
                                         rl["num_rank_rows"])
    part_g = host(rb.partial, np.uint16)
    assert_combine_exact(part_g[written], part_o[written], name)
    out_o, _ = O.combine_partials(part_o, rl["send_row"])
    assert_combine_exact(host(out, np.uint16), out_o, name + " two-level")
    say("  two-level combine ok: partials and outputs equal the oracle's bits")


def test_hierarchical_pass_is_deterministic():
    """Two runs of the whole pass on the same inputs give identical bits."""
    w = W.WORKLOADS["dsv3"]
    inp = W.make_inputs(w, 5, tokens=1500)
    t, h, k = 1500, w.hidden, w.top_k
    runs = []
    for _ in range(2):
        lb = LayerBuffers.allocate(t, h, w.experts, k, w.ranks, 0, dtype=M.MOE_DTYPE_FP8_E4M3)
        rb = RankBuffers.allocate(t, h, w.experts, k, w.ranks, dtype=M.MOE_DTYPE_FP8_E4M3)
        lb.route(dev(inp.logits), dev(inp.bias), w.score_fn, w.groups, w.topk_groups)
        lb.layout()
        rb.rank_layout(lb.topk_idx)
        rb.dispatch(dev(inp.x))
        rb.expand(lb)
        y = lb.dispatched.view(torch.float8_e4m3fn).float().to(torch.bfloat16).view(torch.int16)
        rb.combine_local(lb, y.contiguous())
        out = torch.empty((t, h), dtype=torch.int16, device="cuda")
        rb.combine_partials(out)
        torch.cuda.synchronize()
        runs.append([rb.rank_row.clone(), rb.send_row.clone(), rb.row_token.clone(),
                     rb.sent.clone(), rb.sent_scales.clone(), lb.dispatched.clone(),
                     rb.partial.clone(), out])
    names = ["rank_row", "send_row", "row_token", "sent", "sent_scales", "expanded",
             "partial", "out"]
    for name, a, b in zip(names, runs[0], runs[1]):
        if name in ("partial", "sent", "sent_scales"):   # compare the written rows only
            rows = int(rb.rank_token_offsets[-1].item())
            a, b = a[:rows], b[:rows]
        assert torch.equal(a, b), name
