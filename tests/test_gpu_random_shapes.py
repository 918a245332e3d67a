"""Seeded random sweep over shapes: the GPU path against the CPU oracle on
draws that the hand-picked parity cases do not spell out.

Each case draws, from its own seed: the ranks R and experts per rank (so
E = R * E/R), k, the token count T (often next to a tile or wave boundary),
the capacity (0 = packed, or small enough to drop pairs), the dispatch
format, a hidden size of that format's granularity, repeated or distinct
experts per token, and a fraction of masked slots. It then checks:
  - moe_route on random logits (softmax, or group-limited sigmoid when the
    draw has groups): choices up to logged near-ties, weights within 1 ulp;
  - moe_layout_dispatch (the one-launch path when capacity > 0 and
    T*k <= 1024, else layout then dispatch): every layout output and every
    written row bit for bit; rows no pair reaches keep their poison;
  - moe_combine on random rows and weights: equal bits with the oracle's
    fp32 slot-order chain;
  - the hierarchical pass (rank layout, send, fan-out, per-rank partials,
    their sum): rows, partials and the final sum bit for bit with the
    oracle's two-level chains;
  - the backward pair on the draw's layout: row gradients within one bf16
    ulp, weight gradients within the dot-product bound, dx bit for bit
    (computed by the oracle from the GPU's row gradients).
"""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

import combine_moe_layout_06_amd as M  # noqa: E402
from combine_moe_layout_06_amd import LayerBuffers, RankBuffers  # noqa: E402
from gpu_helpers import (assert_bf16_within_ulp, assert_combine_exact,  # noqa: E402
                         assert_route_close, dev, dot_tolerance, host, poison_like)
from oracle import moe_oracle as O  # noqa: E402
from synth import workloads as W  # noqa: E402

N_CASES = 200
GRAIN = {M.MOE_DTYPE_BF16: 8, M.MOE_DTYPE_FP8_E4M3: 128, M.MOE_DTYPE_MXFP8_E4M3: 32}


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


def draw(seed):
    g = W.rng(90000 + seed)
    R = int(g.choice([1, 2, 3, 4, 5, 8, 16, 32]))
    epr = int(g.choice([1, 2, 3, 4, 8]))
    E = R * epr
    k = int(g.integers(1, min(E, 32) + 1))
    t_max = max(1, 8192 // k)
    T = int(g.choice([0, 1, 2, 63, 64, 65, 127, 128, 129, int(g.integers(1, t_max + 1))]))
    T = min(T, t_max)
    cap = 0 if g.random() < 0.5 else int(g.integers(1, max(2, 2 * T * k // E + 2)))
    dtype = int(g.choice([M.MOE_DTYPE_BF16, M.MOE_DTYPE_FP8_E4M3, M.MOE_DTYPE_MXFP8_E4M3]))
    gr = GRAIN[dtype]
    H = gr * int(g.integers(1, 2048 // gr + 1))
    distinct = bool(g.random() < 0.7)
    mask = float(g.choice([0.0, 0.0, 0.1, 0.5]))
    return dict(T=T, E=E, k=k, R=R, cap=cap, dtype=dtype, H=H, distinct=distinct, mask=mask)


def _oracle_rows(dtype, x, dst, rows):
    if dtype == M.MOE_DTYPE_BF16:
        o, wr = O.dispatch_bf16(x, dst, rows)
        return [o], wr
    f = O.dispatch_fp8 if dtype == M.MOE_DTYPE_FP8_E4M3 else O.dispatch_mxfp8
    q, s, wr = f(x, dst, rows)
    return [q, s], wr


def _check_rows(got_list, want_list, written, rows):
    for gr, wr in zip(got_list, want_list):
        gr = gr.view(wr.dtype) if gr.dtype != wr.dtype else gr
        a, o = gr[:rows][written], wr[written]
        if a.dtype == np.float32:
            a, o = a.view(np.uint32), o.view(np.uint32)
        assert np.array_equal(a, o)
        raw = gr.view(np.uint8).reshape(gr.shape[0], -1)
        assert (raw[:rows][~written] == 0xFF).all()


@pytest.mark.parametrize("seed", range(N_CASES))
def test_route_layout_dispatch_combine(seed):
    c = draw(seed)
    T, E, k, R, cap, dtype, H = c["T"], c["E"], c["k"], c["R"], c["cap"], c["dtype"], c["H"]
    say("random case", seed, c)
    g = W.rng(seed)

    # routing, on draws where it is defined (k distinct experts per token)
    if T > 0:
        groups = [G for G in (1, 2, 4, 8) if E % G == 0 and E // G >= 2]
        G = int(g.choice(groups)) if groups else 1
        kg = int(g.integers(1, G + 1))
        if k <= kg * (E // G):
            sig = G > 1
            logits = g.standard_normal((T, E), dtype=np.float32)
            bias = (0.1 * g.standard_normal(E)).astype(np.float32) if g.random() < 0.5 else None
            fn = M.MOE_SCORE_SIGMOID if sig else M.MOE_SCORE_SOFTMAX
            b0 = LayerBuffers.allocate(T, 8, E, k, R, 0)
            b0.route(dev(logits), dev(bias) if bias is not None else None, fn,
                     G if sig else 1, kg if sig else 1)
            idx_o, w_o = O.route(logits, k, fn, G if sig else 1, kg if sig else 1, bias)
            score = O._sigmoid_f32(logits) if sig else logits
            key = O._selection_key(score, bias)
            assert_route_close(host(b0.topk_idx), host(b0.topk_weights), idx_o, w_o, key,
                               "case %d" % seed)

    # layout + dispatch (one launch or two)
    idx = W.random_topk_idx(g, T, E, k, distinct=c["distinct"], mask_frac=c["mask"])
    x = W.random_bf16_rows(g, T, H)
    b = LayerBuffers.allocate(T, H, E, k, R, cap, dtype=dtype)
    rows = b.num_rows
    b.src_pair = poison_like(max(rows, 1), torch.int32)
    b.dst_row = poison_like((max(T, 1), k), torch.int32)
    b.dispatched = poison_like((max(rows, 1), H), b.dispatched.dtype)
    if dtype != M.MOE_DTYPE_BF16:
        b.scales = poison_like((max(rows, 1),) + tuple(b.scales.shape[1:]), b.scales.dtype)
    if T:
        b.topk_idx.copy_(dev(idx))
    b.layout_dispatch(dev(x) if T else None)
    L = O.layout(idx, E, R, cap)
    for name in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets",
                 "rank_token_counts", "overflow"):
        got = host(getattr(b, name))
        assert np.array_equal(got.reshape(L[name].shape), L[name]), name
    assert np.array_equal(host(b.dst_row)[:T], L["dst_row"])
    assert np.array_equal(host(b.src_pair)[:rows], L["src_pair"])
    want, written = _oracle_rows(dtype, x, L["dst_row"], rows)
    got = [host(b.dispatched)] + ([host(b.scales)] if dtype != M.MOE_DTYPE_BF16 else [])
    _check_rows(got, want, written, rows)

    # combine of random expert rows with random weights
    y = W.random_bf16_rows(g, max(rows, 1), H)
    w = W.random_weights(g, T, k)
    if T:
        b.topk_weights.copy_(dev(w))
    b.combine(dev(y))
    if T:
        ref, _ = O.combine(y, L["dst_row"], w)
        assert_combine_exact(host(b.combined, np.uint16)[:T], ref, "case %d" % seed)
    say("  ok: fused" if M.moe_layout_dispatch_is_fused(T, k, cap) else "  ok: two launches",
        "dropped", int(L["overflow"][0]))


@pytest.mark.parametrize("seed", range(0, N_CASES, 2))
def test_hierarchical_pass(seed):
    c = draw(seed)
    T, E, k, R, cap, dtype, H = c["T"], c["E"], c["k"], c["R"], c["cap"], c["dtype"], c["H"]
    say("random hierarchical case", seed, c)
    g = W.rng(50000 + seed)
    idx = W.random_topk_idx(g, T, E, k, distinct=c["distinct"], mask_frac=c["mask"])
    x = W.random_bf16_rows(g, T, H)
    w = W.random_weights(g, T, k)
    lb = LayerBuffers.allocate(T, H, E, k, R, cap, dtype=dtype)
    rb = RankBuffers.allocate(T, H, E, k, R, dtype=dtype)
    if T:
        lb.topk_idx.copy_(dev(idx))
        lb.topk_weights.copy_(dev(w))
    lb.layout()
    rb.rank_layout(lb.topk_idx)
    rb.dispatch(dev(x) if T else None)
    lb.dispatched.view(torch.uint8).fill_(0xFF)
    if dtype != M.MOE_DTYPE_BF16:
        lb.scales.view(torch.uint8).fill_(0xFF)
    rb.expand(lb)

    L = O.layout(idx, E, R, cap)
    RL = O.rank_layout(idx, E, R)
    for name in ("rank_token_counts", "rank_token_offsets", "rank_row", "send_row"):
        got = host(getattr(rb, name))
        assert np.array_equal(got.reshape(RL[name].shape), RL[name]), name
    nrr = RL["num_rank_rows"]
    assert np.array_equal(host(rb.row_token)[:nrr], RL["row_token"][:nrr])
    # the fanned-out rows equal a flat dispatch of the same tokens
    rows = lb.num_rows
    want, written = _oracle_rows(dtype, x, L["dst_row"], rows)
    got = [host(lb.dispatched)] + ([host(lb.scales)] if dtype != M.MOE_DTYPE_BF16 else [])
    _check_rows(got, want, written, rows)

    # per-rank partials and their sum
    y = W.random_bf16_rows(g, max(rows, 1), H)
    rb.combine_local(lb, dev(y))
    out = torch.zeros((max(T, 1), H), dtype=torch.int16, device="cuda")
    rb.combine_partials(out)
    if T == 0:
        return
    part_o, pw, _ = O.combine_local(y, L["dst_row"], RL["rank_row"], w, rb.num_rank_rows)
    part_g = host(rb.partial, np.uint16)
    live = np.nonzero(pw)[0]
    assert_combine_exact(part_g[live], part_o[live], "partials %d" % seed)
    # final sum: the oracle's sum of the GPU's own partials (one rounding),
    # against the GPU's fp32 sum of them
    ref, _ = O.combine_partials(part_g, RL["send_row"])
    assert_combine_exact(host(out, np.uint16)[:T], ref, "sum %d" % seed)
    say("  ok: rows sent", int(RL["rank_token_offsets"][-1]))


@pytest.mark.parametrize("seed", range(1, N_CASES, 2))
def test_backward_pair(seed):
    c = draw(seed)
    T, E, k, R, cap, H = c["T"], c["E"], c["k"], c["R"], c["cap"], c["H"]
    say("random backward case", seed, c)
    g = W.rng(70000 + seed)
    idx = W.random_topk_idx(g, T, E, k, distinct=c["distinct"], mask_frac=c["mask"])
    L = O.layout(idx, E, R, cap)
    rows, dst = L["num_rows"], L["dst_row"]
    dout = W.random_bf16_rows(g, T, H)
    y = W.random_bf16_rows(g, max(rows, 1), H)
    w = W.random_weights(g, T, k)
    dy_full = poison_like((max(rows, 1), H), torch.int16)
    dw_full = poison_like((max(T, 1), k), torch.float32)
    dx_full = poison_like((max(T, 1), H), torch.int16)
    live_in = (lambda a: dev(a)) if T else (lambda a: None)
    M.moe_combine_backward(T, H, k, rows, live_in(dout), dev(y), live_in(dst), live_in(w),
                           dy_full, dw_full)
    M.moe_dispatch_backward(T, H, k, rows, dy_full, live_in(dst), dx_full)
    if T == 0:
        return
    dy = host(dy_full, np.uint16)
    dw = host(dw_full)[:T]
    want_dy, written, want_dw, dw_abs = O.combine_backward(dout, y, dst, w, rows)
    assert np.all(dy[:rows][~written] == 0xFFFF)          # rows of no pair stay untouched
    assert_bf16_within_ulp(dy[:rows][written], want_dy[written], "case %d dy" % seed)
    live = dst >= 0
    assert np.all(dw[~live] == 0.0)
    err = np.abs(dw.astype(np.float64) - want_dw.astype(np.float64))
    assert np.all(err <= dot_tolerance(H, want_dw.astype(np.float64), dw_abs))
    want_dx, _ = O.dispatch_backward(dy[:max(rows, 1)], dst)
    assert_combine_exact(host(dx_full, np.uint16)[:T], want_dx, "case %d dx" % seed)
