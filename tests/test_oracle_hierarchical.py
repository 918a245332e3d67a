"""Pins of the oracle's deduplicated dispatch and hierarchical combine:
a hand-worked example (where the two-level rounding differs from the flat
combine), plain-loop references for the (token, rank) rows and the partial
sums, the identity "deduplicated dispatch + fan-out = flat dispatch" in
every format, and the special cases R = 1 (one partial: the flat combine)
and one expert per rank (every partial is a single product)."""

import json
import math
import os

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import workloads as W
from exact_f32 import chain_f32  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(vals):
    """bf16 bits of values that are exact in bf16 (asserted)."""
    f = np.asarray(vals, dtype=np.float32)
    b = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(O.bf16_to_f32(b), f)
    return b


def _load():
    with open(os.path.join(GOLDEN, "hierarchical_worked_example.json")) as f:
        return json.load(f)


def test_worked_example_rank_rows():
    ex = _load()
    idx = np.array(ex["topk_idx"], dtype=np.int32)
    e, r = ex["num_experts"], ex["num_ranks"]
    assert [c // (e // r) for c in range(e)] == ex["expert_to_rank"]
    got = O.rank_layout(idx, e, r)
    for name, want in ex["rank_layout"].items():
        g = got[name]
        assert (g.tolist() if hasattr(g, "tolist") else g) == want, name
    # the expert layout of the same routing gives the same distinct counts
    assert O.layout(idx, e, r)["rank_token_counts"].tolist() == \
        ex["rank_layout"]["rank_token_counts"]


@pytest.mark.parametrize("mode,cap", [("packed", 0), ("capacity_1", 1)])
def test_worked_example_hierarchical_combine(mode, cap):
    ex = _load()
    idx = np.array(ex["topk_idx"], dtype=np.int32)
    e, r = ex["num_experts"], ex["num_ranks"]
    case = ex[mode]
    lay = O.layout(idx, e, r, cap)
    assert lay["dst_row"].tolist() == case["dst_row"]
    rl = O.rank_layout(idx, e, r)
    w = np.array(ex["topk_weights"], dtype=np.float32)
    y = _bits(case["expert_rows"])
    dst = np.array(case["dst_row"], dtype=np.int32)
    partial, written, _ = O.combine_local(y, dst, rl["rank_row"], w, rl["num_rank_rows"])
    assert np.nonzero(written)[0].tolist() == case["partial_rows_written"]
    assert np.array_equal(partial[written], _bits(case["partial"]))
    out, _ = O.combine_partials(partial, rl["send_row"])
    assert np.array_equal(out, _bits(case["out"]))
    out2, _, _ = O.combine_hierarchical(y, dst, w, rl)
    assert np.array_equal(out2, out)
    if "flat_combine_out" in case:
        flat, _ = O.combine(y, dst, w)
        assert np.array_equal(flat, _bits(case["flat_combine_out"]))
        assert not np.array_equal(flat, out)     # the rounding order matters


def _loop_rank_layout(idx, e, r):
    """Plain loops: first pass counts the distinct ranks of every token,
    second pass walks the tokens in order with one running counter per
    rank and hands out rows at each token's first slot on a rank."""
    t, k = idx.shape
    epr = e // r
    counts = [0] * r
    for row in idx:
        seen = set()
        for v in row:
            if 0 <= v < e and v // epr not in seen:
                seen.add(v // epr)
                counts[v // epr] += 1
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    nxt = offsets[:-1].copy()
    rank_row = [[-1] * k for _ in range(t)]
    send_row = [[-1] * k for _ in range(t)]
    row_token = [-1] * (t * min(k, r))
    for i in range(t):
        mine = {}
        for j in range(k):
            v = int(idx[i, j])
            if not 0 <= v < e:
                continue
            rk = v // epr
            if rk not in mine:
                mine[rk] = nxt[rk]
                nxt[rk] += 1
                send_row[i][j] = mine[rk]
                row_token[mine[rk]] = i
            rank_row[i][j] = mine[rk]
    return counts, offsets, rank_row, send_row, row_token


@pytest.mark.parametrize("seed,t,e,r,k,distinct,mask", [
    (1, 40, 16, 4, 4, True, 0.0),
    (2, 33, 12, 3, 5, True, 0.2),
    (3, 50, 8, 8, 3, False, 0.1),      # repeated experts in one token
    (4, 29, 10, 1, 4, True, 0.0),      # one rank: one row per token
    (5, 17, 32, 32, 8, True, 0.3),     # one expert per rank
    (6, 64, 24, 6, 8, False, 0.0),     # k > R
])
def test_rank_layout_matches_plain_loops(seed, t, e, r, k, distinct, mask):
    g = W.rng(seed)
    idx = W.random_topk_idx(g, t, e, k, distinct=distinct, mask_frac=mask)
    if seed == 3:
        idx[0, :] = e + 3                  # ids past E count as masked
    got = O.rank_layout(idx, e, r)
    counts, offsets, rank_row, send_row, row_token = _loop_rank_layout(idx, e, r)
    assert got["rank_token_counts"].tolist() == counts
    assert got["rank_token_offsets"].tolist() == offsets
    assert got["rank_row"].tolist() == rank_row
    assert got["send_row"].tolist() == send_row
    assert got["row_token"].tolist() == row_token
    assert got["num_rank_rows"] == t * min(k, r)


@pytest.mark.parametrize("name", ["tiny", "qwen3_skew", "dsv3", "decode"])
def test_rank_layout_invariants_on_workloads(name):
    w = W.WORKLOADS[name]
    inp = W.make_inputs(w, 0, tokens=min(w.tokens, 512))
    idx, _ = O.route(inp.logits, w.top_k, w.score_fn, w.groups, w.topk_groups, inp.bias)
    rl = O.rank_layout(idx, w.experts, w.ranks)
    lay = O.layout(idx, w.experts, w.ranks, w.capacity)
    assert np.array_equal(rl["rank_token_counts"], lay["rank_token_counts"])
    n = int(rl["rank_token_offsets"][-1])
    send = rl["send_row"]
    assert (send >= 0).sum() == n                             # one send per row
    assert sorted(send[send >= 0].tolist()) == list(range(n))
    assert (rl["row_token"][n:] == -1).all()
    epr = w.experts // w.ranks
    off = rl["rank_token_offsets"]
    for t, j in zip(*np.nonzero(rl["rank_row"] >= 0)):
        s = rl["rank_row"][t, j]
        assert rl["row_token"][s] == t
        rk = idx[t, j] // epr
        assert off[rk] <= s < off[rk + 1]
    # rows of one rank in token order
    tok = rl["row_token"][:n]
    for rk in range(w.ranks):
        seg = tok[off[rk]:off[rk + 1]]
        assert (np.diff(seg) > 0).all()


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp8"])
@pytest.mark.parametrize("cap", [0, 6])
def test_dedup_dispatch_then_fanout_equals_flat_dispatch(fmt, cap):
    g = W.rng(11)
    t, e, r, k, h = 48, 16, 4, 4, 256
    idx = W.random_topk_idx(g, t, e, k, mask_frac=0.1)
    x = W.random_bf16_rows(g, t, h)
    lay = O.layout(idx, e, r, cap)
    rl = O.rank_layout(idx, e, r)
    nr = rl["num_rank_rows"]
    if fmt == "bf16":
        flat, fw = O.dispatch_bf16(x, lay["dst_row"], lay["num_rows"])
        sent, sw = O.dispatch_bf16(x, rl["send_row"], nr)
        parts_flat, parts_sent = [flat], [sent]
    else:
        f = O.dispatch_fp8 if fmt == "fp8" else O.dispatch_mxfp8
        fc, fs, fw = f(x, lay["dst_row"], lay["num_rows"])
        sc, ss, sw = f(x, rl["send_row"], nr)
        parts_flat, parts_sent = [fc, fs], [sc, ss]
    n = int(rl["rank_token_offsets"][-1])
    assert sw.sum() == n and sw[:n].all()          # exactly the (token, rank) rows
    assert n < (idx >= 0).sum() or r == e          # fewer rows than pairs here
    for pf, ps in zip(parts_flat, parts_sent):
        got, written = O.expand_rows(ps, rl["rank_row"], lay["src_pair"])
        assert np.array_equal(written, fw)
        assert np.array_equal(got[written], pf[fw])


def _loop_partials(y, dst, rank_row, w, nr):
    """Each (token, rank) row's terms in slot order through the Fraction fp32
    chain of tests/exact_f32.py, one bf16 rounding at the end; math.fsum of
    the terms' magnitudes."""
    t, k = dst.shape
    h = y.shape[1]
    yf = O.bf16_to_f32(y)
    terms = {}
    for i in range(t):
        for j in range(k):
            s = int(rank_row[i, j])
            if s < 0:
                continue
            terms.setdefault(s, [])
            if dst[i, j] >= 0:
                terms[s].append((w[i, j], yf[dst[i, j]]))
    out, mag = {}, {}
    for s, pairs in terms.items():
        ws = [p[0] for p in pairs]
        out[s] = O.round_to_bf16(np.array(
            [chain_f32(ws, [p[1][c] for p in pairs]) for c in range(h)], np.float32))
        mag[s] = np.array([math.fsum(abs(float(p[0]) * float(p[1][c])) for p in pairs)
                           for c in range(h)])
    return out, mag


@pytest.mark.parametrize("seed,cap", [(21, 0), (22, 3)])
def test_partials_match_loop_chains(seed, cap):
    g = W.rng(seed)
    t, e, r, k, h = 30, 12, 3, 4, 24
    idx = W.random_topk_idx(g, t, e, k, mask_frac=0.15)
    lay = O.layout(idx, e, r, cap)
    rl = O.rank_layout(idx, e, r)
    y = W.random_bf16_rows(g, lay["num_rows"], h)
    w = W.random_weights(g, t, k)
    partial, written, mag = O.combine_local(y, lay["dst_row"], rl["rank_row"], w,
                                            rl["num_rank_rows"])
    want, want_mag = _loop_partials(y, lay["dst_row"], rl["rank_row"], w, rl["num_rank_rows"])
    assert sorted(want) == np.nonzero(written)[0].tolist()
    for s, row in want.items():
        assert np.array_equal(partial[s], row), s
        np.testing.assert_allclose(mag[s], want_mag[s], rtol=1e-12, atol=0)
    # final level: the unit-weight chain of the partials in slot order, one
    # rounding
    out, _ = O.combine_partials(partial, rl["send_row"])
    pf = O.bf16_to_f32(partial)
    for i in range(t):
        rows = [int(s) for s in rl["send_row"][i] if s >= 0]
        want_t = O.round_to_bf16(np.array(
            [chain_f32([1.0] * len(rows), [pf[s, c] for s in rows]) for c in range(h)],
            np.float32))
        assert np.array_equal(out[i], want_t), i


def test_one_rank_is_the_flat_combine():
    """R = 1: every token has one partial, the full weighted sum rounded
    once, and adding it to nothing rounds to itself."""
    g = W.rng(31)
    t, e, k, h = 40, 8, 3, 64
    idx = W.random_topk_idx(g, t, e, k, mask_frac=0.1)
    for cap in (0, 4):
        lay = O.layout(idx, e, 1, cap)
        rl = O.rank_layout(idx, e, 1)
        y = W.random_bf16_rows(g, lay["num_rows"], h)
        w = W.random_weights(g, t, k)
        out, _, _ = O.combine_hierarchical(y, lay["dst_row"], w, rl)
        flat, _ = O.combine(y, lay["dst_row"], w)
        live = (idx >= 0).any(axis=1)
        assert np.array_equal(out[live], flat[live])
        # a token with every slot masked has no row and sums nothing
        assert (O.bf16_to_f32(out[~live]) == 0).all()


def test_one_expert_per_rank_partials_are_products():
    g = W.rng(32)
    t, e, k, h = 25, 16, 4, 32
    idx = W.random_topk_idx(g, t, e, k)
    lay = O.layout(idx, e, e)
    rl = O.rank_layout(idx, e, e)
    assert np.array_equal(rl["send_row"], rl["rank_row"])     # no two slots share
    y = W.random_bf16_rows(g, lay["num_rows"], h)
    w = W.random_weights(g, t, k)
    partial, _, _ = O.combine_local(y, lay["dst_row"], rl["rank_row"], w, rl["num_rank_rows"])
    yf = O.bf16_to_f32(y).astype(np.float64)
    for i in range(t):
        for j in range(k):
            want = O.round_to_bf16(float(w[i, j]) * yf[lay["dst_row"][i, j]])
            assert np.array_equal(partial[rl["rank_row"][i, j]], want)


def test_hierarchical_within_two_level_bound_of_flat():
    """|two-level - flat| <= ulp(flat) + sum over partials of half an ulp:
    each partial moves by at most half a bf16 ulp, the final rounding by at
    most one ulp of the result."""
    g = W.rng(33)
    t, e, r, k, h = 64, 32, 8, 8, 64
    idx = W.random_topk_idx(g, t, e, k)
    lay = O.layout(idx, e, r)
    rl = O.rank_layout(idx, e, r)
    y = W.random_bf16_rows(g, lay["num_rows"], h)
    w = W.random_weights(g, t, k)
    out, partial, _ = O.combine_hierarchical(y, lay["dst_row"], w, rl)
    flat, _ = O.combine(y, lay["dst_row"], w)
    a, b = O.bf16_to_f32(out).astype(np.float64), O.bf16_to_f32(flat).astype(np.float64)

    def ulp(v):
        m, ex = np.frexp(np.abs(v))
        return np.ldexp(1.0, ex - 8)

    pf = O.bf16_to_f32(partial).astype(np.float64)
    half = np.zeros((t, h))
    for i in range(t):
        for s in rl["send_row"][i]:
            if s >= 0:
                half[i] += 0.5 * ulp(pf[s])
    bound = np.maximum(ulp(a), ulp(b)) + half
    assert (np.abs(a - b) <= bound).all()
    assert (a != b).any()        # random inputs do hit the double rounding
